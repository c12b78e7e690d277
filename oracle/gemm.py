"""Block-scaled FP8 product, dense and grouped (oracle; test infrastructure only).

Admin Guide ("DeepSeek-V3 Administrator & Developer Guide", doccompiler)
8.5.3 ``fp8_gemm_kernel``: a tiled product of e4m3 operands with an fp32
accumulator, where each K-block's partial dot product is multiplied by the
activation scale of its row and K-block and by the weight scale of its
128x128 block before being added.  Section 6.3 fixes the orientation: the
weight is ``[out, in]``, its scale grid is ``(ceil(out/128), ceil(in/128))``
and the layer computes ``y = x W^T``.

Because ``(sum_k a_k b_k) * sa * sb == sum_k (a_k sa) (b_k sb)`` exactly in the
reals, the reference value is the plain product of the dequantised operands,
formed in fp64 (``gemm``).  Dequantisation to fp64 is exact (a 4-bit e4m3
significand times a 24-bit fp32 scale).  ``gemm_blockwise`` follows the pages'
per-K-block order literally and is used as a brute-force cross-check on small
shapes.

The grouped form (``grouped_gemm``) is the batched reading of the per-expert
loop of Admin Guide 6.4 / 8.4: rows sorted by expert, expert ``e`` owning rows
``offsets[e]:offsets[e+1]`` and its own weight and scale grid.
"""

import numpy as np

from .formats import e4m3_decode
from .quant import BLOCK, expand_block_scales, n_blocks


def dequant_act(y, s):
    """fp64 ``dec(y[m, k]) * s[m, k // 128]``."""
    y = np.asarray(y, dtype=np.uint8)
    M, K = y.shape
    cols = np.arange(K) // BLOCK
    return e4m3_decode(y) * np.asarray(s, np.float64)[:, cols]


def dequant_weight(w, S):
    """fp64 ``dec(w[n, k]) * S[n // 128, k // 128]``."""
    w = np.asarray(w, dtype=np.uint8)
    N, K = w.shape
    return e4m3_decode(w) * expand_block_scales(S, N, K).astype(np.float64)


def gemm(a, a_s, b, b_s):
    """``C = A_hat @ B_hat^T`` in fp64 for e4m3 ``a [M,K]``, ``b [N,K]``."""
    return dequant_act(a, a_s) @ dequant_weight(b, b_s).T


def gemm_rows(a, a_s, b, b_s, rows, cols):
    """Selected outputs ``C[rows[i], cols[j]]`` (fp64) without forming all of C."""
    A = dequant_act(np.asarray(a)[rows], np.asarray(a_s)[rows])
    Bsel = np.asarray(b)[cols]
    Ssel = np.asarray(b_s)[np.asarray(cols) // BLOCK]
    K = Bsel.shape[1]
    kcols = np.arange(K) // BLOCK
    Bh = e4m3_decode(Bsel) * Ssel[:, kcols].astype(np.float64)
    return A @ Bh.T


def gemm_blockwise(a, a_s, b, b_s):
    """Brute force in the pages' order: per output, per K-block, dot then rescale.

    The dot product of one 128-wide block is exact in fp64 (products of two
    e4m3 values have at most 8 significant bits and span 2^-18..2^17, so a
    sum of 128 of them needs fewer than 53 bits); the rescale and the running
    sum are fp64.
    """
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    A = e4m3_decode(a)
    B = e4m3_decode(b)
    out = np.zeros((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for kb in range(n_blocks(K)):
                lo, hi = kb * BLOCK, min(K, (kb + 1) * BLOCK)
                dot = 0.0
                for k in range(lo, hi):
                    dot += A[m, k] * B[n, k]
                acc += dot * float(a_s[m, kb]) * float(b_s[n // BLOCK, kb])
            out[m, n] = acc
    return out


def grouped_gemm(a, a_s, b, b_s, offsets):
    """Per-expert loop: ``C[o_e:o_{e+1}] = gemm(A[o_e:o_{e+1}], W_e)`` in fp64.

    ``b`` is ``[E, N, K]`` e4m3, ``b_s`` is ``[E, ceil(N/128), ceil(K/128)]``,
    ``offsets`` is ``[E+1]`` non-decreasing with ``offsets[0] == 0``.
    Rows of an expert with no rows are simply absent.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    M = int(offsets[-1])
    N = np.asarray(b).shape[1]
    out = np.zeros((M, N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = gemm(a[lo:hi], a_s[lo:hi], b[e], b_s[e])
    return out


def expert_of_rows(offsets, rows):
    """Expert index owning each row (rows sorted by expert)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    return np.searchsorted(offsets, np.asarray(rows), side="right") - 1

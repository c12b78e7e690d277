"""Block quantisation and dequantisation (oracle; test infrastructure only).

* ``act_quant``      -- Admin Guide ("DeepSeek-V3 Administrator & Developer
  Guide", doccompiler) 8.5.1 ``act_quant_kernel``; the per-block scale is
  stored as fp32 (CodeVetter "Data flow", FP8 bullet); the optional ue8m0
  rounding is the User Guide FAQ "What is scale_fmt: ue8m0?".
* ``weight_quant``   -- produces the stored weight format of the DocSearch
  index of the DeepSeek-V3 README, item 3 ("Dequantize FP8 weights using
  weight_scale_inv"): e4m3 codes plus one fp32 multiplier per 128x128 block,
  blocks that are not 128-aligned being zero-padded for the scale.
* ``weight_dequant`` -- Admin Guide 8.5.2 ``weight_dequant_kernel``.

All arithmetic is IEEE binary32 (NumPy float32, correctly rounded), because
the pages convert the data to fp32 before taking the maximum, dividing and
multiplying.

Readings where the pages leave a step open:

* the clamp is applied to the block's absolute maximum before the division by
  448 (the pages' order: absolute max, clamp to 1e-4, divide by 448), and the
  clamp constant is 1e-4 rounded to fp32;
* ``s = amax / 448`` and ``y = x / s`` are correctly rounded fp32 divisions;
* ue8m0 rounds ``s`` up to the smallest power of two not below it, computed
  exactly from the fp32 bits, and the result stays an fp32 value;
* a last block narrower than 128 uses its real elements only, which is what
  zero padding gives (a zero never raises the absolute maximum), and its codes
  are only emitted for the real elements;
* the weight quantiser mirrors the activation quantiser (clamp, /448,
  optional ue8m0) over 128x128 blocks.
"""

import numpy as np

from .formats import bf16_to_f32, e4m3_decode, e4m3_encode, f32_to_bf16

BLOCK = 128
CLAMP = np.float32(1e-4)
E4M3_MAX_F32 = np.float32(448.0)


def n_blocks(n):
    return (int(n) + BLOCK - 1) // BLOCK


def pow2_ceil(s):
    """Smallest power of two >= s for positive normal fp32 s (exact)."""
    s = np.asarray(s, dtype=np.float32)
    m, e = np.frexp(s.astype(np.float64))       # s = m * 2^e, m in [0.5, 1)
    p = np.where(m == 0.5, s.astype(np.float64), np.ldexp(1.0, e))
    return p.astype(np.float32)


def block_scale(amax, ue8m0=False):
    """fp32 scale of one block from its fp32 absolute maximum."""
    a = np.maximum(np.asarray(amax, dtype=np.float32), CLAMP)
    s = a / E4M3_MAX_F32
    if ue8m0:
        s = pow2_ceil(s)
    return s.astype(np.float32)


def act_quant(x_bits, ue8m0=False):
    """Quantise bf16 activations ``[M, K]`` (uint16 bits) per row and per 128 columns.

    Returns ``(y, s)``: e4m3 codes ``uint8 [M, K]`` and fp32 scales
    ``[M, ceil(K/128)]`` with ``x ~= dec(y) * s``.
    """
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("act_quant expects a 2-D input")
    M, K = x.shape
    nb = n_blocks(K)
    y = np.zeros((M, K), dtype=np.uint8)
    s = np.zeros((M, nb), dtype=np.float32)
    for b in range(nb):
        lo, hi = b * BLOCK, min(K, (b + 1) * BLOCK)
        blk = x[:, lo:hi]
        amax = np.max(np.abs(blk), axis=1) if M else np.zeros(0, np.float32)
        sb = block_scale(amax, ue8m0)
        q = (blk / sb[:, None]).astype(np.float32)
        y[:, lo:hi] = e4m3_encode(q)
        s[:, b] = sb
    return y, s


def weight_quant(w, ue8m0=False):
    """Quantise real-valued weights ``[N, K]`` (fp32, or bf16 widened to fp32).

    Returns ``(codes uint8 [N, K], S fp32 [ceil(N/128), ceil(K/128)])`` with
    ``W ~= dec(codes) * S[n//128, k//128]``.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("weight_quant expects a 2-D input")
    N, K = w.shape
    nbn, nbk = n_blocks(N), n_blocks(K)
    codes = np.zeros((N, K), dtype=np.uint8)
    S = np.zeros((nbn, nbk), dtype=np.float32)
    for i in range(nbn):
        r0, r1 = i * BLOCK, min(N, (i + 1) * BLOCK)
        for j in range(nbk):
            c0, c1 = j * BLOCK, min(K, (j + 1) * BLOCK)
            blk = w[r0:r1, c0:c1]
            sb = block_scale(np.max(np.abs(blk)), ue8m0)
            codes[r0:r1, c0:c1] = e4m3_encode((blk / sb).astype(np.float32))
            S[i, j] = sb
    return codes, S


def expand_block_scales(S, N, K):
    """Per-element view of a ``[ceil(N/128), ceil(K/128)]`` scale grid."""
    S = np.asarray(S, dtype=np.float32)
    rows = np.arange(N) // BLOCK
    cols = np.arange(K) // BLOCK
    return S[rows[:, None], cols[None, :]]


def weight_dequant(codes, S):
    """``bf16( fl32( dec(W) * S ) )`` as uint16 bits -- two roundings, as on the pages."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    v = e4m3_decode(codes).astype(np.float32)          # exact
    prod = (v * expand_block_scales(S, N, K)).astype(np.float32)
    return f32_to_bf16(prod)

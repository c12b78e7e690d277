"""Routed-expert steps around the grouped product (oracle; test infrastructure only).

"DeepSeek-V3 Administrator & Developer Guide" (doccompiler), sections 6.4
("MoE expert routing") and 8.4 ("The MoE forward pass -- annotated"): the gate
gives each of the N tokens ``n_activated_experts`` (expert index, weight)
pairs; ``y`` starts as zeros in x's dtype; for each expert i in increasing
order, the pairs (idx, top) with ``indices == i`` are found, the tokens
``x[idx]`` go through expert i, and ``y[idx] += expert(x[idx]) *
weights[idx, top]``.  The expert is the feed-forward ``w2(SiLU(w1 x) * w3 x)``
(section 1.2, Expert row), each linear block-scaled FP8 (``gemm`` here).

The batched form keeps that order:

* ``route``   -- the rows of the grouped product are the (token, slot) pairs
  of expert 0, then expert 1, ...; within an expert in row-major (token, slot)
  order, which is the order in which ``torch.where`` returns them.
* ``gather_act_quant`` -- act_quant of the routed rows ``x[idx]``.
* ``combine`` -- the weighted accumulation into y.

Readings taken where the pages are silent:

* The routing weights are bf16 (the pages run with bf16 as the default
  dtype, section 1.3).  Each contribution ``expert_out * w`` is the product of
  two bf16 tensors, rounded once to bf16; each ``y += p`` is a bf16 addition,
  rounded once; the additions for a token happen in increasing expert order
  (the loop order).  Both operations are formed in fp64 here and rounded to
  bf16, nearest-even, which equals rounding the exact result once: a product
  of two 8-bit significands is exact in fp64; a sum of two bf16 values is
  exact in fp64 unless their exponents are more than 45 apart, and even then
  the fp64 rounding cannot change the bf16 result, because 53 bits are at
  least 2 * 8 + 2 (double rounding to nearest is innocuous at that precision;
  S. A. Figueroa, "When is double rounding innocuous?", 1995).
* A token lists each expert at most once (top-k of distinct experts).
"""

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16
from . import gemm as G
from . import glue
from . import quant as Q


def route(indices, experts):
    """Grouped-product row order of the (token, slot) pairs.

    indices: int [T, k] expert of each (token, slot).
    Returns ``(offsets int64 [E+1], row_token int64 [R], row_slot int64 [R],
    token_rows int64 [T, k])`` with R = T*k: rows offsets[e]:offsets[e+1] are
    expert e's pairs in row-major order; row r is pair (row_token[r],
    row_slot[r]); token_rows[t, j] is the row of pair (t, j).
    """
    ind = np.asarray(indices)
    T, k = ind.shape
    offsets = [0]
    toks, slots = [], []
    for e in range(experts):
        t, j = np.nonzero(ind == e)          # row-major order, as torch.where
        toks.append(t)
        slots.append(j)
        offsets.append(offsets[-1] + len(t))
    row_token = np.concatenate(toks).astype(np.int64) if toks else np.zeros(0, np.int64)
    row_slot = np.concatenate(slots).astype(np.int64) if slots else np.zeros(0, np.int64)
    token_rows = np.full((T, k), -1, np.int64)
    token_rows[row_token, row_slot] = np.arange(len(row_token))
    return np.asarray(offsets, np.int64), row_token, row_slot, token_rows


def gather_act_quant(x_bits, row_token, ue8m0=False):
    """act_quant of the routed rows ``x[row_token]`` (the expert inputs x[idx])."""
    return Q.act_quant(np.asarray(x_bits)[np.asarray(row_token)], ue8m0=ue8m0)


def combine(yr_bits, weights_bits, indices, token_rows):
    """y [T, D] bf16 bits: for each token, over its experts in increasing index,
    y = bf16(y + bf16(yr[row] * w)), starting from y = 0.

    yr_bits: bf16 [R, D] expert outputs by row; weights_bits: bf16 [T, k];
    indices, token_rows: [T, k] as from ``route``.
    """
    yr = bf16_to_f32(yr_bits).astype(np.float64)
    w = bf16_to_f32(weights_bits).astype(np.float64)
    ind = np.asarray(indices)
    rows = np.asarray(token_rows)
    T, k = ind.shape
    y = np.zeros((T, yr.shape[1]), np.float64)
    order = np.argsort(ind, axis=1, kind="stable")      # experts in increasing index
    t = np.arange(T)
    for jj in range(k):
        j = order[:, jj]
        p = bf16_to_f32(f32_to_bf16(yr[rows[t, j]] * w[t, j][:, None])).astype(np.float64)
        y = bf16_to_f32(f32_to_bf16(y + p)).astype(np.float64)
    return f32_to_bf16(y)


def expert_ffn(x_bits, q13, s13, q2, s2, ue8m0=False):
    """One expert on its rows: act_quant -> [w1; w3] product -> bf16 ->
    SiLU(h1) * h3 (bf16) -> act_quant -> w2 product -> bf16.  q13 stacks w1
    (first F rows) over w3."""
    a, a_s = Q.act_quant(x_bits, ue8m0=ue8m0)
    h13 = f32_to_bf16(G.gemm(a, a_s, q13, s13))
    F = q13.shape[0] // 2
    h = glue.silu_mul(h13[:, :F], h13[:, F:])
    hq, hs = Q.act_quant(h, ue8m0=ue8m0)
    return f32_to_bf16(G.gemm(hq, hs, q2, s2))


def moe_forward(x_bits, indices, weights_bits, q13, s13, q2, s2, ue8m0=False):
    """The routed-expert output y [T, D] (bf16 bits) of the pages' loop, with
    per-expert weights q13[e], s13[e], q2[e], s2[e]."""
    E = q13.shape[0]
    offsets, row_token, _, token_rows = route(indices, E)
    yr = np.zeros((len(row_token), q2.shape[1]), np.uint16)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            yr[lo:hi] = expert_ffn(np.asarray(x_bits)[row_token[lo:hi]], q13[e], s13[e], q2[e], s2[e], ue8m0)
    return combine(yr, weights_bits, indices, token_rows)

"""Pins of the oracle's block-scaled product and its grouped form (CPU only).

The per-K-block order of Admin Guide 8.5.3 (brute force) must equal the fp64
product of dequantised operands; integer-valued operands with unit or
power-of-two scales have an exact result computed by integer arithmetic; a
one-hot weight selects a column of A; the grouped form (Admin Guide 6.4 / 8.4)
equals the per-expert loop, reduces to the dense product for one expert, and
permutes with the experts.  Dequantisation is pinned to torch's float8 decode.
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q


def rand_operands(M, N, K, seed, ue8m0=False):
    g = np.random.default_rng(seed)
    x = F.f32_to_bf16(g.standard_normal((M, K)).astype(np.float32))
    a, a_s = Q.act_quant(x, ue8m0=ue8m0)
    w = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    b, b_s = Q.weight_quant(w, ue8m0=ue8m0)
    return a, a_s, b, b_s


def test_dequant_matches_torch():
    a, a_s, b, b_s = rand_operands(7, 140, 300, 1)
    at = torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    cols = torch.arange(300) // 128
    ref = at * torch.from_numpy(a_s).double()[:, cols]
    assert np.array_equal(G.dequant_act(a, a_s), ref.numpy())
    bt = torch.from_numpy(b).view(torch.float8_e4m3fn).double()
    refb = bt * torch.from_numpy(Q.expand_block_scales(b_s, 140, 300)).double()
    assert np.array_equal(G.dequant_weight(b, b_s), refb.numpy())


def test_bruteforce_equals_fp64_product():
    for (M, N, K, seed) in [(3, 5, 128, 2), (4, 130, 300, 3), (2, 3, 7, 4), (5, 129, 257, 5)]:
        a, a_s, b, b_s = rand_operands(M, N, K, seed)
        ref = G.gemm(a, a_s, b, b_s)
        bf = G.gemm_blockwise(a, a_s, b, b_s)
        assert np.allclose(bf, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_integer_operands_exact():
    g = np.random.default_rng(6)
    M, N, K = 9, 140, 384
    vals = np.arange(-4, 5)
    ai = g.choice(vals, (M, K))
    bi = g.choice(vals, (N, K))
    a = F.e4m3_encode(ai.astype(np.float32))
    b = F.e4m3_encode(bi.astype(np.float32))
    a_s = np.ones((M, 3), np.float32)
    b_s = np.full((2, 3), 0.25, np.float32)
    C = G.gemm(a, a_s, b, b_s)
    assert np.array_equal(C, (ai @ bi.T).astype(np.float64) * 0.25)


def test_one_hot_weight_selects_column():
    a, a_s, _, _ = rand_operands(6, 4, 256, 7)
    N, K = 130, 256
    b = np.zeros((N, K), np.uint8)
    cols = np.random.default_rng(8).integers(0, K, N)
    b[np.arange(N), cols] = 0x38                       # 1.0
    b_s = np.full((2, 2), 0.5, np.float32)
    C = G.gemm(a, a_s, b, b_s)
    Ahat = G.dequant_act(a, a_s)
    assert np.array_equal(C, Ahat[:, cols] * 0.5)


def test_zero_k():
    C = G.gemm(np.zeros((3, 0), np.uint8), np.zeros((3, 0), np.float32),
               np.zeros((5, 0), np.uint8), np.zeros((1, 0), np.float32))
    assert C.shape == (3, 5) and np.all(C == 0)


def test_gemm_rows_selects():
    a, a_s, b, b_s = rand_operands(20, 300, 256, 9)
    full = G.gemm(a, a_s, b, b_s)
    rows, cols = np.array([0, 7, 19]), np.array([1, 128, 299])
    assert np.allclose(G.gemm_rows(a, a_s, b, b_s, rows, cols), full[np.ix_(rows, cols)], rtol=1e-14)


def _grouped_case(E, counts, N=140, K=300, seed=10):
    g = np.random.default_rng(seed)
    M = int(sum(counts))
    x = F.f32_to_bf16(g.standard_normal((M, K)).astype(np.float32))
    a, a_s = Q.act_quant(x)
    bs, ss = zip(*[Q.weight_quant((g.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(E)])
    b, b_s = np.stack(bs), np.stack(ss)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return a, a_s, b, b_s, offsets


def test_grouped_equals_loop_with_empty_experts():
    counts = [5, 0, 17, 1, 0, 9]
    a, a_s, b, b_s, off = _grouped_case(6, counts)
    C = G.grouped_gemm(a, a_s, b, b_s, off)
    for e in range(6):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert np.array_equal(C[lo:hi], G.gemm(a[lo:hi], a_s[lo:hi], b[e], b_s[e]))
    assert C.shape == (32, 140)


def test_grouped_single_expert_is_dense():
    a, a_s, b, b_s, off = _grouped_case(1, [23])
    assert np.array_equal(G.grouped_gemm(a, a_s, b, b_s, off), G.gemm(a, a_s, b[0], b_s[0]))


def test_grouped_expert_permutation():
    counts = [4, 7, 0, 3]
    a, a_s, b, b_s, off = _grouped_case(4, counts)
    C = G.grouped_gemm(a, a_s, b, b_s, off)
    perm = [2, 3, 0, 1]
    blocks = [np.arange(off[e], off[e + 1]) for e in range(4)]
    rows = np.concatenate([blocks[e] for e in perm])
    counts_p = [counts[e] for e in perm]
    off_p = np.zeros(5, np.int32)
    off_p[1:] = np.cumsum(counts_p)
    Cp = G.grouped_gemm(a[rows], a_s[rows], b[perm], b_s[perm], off_p)
    assert np.array_equal(Cp, C[rows])


def test_expert_of_rows():
    off = np.array([0, 3, 3, 10], np.int32)
    assert list(G.expert_of_rows(off, [0, 2, 3, 9])) == [0, 0, 2, 2]

"""GPU parity of the routed-expert steps around the grouped product.

Routing and the gathered act_quant are integer/byte results and must equal
the oracle bit for bit; the combine is a fixed sequence of bf16 roundings and
must equal the oracle bit for bit too (oracle/moe.py, from "DeepSeek-V3
Administrator & Developer Guide" 6.4 / 8.4).  The whole routed-expert forward
(route -> gathered act_quant -> grouped [w1;w3] product -> SiLU gate and
act_quant -> grouped w2 product -> combine) is checked stage by stage, each
stage on its own GPU input: the integer and byte stages and the combine
bit-exact, the two FP8 products element-wise within their rounding bound
(their accumulation order is not fixed), the gate within one bf16 unit.  The
final output is then compared with the oracle's ``moe_forward`` element by
element, within a bound propagated from those stage bounds (a one-ulp bf16
difference in the gate's input can move a whole block's e4m3 codes, which
the bound allows only in blocks where the two chains' h differ).
"""

import json
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import gemm as G
from oracle import glue
from oracle import moe
from oracle import quant as Q

from gpu_helpers import dev_bf16, dev_f32, dev_u8, host_bits16, host_f32_bits, host_u8

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def host_i32(t):
    return t.contiguous().cpu().numpy()


def check_route(idx, E):
    off, rt, tr = ds.moe_route(dev_i32(idx), E)
    torch.cuda.synchronize()
    o_off, o_rt, _, o_tr = moe.route(idx, E)
    off, rt, tr = host_i32(off), host_i32(rt), host_i32(tr)
    assert np.array_equal(off, o_off)
    n = int(o_off[-1])
    assert np.array_equal(rt[:n], o_rt)
    assert np.array_equal(tr, o_tr)


def test_route_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "moe_route_small.json")))
    check_route(np.array(g["indices"], np.int32), g["experts"])


@pytest.mark.parametrize("T,E,k", [(4096, 256, 8), (1000, 64, 6), (37, 3, 2), (1, 8, 1), (700, 300, 16)])
def test_route_zipf(T, E, k):
    idx, _ = I.zipf_topk(T, E, k, 1.1, seed=T)
    check_route(idx, E)


def test_route_out_of_range_indices_get_no_row():
    idx, _ = I.zipf_topk(300, 16, 4, 1.1, seed=5)
    idx = idx.copy()
    idx[3, 1] = -1
    idx[77, 0] = 16
    idx[299, 3] = 1 << 30
    # the oracle's route ignores values outside [0, E) by construction
    check_route(idx, 16)


def test_route_no_tokens():
    off, _, tr = ds.moe_route(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 32)
    torch.cuda.synchronize()
    assert torch.all(off == 0) and tr.shape == (0, 8)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_act_quant_rows(fmt):
    T, K = 300, 7168
    x = I.activations((T, K), I.MOE, 31)
    rows = np.random.default_rng(2).integers(0, T, 1111).astype(np.int32)
    rows[:3] = [0, T - 1, 0]  # repeats and both ends
    y, s = ds.act_quant_rows(dev_bf16(x), dev_i32(rows), fmt)
    torch.cuda.synchronize()
    yr, sr = moe.gather_act_quant(x, rows, ue8m0=(fmt == "ue8m0"))
    assert np.array_equal(host_u8(y), yr)
    assert np.array_equal(host_f32_bits(s), sr.view(np.uint32))


def test_act_quant_rows_clamps_indices():
    T, K = 50, 384
    x = I.activations((T, K), I.MOE, 32)
    rows = np.array([-5, 0, 49, 50, 1 << 30, 7], np.int32)
    y, s = ds.act_quant_rows(dev_bf16(x), dev_i32(rows))
    torch.cuda.synchronize()
    yr, sr = Q.act_quant(x[np.clip(rows, 0, T - 1)])
    assert np.array_equal(host_u8(y), yr) and np.array_equal(host_f32_bits(s), sr.view(np.uint32))


@pytest.mark.parametrize("T,E,k,D", [(512, 64, 8, 7168), (200, 16, 2, 300), (33, 40, 16, 136), (64, 8, 1, 64),
                                     (100, 32, 6, 1000), (50, 16, 4, 3004), (40, 64, 8, 2056)])
def test_combine(T, E, k, D):
    idx, w = I.zipf_topk(T, E, k, 1.1, seed=D)
    _, _, _, tr = moe.route(idx, E)
    yr = I.activations((T * k, D), I.MOE, 40 + k, std=3.0)
    out = ds.moe_combine(dev_bf16(yr), dev_i32(idx), dev_bf16(w), dev_i32(tr))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits16(out), moe.combine(yr, w, idx, tr))


def test_combine_skips_pairs_without_row():
    T, E, k, D = 40, 8, 3, 256
    idx, w = I.zipf_topk(T, E, k, 1.1, seed=9)
    idx = idx.copy()
    idx[5, 2] = -1          # no row for this pair
    _, _, _, tr = moe.route(idx, E)
    assert tr[5, 2] == -1
    yr = I.activations((int((tr >= 0).sum()), D), I.MOE, 44)
    out = ds.moe_combine(dev_bf16(yr), dev_i32(idx), dev_bf16(w), dev_i32(tr))
    torch.cuda.synchronize()
    # the oracle sees the pair without a row as contributing nothing: drop it
    keep = tr >= 0
    ref = np.zeros((T, D), np.uint16)
    for t in range(T):
        kk = np.nonzero(keep[t])[0]
        ref[t] = moe.combine(yr, w[t:t + 1, kk], idx[t:t + 1, kk], tr[t:t + 1, kk])[0]
    assert np.array_equal(host_bits16(out), ref)


def test_combine_one_rank_of_experts():
    """The pairs routed to other ranks' experts get no row (routing with the
    local expert count), as in one rank's share under expert parallelism:
    each token combines only its local pairs, bit for bit the oracle's
    combine over those pairs."""
    T, E, k, D, El = 300, 64, 8, 7168, 8
    idx, w = I.zipf_topk(T, E, k, 1.1, seed=12)
    _, _, _, tr = moe.route(idx, El)
    R = int((tr >= 0).sum())
    yr = I.activations((max(R, 1), D), I.MOE, 45, std=3.0)
    out = ds.moe_combine(dev_bf16(yr), dev_i32(idx), dev_bf16(w), dev_i32(tr))
    torch.cuda.synchronize()
    got = host_bits16(out)
    for t in range(T):
        kk = np.nonzero(tr[t] >= 0)[0]
        if len(kk) == 0:
            assert np.all(got[t] == 0), f"token {t} without local pairs"
            continue
        ref = moe.combine(yr, w[t:t + 1, kk], idx[t:t + 1, kk], tr[t:t + 1, kk])[0]
        assert np.array_equal(got[t], ref), f"token {t}"


# Accumulation term of the products' element-wise bound, relative to
# (|A||W|^T)_ij: the matrix instruction sums each K-block's 128 fp8 products in
# hardware whose internal rounding is not documented; measured on random
# operands its error stays below half a bf16 unit plus 1e-5 (|A||W|^T), and in
# strongly cancelling sums (|C| ~ 3e-4 (|A||W|^T)) it reached 2.5e-5 (|A||W|^T)
# at K = 256, with either scale format.  1e-4 leaves a fourfold margin and is
# still about a hundred times tighter than the row/column tolerance.
ACC = 1e-4


def _bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _f64(bits):
    return F.bf16_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_routed_expert_forward(fmt):
    """The whole routed-expert forward, checked stage by stage on each
    stage's own GPU input (routing, gathered quantisation, gate
    quantisation and combine bit-exact; the two products element-wise
    within the product's rounding bound), then end to end against the
    oracle's chain with an element-wise bound propagated through the
    stages."""
    T, D, Fi, E, k = 160, 512, 256, 8, 2
    ue = fmt == "ue8m0"
    x = I.activations((T, D), I.MOE, 50)
    idx, w = I.zipf_topk(T, E, k, 1.1, seed=51)
    q13, s13, q2, s2 = [], [], [], []
    for e in range(E):
        a, b = Q.weight_quant(I.weights_f32((2 * Fi, D), I.MOE, 60 + e), ue8m0=ue)
        c, d = Q.weight_quant(I.weights_f32((D, Fi), I.MOE, 80 + e), ue8m0=ue)
        q13.append(a); s13.append(b); q2.append(c); s2.append(d)
    q13, s13, q2, s2 = map(np.stack, (q13, s13, q2, s2))

    xd, idd, wd = dev_bf16(x), dev_i32(idx), dev_bf16(w)
    off, row_token, tr = ds.moe_route(idd, E)
    xq, xs = ds.act_quant_rows(xd, row_token, fmt)
    h13 = ds.grouped_gemm(xq, xs, dev_u8(q13), dev_f32(s13), off, scale_fmt=fmt)
    hq, hs, h = ds.silu_mul_act_quant(h13[:, :Fi], h13[:, Fi:], fmt, return_h=True)
    yr = ds.grouped_gemm(hq, hs, dev_u8(q2), dev_f32(s2), off, scale_fmt=fmt)
    y = ds.moe_combine(yr, idd, wd, tr)
    torch.cuda.synchronize()
    gpu = dict(off=host_i32(off), row_token=host_i32(row_token), tr=host_i32(tr), xq=host_u8(xq),
               xs=xs.cpu().numpy(), h13=host_bits16(h13), h=host_bits16(h), hq=host_u8(hq), hs=hs.cpu().numpy(),
               yr=host_bits16(yr), y=host_bits16(y))
    check_routed_chain(x, idx, w, q13, s13, q2, s2, ue, gpu)


def check_routed_chain(x, idx, w, q13, s13, q2, s2, ue, gpu):
    """Stage-by-stage and end-to-end checks of a routed-expert forward whose
    stage outputs (host arrays) are in ``gpu``; raises AssertionError."""
    T, k = idx.shape
    E, D, Fi = q2.shape[0], q2.shape[1], q2.shape[2]
    # 1. routing and 2. the gathered quantisation: bit-exact
    o_ref, rt_ref, _, tr_ref = moe.route(idx, E)
    assert np.array_equal(gpu["off"], o_ref) and np.array_equal(gpu["tr"], tr_ref), "routing"
    assert np.array_equal(gpu["row_token"], rt_ref), "routing rows"
    xq_ref, xs_ref = moe.gather_act_quant(x, rt_ref, ue8m0=ue)
    assert np.array_equal(gpu["xq"], xq_ref), "gathered act_quant codes"
    assert np.array_equal(np.ascontiguousarray(gpu["xs"], np.float32).view(np.uint32), xs_ref.view(np.uint32))

    # 3. the up-projection on that input: the fp64 product rounded to bf16,
    #    within one bf16 unit plus ACC |A||W|^T for the accumulation
    h13g, hg, hqg, hsg, yrg = gpu["h13"], gpu["h"], gpu["hq"], gpu["hs"], gpu["yr"]
    got_bits = gpu["y"]
    R = T * k
    C13 = np.zeros((R, 2 * Fi))
    d13 = np.zeros((R, 2 * Fi))
    C2g = np.zeros((R, D))
    for e in range(E):
        lo, hi = o_ref[e], o_ref[e + 1]
        if hi == lo:
            continue
        A_hat = G.dequant_act(xq_ref[lo:hi], xs_ref[lo:hi])
        W_hat = G.dequant_weight(q13[e], s13[e])
        C13[lo:hi] = A_hat @ W_hat.T
        d13[lo:hi] = _bf16_ulp(C13[lo:hi]) + ACC * (np.abs(A_hat) @ np.abs(W_hat).T)
        # 5. the down-projection on the GPU's own quantised h, same bound
        H_hat = G.dequant_act(hqg[lo:hi], hsg[lo:hi])
        W2_hat = G.dequant_weight(q2[e], s2[e])
        C2g[lo:hi] = H_hat @ W2_hat.T
        d2 = _bf16_ulp(C2g[lo:hi]) + ACC * (np.abs(H_hat) @ np.abs(W2_hat).T)
        assert np.all(np.abs(_f64(yrg[lo:hi]) - C2g[lo:hi]) <= d2), f"down-projection, expert {e}"
    assert np.all(np.abs(_f64(h13g) - C13) <= d13), "up-projection outside its rounding bound"

    # 4. the gate on the GPU's h13 (within one bf16 unit of the correctly
    #    rounded value), and the quantisation of the GPU's h: bit-exact
    h_on_gpu_input = glue.silu_mul(h13g[:, :Fi], h13g[:, Fi:])
    rv = _f64(h_on_gpu_input)
    assert np.all((np.abs(_f64(hg) - rv) <= _bf16_ulp(rv) + 1e-40) | ((np.abs(rv) < 2.0 ** -100) & (_f64(hg) == 0)))
    hq_o, hs_o = Q.act_quant(hg, ue8m0=ue)
    assert np.array_equal(hqg, hq_o), "gate quantisation codes"
    assert np.array_equal(np.ascontiguousarray(hsg, np.float32).view(np.uint32), hs_o.view(np.uint32))

    # 6. the combine on the GPU's expert outputs: bit-exact
    assert np.array_equal(got_bits, moe.combine(yrg, w, idx, tr_ref)), "combine"

    # End to end, element-wise, against the oracle's own chain (which is
    # moe_forward's): bound the difference of each stage's result from the
    # bounds above and propagate it.
    h13_ref = F.f32_to_bf16(C13)
    h_ref = glue.silu_mul(h13_ref[:, :Fi], h13_ref[:, Fi:])
    hq_ref, hs_ref = Q.act_quant(h_ref, ue8m0=ue)
    yr_ref = np.zeros((R, D), np.uint16)
    C2r = np.zeros((R, D))
    for e in range(E):
        lo, hi = o_ref[e], o_ref[e + 1]
        if hi > lo:
            C2r[lo:hi] = G.dequant_act(hq_ref[lo:hi], hs_ref[lo:hi]) @ G.dequant_weight(q2[e], s2[e]).T
            yr_ref[lo:hi] = F.f32_to_bf16(C2r[lo:hi])
    out_ref = moe.combine(yr_ref, w, idx, tr_ref)
    assert np.array_equal(out_ref, moe.moe_forward(x, idx, w, q13, s13, q2, s2, ue8m0=ue))
    # h: the gate's slope is below 1.1, so |dh| <= 1.1 |h3| d1 + |SiLU(h1)| d3 + d1 d3 plus one bf16
    # unit of each side's rounding
    g1, g3 = _f64(h13_ref[:, :Fi]), _f64(h13_ref[:, Fi:])
    d1, d3 = d13[:, :Fi], d13[:, Fi:]
    with np.errstate(over="ignore"):
        sil = np.abs(glue.silu(g1))
    hr = _f64(h_ref)
    dh = 1.1 * np.abs(g3) * d1 + sil * d3 + d1 * d3 + 2 * _bf16_ulp(np.abs(hr) + 1e-30)
    # quantised h, element by element: where the two chains' block scales
    # agree, an element whose h agrees bit for bit has the same code, and
    # otherwise the two codes differ by at most |dh| plus one e4m3 step at
    # that magnitude (two half-step roundings); where the scales differ, both
    # quantisation errors (half an e4m3 step: 2^-4 relative, or 2^-10 s below
    # the normal range) plus |dh|
    s_g = np.repeat(np.asarray(hsg, np.float64), 128, axis=1)
    s_r = np.repeat(np.asarray(hs_ref, np.float64), 128, axis=1)
    same_s = np.repeat(np.ascontiguousarray(hsg, np.float32).view(np.uint32) == hs_ref.view(np.uint32), 128, axis=1)
    hmax = np.maximum(np.abs(_f64(hg)), np.abs(hr))
    v = hmax / s_r
    step = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3), 2.0 ** -9) * s_r
    loose = 2.0 ** -4 * (np.abs(_f64(hg)) + np.abs(hr)) + 2.0 ** -10 * (s_g + s_r) + dh
    dq = np.where(same_s, np.where(hg == h_ref, 0.0, dh + step), loose)
    # expert outputs: |dy| <= |dq| |W2|^T + the GPU product's bound + both bf16 roundings
    dy = np.zeros((R, D))
    for e in range(E):
        lo, hi = o_ref[e], o_ref[e + 1]
        if hi > lo:
            W2a = np.abs(G.dequant_weight(q2[e], s2[e]))
            H_hat = G.dequant_act(hqg[lo:hi], hsg[lo:hi])
            dy[lo:hi] = dq[lo:hi] @ W2a.T + ACC * (np.abs(H_hat) @ W2a.T)
    dy += _bf16_ulp(C2g) + _bf16_ulp(C2r)
    # combine: sum_j |w_j| |dy_j| plus, for each chain, its 2k bf16 roundings
    # (each at most 2^-8 of a partial sum bounded by sum_j |w_j y_j|)
    wv = _f64(w)
    bound = np.zeros((T, D))
    mag = np.zeros((T, D))
    for j in range(k):
        rows = tr_ref[:, j]
        bound += np.abs(wv[:, j:j + 1]) * dy[rows]
        mag += np.abs(wv[:, j:j + 1]) * np.maximum(np.abs(_f64(yrg[rows])), np.abs(_f64(yr_ref[rows])))
    bound += 2 * (2 * k + 1) * 2.0 ** -8 * mag + 1e-30
    diff = np.abs(_f64(got_bits) - _f64(out_ref))
    bad = diff > bound
    assert not bad.any(), f"end-to-end output outside its bound at {np.argwhere(bad)[:5].tolist()}"

"""GPU parity of the routed-expert steps around the grouped product.

Routing and the gathered act_quant are integer/byte results and must equal
the oracle bit for bit; the combine is a fixed sequence of bf16 roundings and
must equal the oracle bit for bit too (oracle/moe.py, from "DeepSeek-V3
Administrator & Developer Guide" 6.4 / 8.4).  The whole routed-expert forward
(route -> gathered act_quant -> grouped [w1;w3] product -> SiLU gate and
act_quant -> grouped w2 product -> combine) is compared with the oracle's
``moe_forward`` within a product tolerance: its two FP8 products are not
bit-reproducible, and a one-ulp bf16 difference in the gate input can move an
e4m3 code by one step.
"""

import json
import os

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
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
                                     (100, 32, 6, 1000)])
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


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_routed_expert_forward(fmt):
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
    ref = F.bf16_to_f32(moe.moe_forward(x, idx, w, q13, s13, q2, s2, ue8m0=ue)).astype(np.float64)

    xd, idd, wd = dev_bf16(x), dev_i32(idx), dev_bf16(w)
    off, row_token, tr = ds.moe_route(idd, E)
    xq, xs = ds.act_quant_rows(xd, row_token, fmt)
    h13 = ds.grouped_gemm(xq, xs, dev_u8(q13), dev_f32(s13), off, scale_fmt=fmt)
    hq, hs = ds.silu_mul_act_quant(h13[:, :Fi], h13[:, Fi:], fmt)
    yr = ds.grouped_gemm(hq, hs, dev_u8(q2), dev_f32(s2), off, scale_fmt=fmt)
    y = ds.moe_combine(yr, idd, wd, tr)
    torch.cuda.synchronize()
    got = F.bf16_to_f32(host_bits16(y)).astype(np.float64)
    assert np.all(np.isfinite(got))
    fro = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert fro <= 2e-2, f"relative Frobenius error {fro:.3e}"
    row = np.abs(got - ref).max(axis=1) / (np.abs(ref).max(axis=1) + 1e-30)
    assert np.median(row) <= 2e-2 and row.max() <= 0.25, (np.median(row), row.max())

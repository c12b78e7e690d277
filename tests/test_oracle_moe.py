"""Pins of the routed-expert oracle (oracle/moe.py) on the CPU.

route: a hand-worked example (tests/golden/moe_route_small.json) and
invariants against np.bincount on Zipf-routed tokens.  combine: closed forms
that fix the expert order, the bf16 rounding of each product and of each
addition, and an error bound against the fp64 sum.  moe_forward: with all
experts equal and weights 1/2, the routed output is the dense expert's.
"""

import json
import os

import numpy as np
import pytest

from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import moe
from oracle import quant as Q

HERE = os.path.dirname(os.path.abspath(__file__))


def bf(v):
    return F.f32_to_bf16(np.asarray(v, np.float64))


def test_route_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "moe_route_small.json")))
    off, rt, rs, tr = moe.route(np.array(g["indices"]), g["experts"])
    assert off.tolist() == g["offsets"]
    assert rt.tolist() == g["row_token"]
    assert rs.tolist() == g["row_slot"]
    assert tr.tolist() == g["token_rows"]


def test_route_invariants_zipf():
    idx, _ = I.zipf_topk(512, 64, 6, 1.1)
    off, rt, rs, tr = moe.route(idx, 64)
    assert np.array_equal(np.diff(off), np.bincount(idx.ravel(), minlength=64))
    R = idx.size
    assert off[-1] == R and sorted(tr.ravel().tolist()) == list(range(R))
    # row r is pair (rt[r], rs[r]) of expert e, and token_rows inverts it
    for e in range(64):
        rows = np.arange(off[e], off[e + 1])
        assert np.all(idx[rt[rows], rs[rows]] == e)
        flat = rt[rows] * idx.shape[1] + rs[rows]
        assert np.all(np.diff(flat) > 0), "rows of an expert follow row-major pair order"
    assert np.all(tr[rt, rs] == np.arange(R))


def test_route_empty_and_unused_experts():
    off, rt, rs, tr = moe.route(np.zeros((0, 4), np.int32), 3)
    assert off.tolist() == [0, 0, 0, 0] and rt.size == 0 and tr.shape == (0, 4)
    off, _, _, _ = moe.route(np.array([[5, 5]]).reshape(2, 1), 8)
    assert off.tolist() == [0, 0, 0, 0, 0, 0, 2, 2, 2]


def test_gather_act_quant_identity_and_permutation():
    x = I.activations((20, 384), I.MOE, 5)
    y0, s0 = Q.act_quant(x)
    y1, s1 = moe.gather_act_quant(x, np.arange(20))
    assert np.array_equal(y0, y1) and np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
    perm = np.random.default_rng(1).permutation(20)
    y2, s2 = moe.gather_act_quant(x, perm)
    assert np.array_equal(y2, y0[perm]) and np.array_equal(s2, s0[perm])


def test_combine_single_expert_unit_weight():
    yr = I.activations((12, 64), I.MOE, 7)
    idx = np.arange(12, dtype=np.int32)[::-1].reshape(12, 1) % 5
    _, _, _, tr = moe.route(idx, 5)
    out = moe.combine(yr, bf(np.ones((12, 1))), idx, tr)
    assert np.array_equal(out, yr[tr[:, 0]])


def test_combine_equal_quarters():
    # four contributions of v/4 each: v/4, v/2, 3v/4 and v are all exact in bf16
    v = bf(np.array([[1.5, -3.25, 96.0, 0.0078125]]))
    yr = np.repeat(v, 4, axis=0)
    idx = np.array([[3, 0, 2, 1]], np.int32)
    _, _, _, tr = moe.route(idx, 4)
    out = moe.combine(yr, bf(np.full((1, 4), 0.25)), idx, tr)
    assert np.array_equal(out, v[0][None, :])


@pytest.mark.parametrize("big_expert,expect", [(0, 1.0), (2, 1.0 + 2.0 ** -7)])
def test_combine_order_and_rounding_of_sums(big_expert, expect):
    # one 1.0 and two 2^-8 contributions.  Increasing expert order with bf16
    # rounding after each addition: if 1.0 comes first, 1 + 2^-8 is a tie and
    # rounds to 1.0 twice; if it comes last, 2^-8 + 2^-8 = 2^-7 is exact and
    # 1 + 2^-7 is a bf16 value.  (The fp64 sum would be 1 + 2^-7 either way.)
    idx = np.array([[0, 1, 2]], np.int32)
    vals = np.full(3, 2.0 ** -8)
    vals[big_expert] = 1.0
    _, _, _, tr = moe.route(idx, 3)
    yr = bf(vals[:, None])  # row r belongs to expert r here
    out = moe.combine(yr, bf(np.ones((1, 3))), idx, tr)
    assert F.bf16_to_f32(out)[0, 0] == np.float32(expect)


def test_combine_rounds_each_product():
    # p1 = (1 + 2^-7)^2 = 1 + 2^-6 + 2^-14 rounds to 1 + 2^-6; adding 2^-8 then
    # lands exactly on the tie between 1 + 2^-6 and 1 + 3*2^-7, which rounds to
    # the even 1 + 2^-6.  Without the product rounding the sum would exceed
    # the tie and round up.
    idx = np.array([[4, 9]], np.int32)
    _, _, _, tr = moe.route(idx, 10)
    yr = bf(np.array([[1.0 + 2.0 ** -7], [2.0 ** -8]]))
    w = bf(np.array([[1.0 + 2.0 ** -7, 1.0]]))
    out = moe.combine(yr, w, idx, tr)
    assert F.bf16_to_f32(out)[0, 0] == np.float32(1.0 + 2.0 ** -6)


def test_combine_error_bound_random():
    idx, w = I.zipf_topk(300, 32, 8, 1.1)
    _, _, _, tr = moe.route(idx, 32)
    yr = I.activations((idx.size, 96), I.MOE, 11)
    out = F.bf16_to_f32(moe.combine(yr, w, idx, tr)).astype(np.float64)
    terms = F.bf16_to_f32(yr).astype(np.float64)[tr] * F.bf16_to_f32(w).astype(np.float64)[:, :, None]
    exact = terms.sum(axis=1)
    bound = 2 * 8 * 2.0 ** -8 * np.abs(terms).sum(axis=1) + 1e-30
    assert np.all(np.abs(out - exact) <= bound)


def test_moe_forward_equal_experts_is_dense_expert():
    T, D, Fi, E, k = 24, 256, 128, 4, 2
    x = I.activations((T, D), I.MOE, 21)
    q13, s13 = Q.weight_quant(I.weights_f32((2 * Fi, D), I.MOE, 22))
    q2, s2 = Q.weight_quant(I.weights_f32((D, Fi), I.MOE, 23))
    g = np.random.default_rng(3)
    idx = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = bf(np.full((T, k), 0.5))
    stack = lambda a: np.stack([a] * E)
    y = moe.moe_forward(x, idx, w, stack(q13), stack(s13), stack(q2), stack(s2))
    dense = moe.expert_ffn(x, q13, s13, q2, s2)
    assert np.array_equal(y, dense)

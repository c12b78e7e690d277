"""The routed-expert chain check of test_gpu_moe on the CPU: it must accept a
chain whose stages deviate from the oracle only as a correct GPU chain may
(products rounded after an fp32-sized accumulation error, a gate that is one
bf16 unit off in a few elements), and reject chains with a planted mistake
(a mis-routed expert, a dropped weight, a wrong product, a wrong scale).
"""

import numpy as np
import pytest

from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import gemm as G
from oracle import glue
from oracle import moe
from oracle import quant as Q

from test_gpu_moe import check_routed_chain


def _problem(ue):
    T, D, Fi, E, k = 96, 256, 128, 6, 2
    x = I.activations((T, D), I.MOE, 150)
    idx, w = I.zipf_topk(T, E, k, 1.1, seed=151)
    q13, s13, q2, s2 = [], [], [], []
    for e in range(E):
        a, b = Q.weight_quant(I.weights_f32((2 * Fi, D), I.MOE, 160 + e), ue8m0=ue)
        c, d = Q.weight_quant(I.weights_f32((D, Fi), I.MOE, 180 + e), ue8m0=ue)
        q13.append(a); s13.append(b); q2.append(c); s2.append(d)
    return x, idx, w, *map(np.stack, (q13, s13, q2, s2))


def _simulated_chain(x, idx, w, q13, s13, q2, s2, ue, rng, plant=None):
    """A chain as a correct GPU computes it: the oracle's stages with the
    products perturbed by up to 1e-6 |A||W|^T before bf16 rounding and the
    gate moved by one bf16 unit in 0.2% of its elements."""
    E = q13.shape[0]
    Fi = q2.shape[2]
    off, rt, _, tr = moe.route(idx, E)
    xq, xs = moe.gather_act_quant(x, rt, ue8m0=ue)
    R = len(rt)
    h13 = np.zeros((R, 2 * Fi), np.uint16)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            A = G.dequant_act(xq[lo:hi], xs[lo:hi])
            W = G.dequant_weight(q13[e], s13[e])
            C = A @ W.T + rng.uniform(-1e-6, 1e-6, (hi - lo, 2 * Fi)) * (np.abs(A) @ np.abs(W).T)
            h13[lo:hi] = F.f32_to_bf16(C)
    h = glue.silu_mul(h13[:, :Fi], h13[:, Fi:])
    flip = rng.random(h.shape) < 2e-3
    h = np.where(flip & (h & 0x7F80 != 0) & (h & 0x7F80 != 0x7F80), h + rng.choice([-1, 1], h.shape), h)
    h = h.astype(np.uint16)
    hq, hs = Q.act_quant(h, ue8m0=ue)
    if plant == "scale":
        hs = hs.copy()
        hs[3, 0] *= 2
    yr = np.zeros((R, q2.shape[1]), np.uint16)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            e2 = (e + 1) % E if plant == "misroute" and e == 2 else e
            A = G.dequant_act(hq[lo:hi], hs[lo:hi])
            W = G.dequant_weight(q2[e2], s2[e2])
            C = A @ W.T + rng.uniform(-1e-6, 1e-6, (hi - lo, W.shape[0])) * (np.abs(A) @ np.abs(W).T)
            if plant == "product" and e == 1:
                C = C * 1.01
            yr[lo:hi] = F.f32_to_bf16(C)
    wts = w.copy()
    if plant == "weight":
        wts[5, 1] = 0
    y = moe.combine(yr, wts, idx, tr)
    return dict(off=off, row_token=rt, tr=tr, xq=xq, xs=xs, h13=h13, h=h, hq=hq, hs=hs, yr=yr, y=y)


@pytest.mark.parametrize("ue", [False, True])
def test_accepts_a_correct_chain(ue):
    prob = _problem(ue)
    for seed in range(3):
        check_routed_chain(*prob, ue, _simulated_chain(*prob, ue, np.random.default_rng(seed)))


@pytest.mark.parametrize("plant", ["misroute", "weight", "product", "scale"])
def test_rejects_planted_mistakes(plant):
    prob = _problem(False)
    with pytest.raises(AssertionError):
        check_routed_chain(*prob, False, _simulated_chain(*prob, False, np.random.default_rng(0), plant))

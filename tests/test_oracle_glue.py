"""Pins of the SiLU-gate oracle (CPU only), Admin Guide 1.2 (MLP / Expert).

SiLU has closed forms and identities independent of how it is evaluated:
SiLU(0) = 0, SiLU(v) - SiLU(-v) = v, SiLU(v) = v * logistic(v) (scipy's
expit); the bf16 rounding of the product is checked against an exact
rational rounding of the same fp64 value.
"""

import numpy as np
from scipy.special import expit

from oracle import formats as F
from oracle import glue


def test_silu_identities():
    v = np.linspace(-30, 30, 10001)
    s = glue.silu(v)
    assert glue.silu(np.array([0.0]))[0] == 0.0
    assert np.allclose(s - glue.silu(-v), v, rtol=0, atol=1e-13)
    assert np.allclose(s, v * expit(v), rtol=1e-14, atol=1e-300)
    assert np.all(glue.silu(np.array([-800.0, 800.0])) == np.array([-0.0, 800.0]))


def test_silu_mul_rounding():
    g = np.random.default_rng(0)
    gb = F.f32_to_bf16((g.standard_normal(4000) * 3).astype(np.float32))
    ub = F.f32_to_bf16((g.standard_normal(4000) * 3).astype(np.float32))
    h = glue.silu_mul(gb, ub)
    exact = glue.silu_mul_f64(gb, ub)
    for hv, ev in zip(h, exact):
        assert hv == F.f32_to_bf16_scalar(ev)

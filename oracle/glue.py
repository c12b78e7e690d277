"""SiLU(g) * u between the up and down projections (oracle; test infrastructure only).

Admin Guide ("DeepSeek-V3 Administrator & Developer Guide", doccompiler) 1.2,
``MLP`` and ``Expert`` rows: the feed-forward computes ``w2(SiLU(w1 x) * w3 x)``.
The pages name only the formula.  Reading taken: the inputs are the bf16
outputs of the two up-projection products, SiLU(g) = g / (1 + exp(-g)), the
product with u is formed at higher precision (fp64 here) and rounded once to
bf16 (round-to-nearest-even).  The result is then quantised by ``act_quant``.

A GPU evaluation in fp32 with a hardware exponential is not bit-reproducible
against this; comparisons against ``silu_mul`` allow one bf16 unit in the last
place (see the tests), and the quantised output is compared bit-exactly only
on blocks whose bf16 values agree.
"""

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def silu_mul(g_bits, u_bits):
    """``bf16(SiLU(g) * u)`` from bf16 bit patterns, returned as uint16 bits."""
    g = bf16_to_f32(g_bits).astype(np.float64)
    u = bf16_to_f32(u_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        h = silu(g) * u
    return f32_to_bf16(h)


def silu_mul_f64(g_bits, u_bits):
    """Unrounded fp64 value of SiLU(g) * u (used to bound the GPU's error)."""
    g = bf16_to_f32(g_bits).astype(np.float64)
    u = bf16_to_f32(u_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        return silu(g) * u

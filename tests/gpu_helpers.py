"""Helpers shared by the GPU parity tests: host<->device transfer of raw bits and
the product tolerance check.

GEMM tolerance (the product's accumulation order is not fixed, so results are
compared against the fp64 oracle of the same quantised operands):
  max_ij |C - C_ref| / (||A_hat_i||_2 ||W_hat_j||_2) <= 1e-2   and
  ||C - C_ref||_F / ||C_ref||_F <= 5e-3.
The bf16 rounding of the output alone contributes at most 2^-9 relative per
element (about 1.1e-3 in the Frobenius ratio for random data); fp32
accumulation over K <= 18432 adds far less.
"""

import numpy as np
import torch

from oracle import formats as F
from oracle import gemm as G

MAX_REL_ROWCOL = 1e-2
FRO_REL = 5e-3


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(b):
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_scales(a_s, layout):
    """Activation scales [M, KB] on the device, stored row-major ("row") or
    K-block-major ("kb", a transposed view with strides (1, M))."""
    if layout == "row":
        return dev_f32(a_s)
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a_s, np.float32).T)).cuda().t()


def host_bits16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.contiguous().cpu().numpy()


def host_f32_bits(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


def bf16_to_f64(bits):
    return F.bf16_to_f32(bits).astype(np.float64)


def check_product(C_bits, C_ref, A_hat, W_hat, what=""):
    """Tolerance check of a bf16 product against the fp64 oracle (see module doc)."""
    C = bf16_to_f64(C_bits)
    assert C.shape == C_ref.shape, (C.shape, C_ref.shape)
    assert np.all(np.isfinite(C)), f"{what}: non-finite output"
    na = np.linalg.norm(A_hat, axis=1)
    nw = np.linalg.norm(W_hat, axis=1)
    denom = np.outer(na, nw)
    err = np.abs(C - C_ref)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(denom > 0, err / denom, np.where(err > 0, np.inf, 0.0))
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= MAX_REL_ROWCOL, f"{what}: max row/col-scaled error {worst:.3e}"
    fro_ref = np.linalg.norm(C_ref)
    if fro_ref > 0:
        fro = float(np.linalg.norm(C - C_ref) / fro_ref)
        assert fro <= FRO_REL, f"{what}: relative Frobenius error {fro:.3e}"
    return worst


def check_gemm_full(C_bits, a, a_s, b, b_s, what=""):
    A_hat = G.dequant_act(a, a_s)
    W_hat = G.dequant_weight(b, b_s)
    return check_product(C_bits, A_hat @ W_hat.T, A_hat, W_hat, what)

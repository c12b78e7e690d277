"""dsfp8: block-scaled FP8 linear layer for AMD MI355X (gfx950).

Python binding of libdsfp8.so.  Each function checks tensor placement and
dtypes, allocates its outputs with torch on the input's device, and calls the
C entry point of the same name on torch's current stream; every step of the
computation runs in the library's HIP kernels.  e4m3 tensors are exchanged as
``torch.uint8`` (``torch.float8_e4m3fn`` inputs are accepted and viewed as
bytes).  Scales are ``torch.float32``.  Activation scales are indexed
``[M, ceil(K/128)]`` as on the pages; the quantisers return them stored
K-block-major (a transposed view, strides ``(1, M)``), which is the layout the
products read fastest, and the products accept either storage order.

The operations follow the DeepSeek-V3 inference kernels as described in the
"DeepSeek-V3 Administrator & Developer Guide" (sections 6.3, 6.4, 8.5) and the
DocSearch index of the DeepSeek-V3 README (item 3, weight_scale_inv); see
include/dsfp8.h for the exact contracts.
"""

import torch

from . import _lib

BLOCK = 128
_SCALE_FMT = {"fp32": 0, "ue8m0": 1}


class Dsfp8Error(ValueError):
    """A libdsfp8 call rejected its arguments or failed to launch."""


def kblocks(n):
    return (int(n) + BLOCK - 1) // BLOCK


def status_string(st):
    return _lib.load().dsfp8_status_string(int(st)).decode()


def abi_version():
    return _lib.load().dsfp8_abi_version()


def _check(name, st):
    if st != 0:
        raise Dsfp8Error(f"{name}: {status_string(st)} (status {st})")


def _fmt(scale_fmt):
    if scale_fmt not in _SCALE_FMT:
        raise Dsfp8Error(f"scale_fmt must be one of {sorted(_SCALE_FMT)}, got {scale_fmt!r}")
    return _SCALE_FMT[scale_fmt]


def _bytes(t):
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def _mat(t, name, dtypes, dim=2):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise Dsfp8Error(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise Dsfp8Error(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.dim() != dim:
        raise Dsfp8Error(f"{name} must be {dim}-D, got {t.dim()} dimensions")
    if t.numel() > 0 and t.stride(-1) != 1:
        raise Dsfp8Error(f"{name}: the last dimension needs stride 1")
    return t


def _ld(t):
    return t.stride(-2) if t.numel() > 0 else t.shape[-1]


def _scale_strides(t):
    """(row stride, K-block stride) of an activation-scale matrix [M, KB]."""
    M, KB = t.shape
    rs = t.stride(0) if M > 1 else (1 if KB <= 1 or t.stride(1) != 1 else KB)
    ks = t.stride(1) if KB > 1 else (1 if M <= 1 or t.stride(0) != 1 else M)
    return rs, ks


def _scale_matrix(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.dim() != 2:
        raise Dsfp8Error(f"{name} must be a 2-D float32 CUDA tensor")
    return _scale_strides(t)


def new_scales(M, KB, device):
    """An activation-scale matrix [M, KB] stored K-block-major (strides (1, M))."""
    return torch.empty((KB, M), dtype=torch.float32, device=device).t()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _out(out, shape, dtype, device, name):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _mat(_bytes(out), name, (dtype,), dim=len(shape))
    if tuple(out.shape) != tuple(shape) or out.device != device:
        raise Dsfp8Error(f"{name} must be {tuple(shape)} on {device}, got {tuple(out.shape)} on {out.device}")
    return _bytes(out)


def _scales_out(out, M, KB, device):
    if out is None:
        return new_scales(M, KB, device)
    if tuple(out.shape) != (M, KB) or out.device != device:
        raise Dsfp8Error(f"s must be {(M, KB)} on {device}, got {tuple(out.shape)} on {out.device}")
    _scale_matrix(out, "s")
    return out


def act_quant(x, scale_fmt="fp32", out=None):
    """Quantise bf16 ``x [M, K]`` per row and per 128 columns.

    Returns ``(y uint8 [M, K], s float32 [M, ceil(K/128)])`` with x ~= e4m3(y) * s.
    ``out`` may supply preallocated ``(y, s)`` (row strides are honoured; s
    may be row-major or K-block-major).
    """
    _mat(x, "x", (torch.bfloat16,))
    M, K = x.shape
    yo, so = out if out is not None else (None, None)
    y = _out(yo, (M, K), torch.uint8, x.device, "y")
    s = _scales_out(so, M, kblocks(K), x.device)
    srs, sks = _scale_strides(s)
    st = _lib.load().dsfp8_act_quant(x.data_ptr(), M, K, _ld(x), y.data_ptr(), _ld(y), s.data_ptr(), srs, sks,
                                     _fmt(scale_fmt), _stream(x))
    _check("act_quant", st)
    return y, s


def silu_mul_act_quant(g, u, scale_fmt="fp32", return_h=False, out=None):
    """``act_quant(bf16(SiLU(g) * u))`` in one pass; optionally also return h.

    ``out`` may supply preallocated ``(y, s)``."""
    _mat(g, "g", (torch.bfloat16,))
    _mat(u, "u", (torch.bfloat16,))
    if g.shape != u.shape:
        raise Dsfp8Error(f"g and u must have the same shape, got {tuple(g.shape)} and {tuple(u.shape)}")
    M, I = g.shape
    yo, so = out if out is not None else (None, None)
    y = _out(yo, (M, I), torch.uint8, g.device, "y")
    s = _scales_out(so, M, kblocks(I), g.device)
    srs, sks = _scale_strides(s)
    h = torch.empty((M, I), dtype=torch.bfloat16, device=g.device) if return_h else None
    st = _lib.load().dsfp8_silu_mul_act_quant(
        g.data_ptr(), _ld(g), u.data_ptr(), _ld(u), M, I, y.data_ptr(), _ld(y), s.data_ptr(), srs, sks,
        h.data_ptr() if h is not None else None, I, _fmt(scale_fmt), _stream(g))
    _check("silu_mul_act_quant", st)
    return (y, s, h) if return_h else (y, s)


def weight_quant(w, scale_fmt="fp32"):
    """Quantise fp32 or bf16 weights ``[N, K]`` to e4m3 with 128x128 fp32 block scales."""
    _mat(w, "w", (torch.float32, torch.bfloat16))
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    S = torch.empty((kblocks(N), kblocks(K)), dtype=torch.float32, device=w.device)
    dtype = 0 if w.dtype == torch.float32 else 1
    st = _lib.load().dsfp8_weight_quant(w.data_ptr(), dtype, N, K, _ld(w), q.data_ptr(), K, S.data_ptr(),
                                        kblocks(K), _fmt(scale_fmt), _stream(w))
    _check("weight_quant", st)
    return q, S


def weight_dequant(q, S, out=None):
    """bf16 ``[N, K]`` = e4m3 ``q`` times its 128x128 block scale ``S``."""
    q = _mat(_bytes(q), "w", (torch.uint8,))
    _mat(S, "s", (torch.float32,))
    N, K = q.shape
    if tuple(S.shape) != (kblocks(N), kblocks(K)):
        raise Dsfp8Error(f"scale grid must be {(kblocks(N), kblocks(K))}, got {tuple(S.shape)}")
    out = _out(out, (N, K), torch.bfloat16, q.device, "out")
    st = _lib.load().dsfp8_weight_dequant(q.data_ptr(), N, K, _ld(q), S.data_ptr(), _ld(S), out.data_ptr(),
                                          _ld(out), _stream(q))
    _check("weight_dequant", st)
    return out


def gemm(a, a_s, b, b_s, out=None, scale_fmt="fp32"):
    """bf16 ``C [M, N] = A W^T`` with per-K-block scales (A e4m3 [M,K], W e4m3 [N,K]).

    ``scale_fmt="ue8m0"`` declares every scale a power of two (as produced by
    the quantisers with that format); the matrix instruction then applies
    them from their exponents.
    """
    a = _mat(_bytes(a), "a", (torch.uint8,))
    b = _mat(_bytes(b), "b", (torch.uint8,))
    ars, aks = _scale_matrix(a_s, "a_s")
    _mat(b_s, "b_s", (torch.float32,))
    M, K = a.shape
    N, K2 = b.shape
    if K2 != K:
        raise Dsfp8Error(f"a and b disagree on K: {K} vs {K2}")
    if tuple(a_s.shape) != (M, kblocks(K)) or tuple(b_s.shape) != (kblocks(N), kblocks(K)):
        raise Dsfp8Error("scale shapes must be a_s [M, ceil(K/128)] and b_s [ceil(N/128), ceil(K/128)]")
    lib = _lib.load()
    c = _out(out, (M, N), torch.bfloat16, a.device, "out")
    wsb = lib.dsfp8_gemm_workspace_bytes(M, N, K)
    # zero-filled, as the split products' arrival counters require
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=a.device) if wsb else None
    st = lib.dsfp8_gemm(a.data_ptr(), _ld(a), a_s.data_ptr(), ars, aks, b.data_ptr(), _ld(b), b_s.data_ptr(),
                        _ld(b_s), c.data_ptr(), _ld(c), M, N, K, _fmt(scale_fmt),
                        ws.data_ptr() if ws is not None else None, wsb, _stream(a))
    _check("gemm", st)
    return c


def grouped_gemm(a, a_s, b, b_s, offsets, out=None, workspace=None, scale_fmt="fp32"):
    """Per-expert product over row ranges: rows ``offsets[e]:offsets[e+1]`` of A use W[e].

    ``b`` is e4m3 ``[E, N, K]``, ``b_s`` fp32 ``[E, ceil(N/128), ceil(K/128)]``,
    ``offsets`` int32 ``[E+1]`` on the device.  Returns bf16 ``[M_total, N]``.
    ``scale_fmt`` as for :func:`gemm`.
    """
    a = _mat(_bytes(a), "a", (torch.uint8,))
    b = _mat(_bytes(b), "b", (torch.uint8,), dim=3)
    ars, aks = _scale_matrix(a_s, "a_s")
    _mat(b_s, "b_s", (torch.float32,), dim=3)
    if not offsets.is_cuda or offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise Dsfp8Error("offsets must be a contiguous int32 CUDA tensor of length E+1")
    M, K = a.shape
    E, N, K2 = b.shape
    if K2 != K or offsets.numel() != E + 1:
        raise Dsfp8Error("shape mismatch between a, b and offsets")
    if not b.is_contiguous() or not b_s.is_contiguous():
        raise Dsfp8Error("b and b_s need contiguous storage")
    if tuple(b_s.shape) != (E, kblocks(N), kblocks(K)) or tuple(a_s.shape) != (M, kblocks(K)):
        raise Dsfp8Error("scale shapes must be a_s [M, ceil(K/128)] and b_s [E, ceil(N/128), ceil(K/128)]")
    lib = _lib.load()
    c = _out(out, (M, N), torch.bfloat16, a.device, "out")
    wsb = lib.dsfp8_grouped_gemm_workspace_bytes(E, M, N, K)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=a.device)
    st = lib.dsfp8_grouped_gemm(a.data_ptr(), _ld(a), a_s.data_ptr(), ars, aks, b.data_ptr(), K, b_s.data_ptr(),
                                kblocks(K), offsets.data_ptr(), E, M, N, K, c.data_ptr(), _ld(c), _fmt(scale_fmt),
                                workspace.data_ptr(), workspace.numel(), _stream(a))
    _check("grouped_gemm", st)
    return c


def _glu_outputs(M, F, device, out, return_h):
    yo, so = out if out is not None else (None, None)
    y = _out(yo, (M, F), torch.uint8, device, "y")
    s = _scales_out(so, M, kblocks(F), device)
    h = torch.empty((M, F), dtype=torch.bfloat16, device=device) if return_h else None
    return y, s, h


def gemm_silu_mul_act_quant(a, a_s, w13, w13_s, scale_fmt="fp32", return_h=False, out=None):
    """The gated up-projection in one kernel: ``act_quant(bf16(SiLU(h1) * h3))``
    with ``h1 = gemm(a, a_s, w1, s1)`` and ``h3 = gemm(a, a_s, w3, s3)``, where
    ``w13`` e4m3 ``[2F, K]`` stacks w1 over w3 and ``w13_s`` their scale grids
    ``[2F/128, ceil(K/128)]``.  Equal to :func:`gemm` followed by
    :func:`silu_mul_act_quant` on the two halves.  Returns ``(y, s)`` or
    ``(y, s, h)``; ``out`` may supply ``(y, s)``.  ``scale_fmt`` applies to the
    operand scales and to the scales produced."""
    a = _mat(_bytes(a), "a", (torch.uint8,))
    w = _mat(_bytes(w13), "w13", (torch.uint8,))
    ars, aks = _scale_matrix(a_s, "a_s")
    _mat(w13_s, "w13_s", (torch.float32,))
    M, K = a.shape
    N2, K2 = w.shape
    if K2 != K or N2 % 2:
        raise Dsfp8Error(f"w13 must be [2F, {K}], got {tuple(w.shape)}")
    F = N2 // 2
    if tuple(a_s.shape) != (M, kblocks(K)) or tuple(w13_s.shape) != (kblocks(N2), kblocks(K)):
        raise Dsfp8Error("scale shapes must be a_s [M, ceil(K/128)] and w13_s [2F/128, ceil(K/128)]")
    y, s, h = _glu_outputs(M, F, a.device, out, return_h)
    srs, sks = _scale_strides(s)
    st = _lib.load().dsfp8_gemm_silu_mul_act_quant(
        a.data_ptr(), _ld(a), a_s.data_ptr(), ars, aks, w.data_ptr(), _ld(w), w13_s.data_ptr(), _ld(w13_s),
        M, F, K, y.data_ptr(), _ld(y), s.data_ptr(), srs, sks, h.data_ptr() if h is not None else None, F,
        _fmt(scale_fmt), _stream(a))
    _check("gemm_silu_mul_act_quant", st)
    return (y, s, h) if return_h else (y, s)


def grouped_gemm_silu_mul_act_quant(a, a_s, w13, w13_s, offsets, scale_fmt="fp32", return_h=False, out=None,
                                    workspace=None, rows=None):
    """Grouped form of :func:`gemm_silu_mul_act_quant`: rows
    ``offsets[e]:offsets[e+1]`` of A use expert e's stacked ``w13[e]`` e4m3
    ``[2F, K]`` and ``w13_s[e]`` ``[2F/128, ceil(K/128)]``.

    ``rows`` (int32 CUDA tensor [M_total], optional): product row r reads row
    ``rows[r]`` of ``a`` and ``a_s`` (clamped to ``[0, a.shape[0])``), so the
    per-token quantised input feeds the experts without a gathered copy."""
    a = _mat(_bytes(a), "a", (torch.uint8,))
    w = _mat(_bytes(w13), "w13", (torch.uint8,), dim=3)
    ars, aks = _scale_matrix(a_s, "a_s")
    _mat(w13_s, "w13_s", (torch.float32,), dim=3)
    if not offsets.is_cuda or offsets.dtype != torch.int32 or offsets.dim() != 1 or not offsets.is_contiguous():
        raise Dsfp8Error("offsets must be a contiguous int32 CUDA tensor of length E+1")
    A_rows, K = a.shape
    if rows is not None:
        if not rows.is_cuda or rows.dtype != torch.int32 or rows.dim() != 1 or not rows.is_contiguous():
            raise Dsfp8Error("rows must be a contiguous 1-D int32 CUDA tensor")
        M = rows.numel()
    else:
        M = A_rows
    E, N2, K2 = w.shape
    if K2 != K or N2 % 2 or offsets.numel() != E + 1:
        raise Dsfp8Error("shape mismatch between a, w13 and offsets")
    if not w.is_contiguous() or not w13_s.is_contiguous():
        raise Dsfp8Error("w13 and w13_s need contiguous storage")
    F = N2 // 2
    if tuple(w13_s.shape) != (E, kblocks(N2), kblocks(K)) or tuple(a_s.shape) != (A_rows, kblocks(K)):
        raise Dsfp8Error("scale shapes must be a_s [rows of a, ceil(K/128)] and w13_s [E, 2F/128, ceil(K/128)]")
    lib = _lib.load()
    y, s, h = _glu_outputs(M, F, a.device, out, return_h)
    srs, sks = _scale_strides(s)
    wsb = lib.dsfp8_grouped_gemm_workspace_bytes(E, M, N2, K)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=a.device)
    tail = (w.data_ptr(), K, w13_s.data_ptr(), kblocks(K), offsets.data_ptr(), E, M, F, K, y.data_ptr(), _ld(y),
            s.data_ptr(), srs, sks, h.data_ptr() if h is not None else None, F, _fmt(scale_fmt),
            workspace.data_ptr(), workspace.numel(), _stream(a))
    if rows is None:
        st = lib.dsfp8_grouped_gemm_silu_mul_act_quant(a.data_ptr(), _ld(a), a_s.data_ptr(), ars, aks, *tail)
    else:
        st = lib.dsfp8_grouped_gemm_silu_mul_act_quant_gather(a.data_ptr(), A_rows, _ld(a), a_s.data_ptr(), ars,
                                                              aks, rows.data_ptr(), *tail)
    _check("grouped_gemm_silu_mul_act_quant", st)
    return (y, s, h) if return_h else (y, s)


# ---- routed experts ------------------------------------------------------------------

def act_quant_rows(x, rows, scale_fmt="fp32", out=None):
    """``act_quant(x[rows])`` without forming the gathered copy: e4m3 ``[len(rows), K]``
    and its scales.  ``rows`` is an int32 CUDA tensor; entries are clamped to
    ``[0, x.shape[0])``."""
    x = _mat(x, "x", (torch.bfloat16,))
    if not rows.is_cuda or rows.dtype != torch.int32 or rows.dim() != 1 or not rows.is_contiguous():
        raise Dsfp8Error("rows must be a contiguous int32 CUDA tensor")
    T, K = x.shape
    M = rows.numel()
    y, s = (None, None) if out is None else out
    y = _out(y, (M, K), torch.uint8, x.device, "y")
    s = _scales_out(s, M, kblocks(K), x.device)
    srs, sks = _scale_strides(s)
    st = _lib.load().dsfp8_act_quant_rows(x.data_ptr(), T, _ld(x), rows.data_ptr(), M, K, y.data_ptr(), _ld(y),
                                          s.data_ptr(), srs, sks, _fmt(scale_fmt), _stream(x))
    _check("act_quant_rows", st)
    return y, s


def _int32_mat(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or t.dim() != 2:
        raise Dsfp8Error(f"{name} must be a 2-D int32 CUDA tensor")
    if t.numel() > 0 and t.stride(-1) != 1:
        raise Dsfp8Error(f"{name}: the last dimension needs stride 1")
    return t


def moe_route(indices, experts):
    """Row order of the grouped product for the gate's ``indices [T, k]`` (int32).

    Returns ``(offsets int32 [E+1], row_token int32 [T*k], token_rows int32 [T, k])``:
    rows ``offsets[e]:offsets[e+1]`` are expert e's (token, slot) pairs in row-major
    order, ``row_token[r]`` is the token of row r and ``token_rows[t, j]`` the row
    of pair (t, j) (-1 when its index is outside ``[0, E)``).
    """
    indices = _int32_mat(indices, "indices")
    T, k = indices.shape
    lib = _lib.load()
    dev = indices.device
    offsets = torch.empty(experts + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    token_rows = torch.empty((T, k), dtype=torch.int32, device=dev)
    wsb = lib.dsfp8_moe_route_workspace_bytes(T, k, experts)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=dev)
    st = lib.dsfp8_moe_route(indices.data_ptr(), T, k, _ld(indices), experts, offsets.data_ptr(),
                             row_token.data_ptr(), token_rows.data_ptr(), ws.data_ptr(), ws.numel(), _stream(indices))
    _check("moe_route", st)
    return offsets, row_token, token_rows


def moe_combine(yr, indices, weights, token_rows, out=None):
    """bf16 ``[T, D]``: per token, the bf16 sum over its experts (in increasing
    index) of ``bf16(yr[token_rows[t, j]] * weights[t, j])``, as the pages' loop
    accumulates ``y[idx] += expert(x[idx]) * weights[idx, top]``."""
    yr = _mat(yr, "yr", (torch.bfloat16,))
    indices = _int32_mat(indices, "indices")
    weights = _mat(weights, "weights", (torch.bfloat16,))
    token_rows = _int32_mat(token_rows, "token_rows")
    T, k = indices.shape
    if tuple(weights.shape) != (T, k) or tuple(token_rows.shape) != (T, k) or not token_rows.is_contiguous():
        raise Dsfp8Error("weights and token_rows must be [T, k] (token_rows contiguous) like indices")
    R, D = yr.shape
    out = _out(out, (T, D), torch.bfloat16, yr.device, "out")
    st = _lib.load().dsfp8_moe_combine(yr.data_ptr(), R, _ld(yr), indices.data_ptr(), _ld(indices),
                                       weights.data_ptr(), _ld(weights), token_rows.data_ptr(), T, k, D,
                                       out.data_ptr(), _ld(out), _stream(yr))
    _check("moe_combine", st)
    return out

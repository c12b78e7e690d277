"""GPU check of dsfp8_grouped_gemm_noalloc, the grouped product whose tile
schedule lives in the library's static device scratch instead of a caller
workspace.

Two calls in a row through the C ABI, the second with fewer experts and rows
than the first (so a stale schedule left by the first call would show), each
compared bit for bit with dsfp8_grouped_gemm on the same inputs (the same
kernels, so the outputs must be identical), and the first also against the
per-expert fp64 oracle within the product tolerance.  A third call on the
register-staged path (K not a multiple of 16) and a ue8m0 call follow.
"""

import numpy as np
import pytest
import torch

from block_scaled_fp8_act_amd import _lib
from block_scaled_fp8_act_amd import inputs as I
from oracle import gemm as G
from oracle import quant as Q

from gpu_helpers import check_product, dev_f32, dev_scales, dev_u8, host_bits16

pytestmark = pytest.mark.gpu


def _case(counts, N, K, seed, ue8m0=False):
    counts = np.asarray(counts)
    E = len(counts)
    M = int(counts.sum())
    x = I.activations((M, K), I.MOE, seed)
    a, a_s = Q.act_quant(x, ue8m0=ue8m0)
    qs = [Q.weight_quant(I.weights_f32((N, K), I.MOE, 1000 * seed + e), ue8m0=ue8m0) for e in range(E)]
    b = np.stack([q for q, _ in qs])
    b_s = np.stack([s for _, s in qs])
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return a, a_s, b, b_s, off


def _both(a, a_s, b, b_s, off, fmt):
    """(workspace form, allocation-free form) outputs as bf16 bits."""
    lib = _lib.load()
    E, N, K = b.shape
    M = a.shape[0]
    kbk = (K + 127) // 128
    A, AS, B, BS = dev_u8(a), dev_scales(a_s, "kb"), dev_u8(b), dev_f32(b_s)
    offd = torch.from_numpy(off).cuda()
    srs, sks = AS.stride(0), AS.stride(1)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for form in ("workspace", "noalloc"):
        c = torch.full((M, N), -1.0, dtype=torch.bfloat16, device="cuda")
        if form == "workspace":
            wsb = lib.dsfp8_grouped_gemm_workspace_bytes(E, M, N, K)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            st = lib.dsfp8_grouped_gemm(A.data_ptr(), K, AS.data_ptr(), srs, sks, B.data_ptr(), K, BS.data_ptr(), kbk,
                                        offd.data_ptr(), E, M, N, K, c.data_ptr(), N, fmt, ws.data_ptr(), wsb, stream)
        else:
            st = lib.dsfp8_grouped_gemm_noalloc(A.data_ptr(), K, AS.data_ptr(), srs, sks, B.data_ptr(), K,
                                                BS.data_ptr(), kbk, offd.data_ptr(), E, M, N, K, c.data_ptr(), N, fmt,
                                                stream)
        assert st == 0, (form, lib.dsfp8_status_string(st))
        torch.cuda.synchronize()
        outs.append(host_bits16(c))
    return outs


def _oracle_check(C, a, a_s, b, b_s, off):
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        A_hat = G.dequant_act(a[lo:hi], a_s[lo:hi])
        W_hat = G.dequant_weight(b[e], b_s[e])
        check_product(C[lo:hi], A_hat @ W_hat.T, A_hat, W_hat, f"expert {e}")


def test_noalloc_two_calls_second_smaller():
    # first call: 12 experts, all three tile heights, empty experts, 1770 rows
    first = [5, 0, 17, 1, 300, 9, 64, 65, 128, 257, 700, 224]
    a, a_s, b, b_s, off = _case(first, 384, 512, 3)
    ws, na = _both(a, a_s, b, b_s, off, 0)
    assert np.array_equal(ws, na), "first call: allocation-free form differs from the workspace form"
    _oracle_check(na, a, a_s, b, b_s, off)
    # second call, smaller: 4 experts, 200 rows; the first call's schedule
    # (more experts, more tiles) is still in the scratch
    second = [3, 0, 130, 67]
    a, a_s, b, b_s, off = _case(second, 256, 256, 4)
    ws, na = _both(a, a_s, b, b_s, off, 0)
    assert np.array_equal(ws, na), "second call: allocation-free form differs from the workspace form"
    _oracle_check(na, a, a_s, b, b_s, off)


def test_noalloc_register_path_and_ue8m0():
    # K = 1000: the register-staged path with one tile class
    a, a_s, b, b_s, off = _case([40, 0, 129, 7], 140, 1000, 5)
    ws, na = _both(a, a_s, b, b_s, off, 0)
    assert np.array_equal(ws, na)
    _oracle_check(na, a, a_s, b, b_s, off)
    a, a_s, b, b_s, off = _case([70, 3, 300, 0, 129], 256, 512, 6, ue8m0=True)
    ws, na = _both(a, a_s, b, b_s, off, 1)
    assert np.array_equal(ws, na)
    _oracle_check(na, a, a_s, b, b_s, off)

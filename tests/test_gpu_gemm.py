"""GPU parity of the block-scaled FP8 product (Admin Guide 8.5.3 / 6.3).

Against the fp64 oracle of the same quantised operands with the tolerance of
gpu_helpers; bit-exact where the exact result is representable (integer
operands with power-of-two scales).  Shapes: every workload's products (the
large prefill products on sampled outputs), tails in M, N and K, the
unaligned load widths, strided operands, K = 0 and single elements.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import _lib
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q

from gpu_helpers import (bf16_to_f64, check_gemm_full, check_product, dev_bf16, dev_f32, dev_scales, dev_u8,
                         host_bits16, host_u8)

pytestmark = pytest.mark.gpu


def operands(M, N, K, cid, ue8m0=False, outliers=0.0):
    x = I.activations((M, K), cid, 0, outlier_frac=outliers)
    a, a_s = Q.act_quant(x, ue8m0=ue8m0)
    b, b_s = Q.weight_quant(I.weights_f32((N, K), cid, 1), ue8m0=ue8m0)
    return a, a_s, b, b_s


def run(a, a_s, b, b_s, layout="kb", scale_fmt="fp32"):
    c = ds.gemm(dev_u8(a), dev_scales(a_s, layout), dev_u8(b), dev_f32(b_s), scale_fmt=scale_fmt)
    torch.cuda.synchronize()
    return host_bits16(c)


@pytest.mark.parametrize("layout", ["kb", "row"])
def test_tiny(layout):
    a, a_s, b, b_s = operands(16, 256, 512, I.TINY)
    check_gemm_full(run(a, a_s, b, b_s, layout), a, a_s, b, b_s, "tiny")


@pytest.mark.parametrize("layout", ["kb", "row"])
def test_decode_qa(layout):
    a, a_s, b, b_s = operands(32, 1536, 7168, I.DECODE_QA, outliers=0.01)
    check_gemm_full(run(a, a_s, b, b_s, layout), a, a_s, b, b_s, "decode_qa")


@pytest.mark.parametrize("layout", ["kb", "row"])
def test_ragged_ue8m0(layout):
    a, a_s, b, b_s = operands(333, 2500, 1000, I.RAGGED, ue8m0=True)
    check_gemm_full(run(a, a_s, b, b_s, layout), a, a_s, b, b_s, "ragged")


@pytest.mark.parametrize("layout", ["kb", "row"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (1, 256, 128), (129, 130, 300), (200, 64, 200), (65, 300, 100),
                                   (17, 129, 99), (128, 128, 256), (300, 520, 1544), (2, 2000, 16),
                                   (257, 384, 640), (100, 1000, 4096),
                                   # K % 16 == 0 with a partial last K-block (direct-to-LDS loads)
                                   (64, 300, 400), (257, 384, 656), (300, 520, 1552)])
def test_edge_shapes(M, N, K, layout):
    a, a_s, b, b_s = operands(M, N, K, I.TINY)
    check_gemm_full(run(a, a_s, b, b_s, layout), a, a_s, b, b_s, f"{M}x{N}x{K}")


@pytest.mark.parametrize("layout", ["kb", "row"])
def test_large_tile_path_with_tails(layout):
    # Enough 256x256 tiles to select the large-tile pipeline, with partial
    # tiles in M (1300 = 5*256 + 20) and N (11000 = 42*256 + 248); full check.
    a, a_s, b, b_s = operands(1300, 11000, 640, I.TINY)
    check_gemm_full(run(a, a_s, b, b_s, layout), a, a_s, b, b_s, "1300x11000x640")


def test_large_tile_path_partial_k_block():
    # the 256 x 256 tiles with K = 5 * 128 + 80: the last K-block's chunks past K read as zero
    a, a_s, b, b_s = operands(1300, 11000, 720, I.TINY)
    check_gemm_full(run(a, a_s, b, b_s), a, a_s, b, b_s, "1300x11000x720")


def test_layouts_bit_identical():
    # The storage order of the activation scales changes only how they are
    # fetched, never the arithmetic.
    a, a_s, b, b_s = operands(300, 520, 1536, I.TINY)
    assert np.array_equal(run(a, a_s, b, b_s, "kb"), run(a, a_s, b, b_s, "row"))


def test_k_zero_writes_zeros():
    a = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    a_s = torch.empty((5, 0), dtype=torch.float32, device="cuda")
    b = torch.empty((7, 0), dtype=torch.uint8, device="cuda")
    b_s = torch.empty((1, 0), dtype=torch.float32, device="cuda")
    c = ds.gemm(a, a_s, b, b_s)
    torch.cuda.synchronize()
    assert c.shape == (5, 7) and torch.all(c == 0)


@pytest.mark.parametrize("scale_fmt", ["fp32", "ue8m0"])
def test_integer_operands_bit_exact(scale_fmt):
    # The scales are powers of two, so the ue8m0 form (scales applied inside
    # the matrix instruction, per row and 32-byte K slice) must agree too.
    g = np.random.default_rng(11)
    M, N, K = 200, 300, 1024
    ai = g.integers(-4, 5, (M, K))
    bi = g.integers(-4, 5, (N, K))
    a = F.e4m3_encode(ai.astype(np.float32))
    b = F.e4m3_encode(bi.astype(np.float32))
    a_s = np.ldexp(np.ones((M, 8), np.float32), g.integers(-3, 1, (M, 8))).astype(np.float32)
    b_s = np.ldexp(np.ones((3, 8), np.float32), g.integers(-3, 1, (3, 8))).astype(np.float32)
    C = run(a, a_s, b, b_s, scale_fmt=scale_fmt)
    ref = G.gemm(a, a_s, b, b_s)
    # Every partial sum is a multiple of 2^-6 of magnitude at most
    # 8 * 128 * 16 = 2^14, hence exact in fp32 in any order; the only rounding
    # left is the final one to bf16.
    assert np.array_equal(C, F.f32_to_bf16(ref))


@pytest.mark.parametrize("M,N,K", [
    (1300, 11000, 640),   # 256 x 256 tiles
    (1300, 11000, 720),   # 256 x 256 tiles, partial last K-block
    (257, 384, 656),      # 128 x 128 tiles, partial last K-block
    (100, 1000, 4096),    # split K
    (333, 2500, 1000),    # K % 16 != 0: register-staged pipeline (general fp32 path)
])
def test_ue8m0_scaled_product(M, N, K):
    # power-of-two activation and weight scales, declared as such: checked
    # against the oracle, and against the same product with fp32-format scales
    a, a_s, b, b_s = operands(M, N, K, I.RAGGED, ue8m0=True)
    C = run(a, a_s, b, b_s, scale_fmt="ue8m0")
    check_gemm_full(C, a, a_s, b, b_s, f"ue8m0 {M}x{N}x{K}")
    C32 = run(a, a_s, b, b_s)
    A_hat = G.dequant_act(a, a_s)
    W_hat = G.dequant_weight(b, b_s)
    check_product(C, bf16_to_f64(C32), A_hat, W_hat, f"ue8m0 vs fp32 form {M}x{N}x{K}")


def test_one_hot_weight():
    a, a_s, _, _ = operands(64, 4, 512, I.TINY)
    N, K = 384, 512
    b = np.zeros((N, K), np.uint8)
    cols = np.random.default_rng(12).integers(0, K, N)
    b[np.arange(N), cols] = 0x38
    b_s = np.full((3, 4), 0.5, np.float32)
    C = run(a, a_s, b, b_s)
    ref = G.dequant_act(a, a_s)[:, cols] * 0.5
    # one non-zero product per output: rounded once to fp32 (the fma with the
    # scale), then to bf16
    assert np.array_equal(C, F.f32_to_bf16(ref.astype(np.float32)))


def test_strided_operands():
    a, a_s, b, b_s = operands(200, 200, 384, I.TINY)
    A = np.zeros((200, 512), np.uint8); A[:, :384] = a
    B = np.zeros((200, 400), np.uint8); B[:, 16:400] = b
    S = np.zeros((200, 5), np.float32); S[:, 1:4] = a_s           # row stride 5
    c = ds.gemm(dev_u8(A)[:, :384], dev_f32(S)[:, 1:4], dev_u8(B)[:, 16:400], dev_f32(b_s))
    torch.cuda.synchronize()
    check_gemm_full(host_bits16(c), a, a_s, b, b_s, "strided")


def _sampled_product(M, N, K, seed, row_pick, nblocks, fmt="fp32"):
    """GEMM at full size with device-drawn inputs; compare sampled outputs.

    x and W are drawn on the device; the GPU quantises them; the oracle
    quantises the sampled rows / weight block-rows from the same source values,
    must agree bit-exactly with the GPU's bytes, and then supplies the
    reference product for those rows and columns.
    """
    ue = fmt == "ue8m0"
    xf = I.device_normal((M, K), seed=seed, std=1.0, device="cuda", dtype=torch.bfloat16)
    wf = I.device_normal((N, K), seed=seed + 1, std=0.02, device="cuda")
    a, a_s = ds.act_quant(xf, fmt)
    b, b_s = ds.weight_quant(wf, fmt)
    c = ds.gemm(a, a_s, b, b_s, scale_fmt=fmt)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(seed).choice(M, row_pick, replace=False))
    rows[-1] = M - 1
    kb = (N + 127) // 128
    blks = sorted({0, kb - 1, *np.random.default_rng(seed + 2).choice(kb, nblocks, replace=False).tolist()})
    xr = xf[torch.from_numpy(rows).cuda()].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ar, asr = Q.act_quant(xr, ue8m0=ue)
    assert np.array_equal(host_u8(a[torch.from_numpy(rows).cuda()]), ar)
    A_hat = G.dequant_act(ar, asr)
    for bi in blks:
        n0, n1 = bi * 128, min(N, bi * 128 + 128)
        wr = wf[n0:n1].cpu().numpy()
        br, bsr = Q.weight_quant(wr, ue8m0=ue)
        assert np.array_equal(host_u8(b[n0:n1]), br)
        W_hat = G.dequant_weight(br, bsr)
        Cg = host_bits16(c[torch.from_numpy(rows).cuda(), n0:n1])
        check_product(Cg, A_hat @ W_hat.T, A_hat, W_hat, f"{M}x{N}x{K} block {bi}")


@pytest.mark.parametrize("M,N,K,fmt", [(1, 4608, 7168, "fp32"), (16, 7168, 2048, "fp32"), (8, 1536, 7168, "ue8m0"),
                                       (5, 300, 1040, "fp32"), (16, 129, 16, "ue8m0"),
                                       (32, 7168, 2048, "fp32"), (17, 2100, 1040, "ue8m0"), (24, 4100, 528, "fp32"),
                                       (17, 1000, 1040, "fp32"), (32, 256, 2048, "ue8m0"), (24, 16384, 4096, "fp32")])
def test_decode_rows(M, N, K, fmt):
    # at most 16 rows with K % 16 == 0 (and 17 to 32 rows with two activation
    # fragments for 2048 < N <= 8192, for N and K at most 2048, and for
    # 16384 <= N < 32768 with K > 2048): the kernel that splits K across the
    # waves of one workgroup per 16 columns (ragged N and K included)
    a, a_s, b, b_s = operands(M, N, K, I.DECODE_QA, ue8m0=(fmt == "ue8m0"), outliers=0.01)
    for layout in ("kb", "row"):
        check_gemm_full(run(a, a_s, b, b_s, layout, scale_fmt=fmt), a, a_s, b, b_s, f"{M}x{N}x{K} {fmt} {layout}")


@pytest.mark.parametrize("M,N,K,fmt", [
    (32, 1024, 1024, "fp32"),     # staged in LDS, 32x64 tiles, one workgroup per tile
    (32, 1024, 4096, "ue8m0"),    # the same, K split 4 ways
    (20, 1000, 1000, "fp32"),     # 32x64 tiles, rows only 8-byte aligned (4-byte loads to LDS)
    (30, 1000, 3000, "ue8m0"),    # the same, K split 3 ways
    (24, 2048, 7168, "fp32"),     # 32x32 tiles, two K-blocks per wave, K split 4 ways
    (32, 600, 7000, "fp32"),      # the same with 8-byte aligned rows
    (100, 1000, 4096, "fp32"),    # 64x32 tiles, K split 4 ways
    (70, 900, 2008, "ue8m0"),     # the same with 8-byte aligned rows, K split 2 ways
    (333, 2500, 1000, "fp32"),    # 64x64 tiles, 8-byte aligned rows
    (64, 4096, 7168, "fp32"),     # operands staged in registers, 64x32 tiles
    (48, 2048, 7000, "ue8m0"),    # the same with 8-byte aligned rows
    (32, 2048, 16384, "fp32"),    # registers, 32x64 tiles, K split 8 ways
    (32, 1024, 16384, "ue8m0"),   # registers, 32x32 tiles
])
def test_one_launch_forms(M, N, K, fmt):
    """Products with few output tiles run in one launch of the small-product
    kernel, in the form and tile shape their size selects (comments above:
    where the operands are staged, the tile, the load width for rows that are
    only 8-byte aligned, the K split): each against the oracle in full."""
    a, a_s, b, b_s = operands(M, N, K, I.DECODE_QA, ue8m0=(fmt == "ue8m0"), outliers=0.01)
    check_gemm_full(run(a, a_s, b, b_s, "kb", scale_fmt=fmt), a, a_s, b, b_s, f"{M}x{N}x{K} {fmt}")


def test_dense_ffn_up_sampled():
    _sampled_product(4096, 18432, 7168, 50, 256, 4)


def test_dense_ffn_up_sampled_ue8m0():
    # power-of-two scales applied by the MFMA on the 256 x 256 tiles
    _sampled_product(4096, 18432, 7168, 55, 256, 4, "ue8m0")


def test_dense_ffn_down_sampled_ue8m0():
    _sampled_product(4096, 7168, 18432, 75, 128, 3, "ue8m0")


def test_dense_ffn_up_stacked_sampled():
    _sampled_product(4096, 36864, 7168, 60, 128, 3)


def test_dense_ffn_down_sampled():
    _sampled_product(4096, 7168, 18432, 70, 128, 3)


@pytest.mark.parametrize("shapes", [
    [(32, 1536, 7168), (32, 1536, 7168), (333, 2500, 1000), (100, 1000, 4096), (32, 1536, 7168)],
    [(64, 300, 400), (257, 384, 640), (17, 300, 1536), (64, 300, 400)],
])
def test_split_products_reuse_one_workspace(shapes):
    """Products that split K over workgroups keep per-tile arrival counters at
    the start of the workspace and clear them when they finish: one workspace,
    zero-filled once, serves a sequence of calls of different shapes, and a
    repeated call gives the same bits (the last workgroup to arrive adds the
    splits in split order, whichever it is).  The output is filled with a
    sentinel before each call, so a call that found a counter not cleared
    (and so never stored) would show."""
    lib = _lib.load()
    need = max(lib.dsfp8_gemm_workspace_bytes(M, N, K) for M, N, K in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    first = {}
    for i, (M, N, K) in enumerate(shapes):
        a, a_s, b, b_s = operands(M, N, K, I.TINY)
        A, AS, B, BS = dev_u8(a), dev_scales(a_s, "kb"), dev_u8(b), dev_f32(b_s)
        c = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        st = lib.dsfp8_gemm(A.data_ptr(), K, AS.data_ptr(), AS.stride(0), AS.stride(1), B.data_ptr(), K,
                            BS.data_ptr(), BS.stride(0), c.data_ptr(), N, M, N, K, 0, ws.data_ptr(), need, stream)
        assert st == 0
        torch.cuda.synchronize()
        got = host_bits16(c)
        check_gemm_full(got, a, a_s, b, b_s, f"call {i}: {M}x{N}x{K}")
        if (M, N, K) in first:
            assert np.array_equal(got, first[(M, N, K)]), f"call {i}: repeated {M}x{N}x{K} differs"
        first.setdefault((M, N, K), got)

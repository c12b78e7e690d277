"""The C ABI on the host (no GPU, no kernel launch).

libdsfp8.so must load without a GPU and export every function that
include/dsfp8.h declares.  Argument validation runs before any HIP call, so
each error status can be provoked here with fake (never dereferenced)
pointers; only calls that are rejected are made.
"""

import ctypes
import os
import re

import pytest

from block_scaled_fp8_act_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsfp8.h")

OK, NULL, SHAPE, LD, ALIGN, FMT, WS, LAUNCH, DTYPE, UNSUP, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10
P = 0x10000          # a fake, 256-byte aligned device address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsfp8_status|size_t|int|const char\*)\s+(dsfp8_\w+)\(", text, re.M)))


def header_constant(name):
    m = re.search(rf"{name}\s*=?\s*(-?\d+)", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_scaled_fp8_act_amd import build
        build.build()
    return _lib.load()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_abi_version_and_strings(lib):
    assert lib.dsfp8_abi_version() == header_constant("#define DSFP8_ABI_VERSION")
    for st in (OK, NULL, SHAPE, LD, ALIGN, FMT, WS, LAUNCH, DTYPE, UNSUP, SCRATCH):
        s = lib.dsfp8_status_string(st)
        assert s and s != b"unknown status"
    assert lib.dsfp8_status_string(12345) == b"unknown status"


def test_status_codes_match_header():
    for name, v in [("DSFP8_ERR_NULL", NULL), ("DSFP8_ERR_SHAPE", SHAPE), ("DSFP8_ERR_LD", LD),
                    ("DSFP8_ERR_ALIGN", ALIGN), ("DSFP8_ERR_SCALE_FMT", FMT), ("DSFP8_ERR_WORKSPACE", WS),
                    ("DSFP8_ERR_LAUNCH", LAUNCH), ("DSFP8_ERR_DTYPE", DTYPE),
                    ("DSFP8_ERR_UNSUPPORTED", UNSUP), ("DSFP8_ERR_SCRATCH", SCRATCH)]:
        assert header_constant(name) == v


def test_act_quant_validation(lib):
    f = lib.dsfp8_act_quant
    # x, M, K, ldx, y, ldy, s, s_row_stride, s_kb_stride, fmt, stream
    assert f(P, -1, 128, 128, P, 128, P, 1, 1, 0, None) == SHAPE
    assert f(P, 4, 1 << 31, 1 << 31, P, 1 << 31, P, 1 << 24, 1, 0, None) == SHAPE
    assert f(P, 4, 128, 128, P, 128, P, 1, 1, 2, None) == FMT
    assert f(None, 4, 128, 128, P, 128, P, 1, 1, 0, None) == NULL
    assert f(P, 4, 128, 128, None, 128, P, 1, 1, 0, None) == NULL
    assert f(P, 4, 128, 128, P, 128, None, 1, 1, 0, None) == NULL
    assert f(P, 4, 128, 100, P, 128, P, 1, 1, 0, None) == LD
    assert f(P, 4, 128, 128, P, 127, P, 1, 1, 0, None) == LD
    assert f(P, 4, 256, 256, P, 256, P, 1, 1, 0, None) == LD          # 2 K-blocks overlap
    assert f(P, 4, 256, 256, P, 256, P, 2, 2, 0, None) == LD          # neither layout
    assert f(P, 4, 256, 256, P, 256, P, 1, 3, 0, None) == LD          # K-block-major needs ks >= M
    assert f(P + 1, 4, 128, 128, P, 128, P, 1, 1, 0, None) == ALIGN    # bf16 needs 2-byte alignment
    assert f(P, 4, 128, 128, P, 128, P + 2, 1, 1, 0, None) == ALIGN    # fp32 needs 4
    # empty problems are valid and launch nothing
    assert f(None, 0, 128, 128, None, 128, None, 1, 1, 0, None) == OK
    assert f(None, 5, 0, 0, None, 0, None, 1, 1, 0, None) == OK


def test_silu_and_weight_validation(lib):
    f = lib.dsfp8_silu_mul_act_quant
    # g, ldg, u, ldu, M, I, y, ldy, s, srs, sks, h, ldh, fmt, stream
    assert f(P, 256, P, 256, 4, 256, P, 256, P, 2, 1, None, 0, 9, None) == FMT
    assert f(P, 256, None, 256, 4, 256, P, 256, P, 2, 1, None, 0, 0, None) == NULL
    assert f(P, 256, P, 256, 4, 256, P, 256, P, 2, 1, P, 100, 0, None) == LD
    assert f(P, 256, P, 256, 4, 256, P, 256, P, 1, 2, None, 0, 0, None) == LD
    assert f(None, 256, None, 256, 0, 256, None, 256, None, 2, 1, None, 0, 0, None) == OK
    q = lib.dsfp8_weight_quant
    assert q(P, 7, 128, 128, 128, P, 128, P, 1, 0, None) == DTYPE
    assert q(P, 0, 128, 128, 128, P, 128, P, 1, 3, None) == FMT
    assert q(P + 2, 0, 128, 128, 128, P, 128, P, 1, 0, None) == ALIGN  # fp32 input
    assert q(P, 0, 300, 128, 128, P, 128, P, 0, 0, None) == LD         # scale grid is [3, 1]
    d = lib.dsfp8_weight_dequant
    assert d(P, -5, 128, 128, P, 1, P, 128, None) == SHAPE
    assert d(None, 5, 128, 128, P, 1, P, 128, None) == NULL
    assert d(P, 5, 128, 128, P, 1, P + 1, 128, None) == ALIGN
    assert d(P, 5, 128, 64, P, 1, P, 128, None) == LD


def test_gemm_validation(lib):
    def g(*args, fmt=0):
        # A, lda, a_s, as_rs, as_ks, B, ldb, b_s, ldbs, C, ldc, M, N, K, [scale_fmt], ws, wsb, stream
        return lib.dsfp8_gemm(*args[:14], fmt, *args[14:])

    assert g(P, 256, P, 2, 1, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None, fmt=2) == FMT
    assert g(P, 256, P, 2, 1, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None, fmt=-1) == FMT
    assert g(P, 256, P, 2, 1, P, 256, P, 2, P, 64, -8, 64, 256, None, 0, None) == SHAPE
    assert g(None, 256, P, 2, 1, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None) == NULL
    assert g(P, 255, P, 2, 1, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None) == LD
    assert g(P, 256, P, 1, 1, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None) == LD
    assert g(P, 256, P, 1, 7, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None) == LD   # ks < M
    assert g(P, 256, P, 2, 1, P, 256, P, 1, P, 64, 8, 64, 256, None, 0, None) == LD   # b_s row too short
    assert g(P, 256, P, 2, 1, P, 256, P, 2, P, 63, 8, 64, 256, None, 0, None) == LD
    assert g(P, 256, P + 1, 2, 1, P, 256, P, 2, P, 64, 8, 64, 256, None, 0, None) == ALIGN
    assert g(P, 256, P, 2, 1, P, 256, P, 2, P + 1, 64, 8, 64, 256, None, 0, None) == ALIGN
    assert lib.dsfp8_gemm_workspace_bytes(4096, 18432, 7168) == 0
    # a decode-shaped product splits K and needs a workspace: 256-byte aligned
    # arrival counters, then fp32 partial sums of the output
    need = lib.dsfp8_gemm_workspace_bytes(32, 1536, 7168)
    assert need >= 256 + 2 * 32 * 1536 * 4 and need % 4 == 0
    assert g(P, 7168, P, 1, 32, P, 7168, P, 56, P, 1536, 32, 1536, 7168, None, 0, None) == WS
    assert g(P, 7168, P, 1, 32, P, 7168, P, 56, P, 1536, 32, 1536, 7168, None, need, None) == NULL
    assert g(P, 7168, P, 1, 32, P, 7168, P, 56, P, 1536, 32, 1536, 7168, P + 4, need, None) == ALIGN


def test_grouped_validation(lib):
    g = lib.dsfp8_grouped_gemm
    names = ["A", "lda", "a_s", "as_rs", "as_ks", "B", "ldb", "b_s", "ldbs", "offsets", "E", "M", "N", "K", "C",
             "ldc", "fmt", "ws", "wsb", "stream"]
    args = [P, 256, P, 1, 100, P, 256, P, 2, P, 4, 100, 64, 256, P, 64, 0, P, 1 << 20, None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return g(*a)

    assert call(fmt=3) == FMT
    assert call(E=0) == SHAPE
    assert call(E=70000) == SHAPE
    assert call(offsets=None) == NULL
    assert call(offsets=P + 2) == ALIGN
    assert call(ldb=100) == LD
    assert call(ldbs=1) == LD
    assert call(as_ks=99) == LD
    need = lib.dsfp8_grouped_gemm_workspace_bytes(4, 100, 64, 256)
    assert need >= 5 * 4
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == NULL
    assert lib.dsfp8_grouped_gemm_workspace_bytes(0, 1, 1, 1) == 0


def test_grouped_noalloc_validation(lib):
    g = lib.dsfp8_grouped_gemm_noalloc
    names = ["A", "lda", "a_s", "as_rs", "as_ks", "B", "ldb", "b_s", "ldbs", "offsets", "E", "M", "N", "K", "C",
             "ldc", "fmt", "stream"]
    args = [P, 256, P, 1, 100, P, 256, P, 2, P, 4, 100, 64, 256, P, 64, 0, None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return g(*a)

    limit = header_constant("#define DSFP8_NOALLOC_MAX_EXPERTS")
    assert limit == 4096
    assert call(fmt=3) == FMT
    assert call(E=0) == SHAPE
    assert call(E=70000) == SHAPE
    assert call(E=limit + 1) == SCRATCH
    assert call(offsets=None) == NULL
    assert call(offsets=P + 2) == ALIGN
    assert call(ldb=100) == LD
    assert call(ldbs=1) == LD
    assert call(as_ks=99) == LD
    assert call(A=None) == NULL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU or PyTorch fallback"):
        _lib.load()


def test_routed_expert_validation(lib):
    # dsfp8_moe_route(indices, T, k, ldi, E, offsets, row_token, token_rows, ws, wsb, stream)
    r = lib.dsfp8_moe_route
    need = lib.dsfp8_moe_route_workspace_bytes(4096, 8, 256)
    assert need == 64 * 256 * 4  # 32768 pairs in 64 chunks of 512
    assert lib.dsfp8_moe_route_workspace_bytes(4096, 17, 256) == 0
    assert lib.dsfp8_moe_route_workspace_bytes(4096, 8, 4097) == 0
    assert r(P, 4096, 0, 8, 256, P, P, P, P, need, None) == SHAPE
    assert r(P, 4096, 17, 17, 256, P, P, P, P, need, None) == SHAPE
    assert r(P, 4096, 8, 8, 0, P, P, P, P, need, None) == SHAPE
    assert r(P, 4096, 8, 8, 4097, P, P, P, P, need, None) == SHAPE
    assert r(P, 4096, 8, 7, 256, P, P, P, P, need, None) == LD
    assert r(None, 4096, 8, 8, 256, P, P, P, P, need, None) == NULL
    assert r(P, 4096, 8, 8, 256, None, P, P, P, need, None) == NULL
    assert r(P, 4096, 8, 8, 256, P, P, P + 2, P, need, None) == ALIGN
    assert r(P, 4096, 8, 8, 256, P, P, P, P, need - 1, None) == WS
    assert r(P, 4096, 8, 8, 256, P, P, P, None, need, None) == NULL
    # dsfp8_moe_combine(yr, R, ldy, indices, ldi, weights, ldw, token_rows, T, k, D, out, ldo, stream)
    c = lib.dsfp8_moe_combine
    assert c(P, 64, 256, P, 8, P, 8, P, 8, 0, 256, P, 256, None) == SHAPE
    assert c(P, 64, 256, P, 8, P, 8, P, 8, 17, 256, P, 256, None) == SHAPE
    assert c(P, 64, 255, P, 8, P, 8, P, 8, 8, 256, P, 256, None) == LD
    assert c(P, 64, 256, P, 8, P, 7, P, 8, 8, 256, P, 256, None) == LD
    assert c(P, 64, 256, P, 8, P, 8, P, 8, 8, 256, P + 1, 256, None) == ALIGN
    assert c(P, 64, 256, None, 8, P, 8, P, 8, 8, 256, P, 256, None) == NULL
    # dsfp8_act_quant_rows(x, x_rows, ldx, rows, M, K, y, ldy, s, srs, sks, fmt, stream)
    q = lib.dsfp8_act_quant_rows
    assert q(P, 0, 256, P, 4, 256, P, 256, P, 1, 4, 0, None) == SHAPE
    assert q(P, 8, 256, None, 4, 256, P, 256, P, 1, 4, 0, None) == NULL
    assert q(P, 8, 256, P + 2, 4, 256, P, 256, P, 1, 4, 0, None) == ALIGN
    assert q(P, 8, 256, P, 4, 256, P, 256, P, 1, 4, 7, None) == FMT
    assert q(P, 8, 255, P, 4, 256, P, 256, P, 1, 4, 0, None) == LD


GLU_NAMES = ["A", "lda", "a_s", "as_rs", "as_ks", "W", "ldw", "w_s", "ldws", "M", "F", "K", "y", "ldy", "s", "srs",
             "sks", "h", "ldh", "fmt", "stream"]
GLU_ARGS = [P, 256, P, 1, 8, P, 256, P, 2, 8, 256, 256, P, 256, P, 1, 8, None, 0, 0, None]


def glu_call(lib, **kw):
    a = list(GLU_ARGS)
    for k, v in kw.items():
        a[GLU_NAMES.index(k)] = v
    return lib.dsfp8_gemm_silu_mul_act_quant(*a)


def test_gated_product_validation(lib):
    assert glu_call(lib, fmt=3) == FMT
    assert glu_call(lib, M=-1) == SHAPE
    assert glu_call(lib, F=1 << 31) == SHAPE
    assert glu_call(lib, A=None) == NULL
    assert glu_call(lib, W=None) == NULL
    assert glu_call(lib, y=None) == NULL
    assert glu_call(lib, ldw=255) == LD
    assert glu_call(lib, ldws=1) == LD            # the stacked scale grid has 2 columns
    assert glu_call(lib, ldy=200) == LD
    assert glu_call(lib, h=P, ldh=100) == LD
    assert glu_call(lib, s=P + 2) == ALIGN
    # layouts outside the fused kernel's pipeline: reported, nothing launched
    assert glu_call(lib, F=200, ldy=200) == UNSUP                  # F not a multiple of 128
    assert glu_call(lib, K=250, lda=256, ldw=256) == UNSUP         # K % 16 != 0
    assert glu_call(lib, lda=264) == UNSUP                         # lda % 16 != 0
    assert glu_call(lib, A=P + 8) == UNSUP                         # A not 16-byte aligned
    assert glu_call(lib, y=P + 4) == UNSUP                         # y rows written 8 bytes at a time
    assert glu_call(lib, ldy=260) == UNSUP
    assert glu_call(lib, h=P + 8, ldh=256) == UNSUP
    # one buffer descriptor spans w1 row n0 to w3 row F + n0 + 127: more than 2^31 bytes is not supported
    assert glu_call(lib, F=1 << 20, ldw=4096, K=4096, lda=4096, ldws=32, ldy=1 << 20, sks=8) == UNSUP
    # empty problems launch nothing
    assert glu_call(lib, M=0) == OK
    assert glu_call(lib, F=0, ldy=0) == OK


def test_grouped_gated_product_validation(lib):
    g = lib.dsfp8_grouped_gemm_silu_mul_act_quant
    names = ["A", "lda", "a_s", "as_rs", "as_ks", "W", "ldw", "w_s", "ldws", "offsets", "E", "M", "F", "K", "y",
             "ldy", "s", "srs", "sks", "h", "ldh", "fmt", "ws", "wsb", "stream"]
    args = [P, 256, P, 1, 100, P, 256, P, 2, P, 4, 100, 256, 256, P, 256, P, 1, 100, None, 0, 0, P, 1 << 20, None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return g(*a)

    assert call(E=0) == SHAPE
    assert call(E=65537) == SHAPE
    assert call(offsets=None) == NULL
    assert call(offsets=P + 2) == ALIGN
    assert call(fmt=7) == FMT
    assert call(wsb=0) == WS
    assert call(ws=None) == NULL
    assert call(F=200, ldy=200) == UNSUP
    assert call(M=0) == OK


def test_grouped_gated_gather_validation(lib):
    g = lib.dsfp8_grouped_gemm_silu_mul_act_quant_gather
    names = ["A", "a_rows", "lda", "a_s", "as_rs", "as_ks", "rows", "W", "ldw", "w_s", "ldws", "offsets", "E", "M",
             "F", "K", "y", "ldy", "s", "srs", "sks", "h", "ldh", "fmt", "ws", "wsb", "stream"]
    args = [P, 40, 256, P, 1, 40, P, P, 256, P, 2, P, 4, 100, 256, 256, P, 256, P, 1, 100, None, 0, 0, P, 1 << 20,
            None]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return g(*a)

    assert call(rows=None) == NULL
    assert call(rows=P + 2) == ALIGN
    assert call(a_rows=0) == SHAPE
    assert call(a_rows=-1) == SHAPE
    assert call(lda=100) == LD                # lda below K
    assert call(E=0) == SHAPE
    assert call(offsets=None) == NULL
    assert call(fmt=7) == FMT
    assert call(wsb=0) == WS
    assert call(F=200, ldy=200) == UNSUP
    # one descriptor spans all of A: a_rows * lda + K must stay below 2^31
    assert call(a_rows=(1 << 31) // 256, as_ks=(1 << 31) // 256, lda=256) == UNSUP
    # ... also where a_rows * lda would overflow 64 bits
    assert call(a_rows=1 << 25, as_ks=1 << 25, lda=1 << 39) == UNSUP
    # no rows: nothing to do, nothing launched (the pointers are never touched)
    assert call(M=0) == OK
    assert call(M=0, rows=None) == OK

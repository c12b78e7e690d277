"""GPU parity of the gated up-projection (product + SiLU gate + act_quant in one
kernel), dense and grouped.

The kernel computes h1 = x w1^T and h3 = x w3^T as the block-scaled product
does ("DeepSeek-V3 Administrator & Developer Guide" 8.5.3 / 6.3), rounds
them to bf16, forms h = bf16(SiLU(h1) * h3) (1.2, the feed-forward
w2(SiLU(w1 x) * w3 x)) and quantises h per 128 columns (8.5.1).  Checks:

* integer operands with power-of-two scales, where every product is exact:
  h1 and h3 equal the oracle's bf16-rounded products bit for bit, so h is
  within one bf16 unit of the oracle's correctly rounded gate (rarely
  different) and (y, s) equal the oracle's act_quant on every block whose h
  agrees;
* random operands: h and the dequantised y * s against the oracle within an
  element-wise bound derived from the roundings involved (below);
* the fused call against the unfused GPU composition (product, then the
  standalone gate-and-quantise kernel), which performs the same arithmetic in
  the same order and must agree bit for bit;
* the dense feed-forward and routed-expert sizes, on sampled rows and blocks.

Element-wise bound for random operands.  With C the exact product and C32
the kernel's fp32 accumulation, |C32 - C| <= 2e-5 * (|A| |W|^T) (at most 56
fp32 additions of rescaled K-block sums plus the MFMA's own fp32 sums of 128
exact products); both sides round to bf16, so the kernel's h1 (and h3)
differs from the oracle's by at most d = ulp_bf16(|C|) + that amount.  SiLU
has slope at most 1.1, so |dh| <= 1.1 |h3| d1 + |SiLU(h1)| d3 + d1 d3 plus
the two bf16 roundings of h (2^-8 |h| together) and the hardware exp and
reciprocal (far below).  The e4m3 codes then satisfy
|y*s - h_gpu| <= 2^-4 |h_gpu| + 2^-10 s (half an e4m3 step: 3 mantissa bits,
smallest subnormal 2^-9).
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import gemm as G
from oracle import glue
from oracle import moe
from oracle import quant as Q

from gpu_helpers import dev_bf16, dev_f32, dev_scales, dev_u8, host_bits16, host_f32_bits, host_u8

pytestmark = pytest.mark.gpu


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def gate_close(hv, rv):
    """The kernel's h against the correctly rounded one: within one bf16 unit,
    or a signed zero where the exact value is below 2^-100 (for h1 < -88 the
    fp32 exponential of -h1 overflows and SiLU(h1) evaluates to -0, as any
    fp32 evaluation of h1 / (1 + e^-h1) does; the exact value is then below
    1e-36)."""
    return (np.abs(hv - rv) <= bf16_ulp(rv) + 1e-40) | ((np.abs(rv) < 2.0 ** -100) & (hv == 0))


def int_operands(M, F_, K, E=1, seed=0):
    """Integer-valued e4m3 operands in [-2, 2] with scales 2^-4..2^-2: every
    partial sum is a multiple of 2^-8 below 2^11 in magnitude (K <= 1040),
    hence exact in fp32 in any order, and the products are of order one, the
    range the gate sees in a real layer."""
    g = np.random.default_rng(seed)
    a = F.e4m3_encode(g.integers(-2, 3, (M, K)).astype(np.float32))
    kb = (K + 127) // 128
    a_s = np.ldexp(np.ones((M, kb), np.float32), g.integers(-4, -1, (M, kb))).astype(np.float32)
    w = F.e4m3_encode(g.integers(-2, 3, (E, 2 * F_, K)).astype(np.float32))
    w_s = np.ldexp(np.ones((E, 2 * F_ // 128, kb), np.float32),
                   g.integers(-4, -1, (E, 2 * F_ // 128, kb))).astype(np.float32)
    return a, a_s, w, w_s


def rand_operands(M, F_, K, E=1, ue8m0=False, seed=0):
    x = I.activations((M, K), I.DENSE_FFN, 500 + seed)
    a, a_s = Q.act_quant(x, ue8m0=ue8m0)
    ws, ss = [], []
    for e in range(E):
        q, s = Q.weight_quant(I.weights_f32((2 * F_, K), I.DENSE_FFN, 600 + 7 * seed + e), ue8m0=ue8m0)
        ws.append(q)
        ss.append(s)
    return a, a_s, np.stack(ws), np.stack(ss)


def oracle_gate(a, a_s, w, w_s):
    """Oracle of one expert: (exact products h1, h3 in fp64, their bf16 bits,
    |A||W|^T for both halves, h bits, (y, s) of act_quant(h))."""
    F_ = w.shape[0] // 2
    A_hat = G.dequant_act(a, a_s)
    W_hat = G.dequant_weight(w, w_s)
    C = A_hat @ W_hat.T
    absC = np.abs(A_hat) @ np.abs(W_hat).T
    hb = F.f32_to_bf16(C)
    h = glue.silu_mul(hb[:, :F_], hb[:, F_:])
    return C, hb, absC, h


def check_quant_of_h(y, s, h, ue8m0, what):
    """The quantisation stage on its own input: on every block, (y, s) must be
    bit for bit the oracle's act_quant of the h that the kernel computed."""
    yo, so = Q.act_quant(h, ue8m0=ue8m0)
    assert np.array_equal(host_f32_bits_np(s), so.view(np.uint32)), f"{what}: scales differ from act_quant(h)"
    assert np.array_equal(np.asarray(y), yo), f"{what}: codes differ from act_quant(h)"


def check_against_oracle(y, s, h, a, a_s, w, w_s, ue8m0, what):
    """Element-wise bound of the module docstring, rows of one expert, and the
    quantisation stage bit-exact on the kernel's own h."""
    check_quant_of_h(y, s, h, ue8m0, what)
    F_ = w.shape[0] // 2
    C, hb, absC, h_ref_bits = oracle_gate(a, a_s, w, w_s)
    h1 = F.bf16_to_f32(hb[:, :F_]).astype(np.float64)
    h3 = F.bf16_to_f32(hb[:, F_:]).astype(np.float64)
    d1 = bf16_ulp(C[:, :F_]) + 2e-5 * absC[:, :F_]
    d3 = bf16_ulp(C[:, F_:]) + 2e-5 * absC[:, F_:]
    h_ref = F.bf16_to_f32(h_ref_bits).astype(np.float64)
    with np.errstate(over="ignore"):
        sil = np.abs(glue.silu(h1))
    bound_h = 1.1 * np.abs(h3) * d1 + sil * d3 + d1 * d3 + 2.0 ** -8 * np.abs(h_ref) + 1e-30
    hg = F.bf16_to_f32(h).astype(np.float64)
    assert np.all(np.isfinite(hg)), what
    bad = np.abs(hg - h_ref) > bound_h
    assert not bad.any(), f"{what}: h outside its bound at {np.argwhere(bad)[:5].tolist()}"
    deq = G.dequant_act(y, s)
    cols = np.arange(F_) // 128
    s_el = np.asarray(s, np.float64)[:, cols]
    bound_q = 2.0 ** -4 * (np.abs(h_ref) + bound_h) + 2.0 ** -10 * s_el + bound_h
    bad = np.abs(deq - h_ref) > bound_q
    assert not bad.any(), f"{what}: y*s outside its bound at {np.argwhere(bad)[:5].tolist()}"
    if ue8m0:
        sb = host_f32_bits_np(s)
        assert np.all(sb & 0x007FFFFF == 0), f"{what}: ue8m0 scale not a power of two"


def host_f32_bits_np(s):
    return np.ascontiguousarray(s, np.float32).view(np.uint32)


def run_dense(a, a_s, w, w_s, fmt="fp32", layout="kb"):
    y, s, h = ds.gemm_silu_mul_act_quant(dev_u8(a), dev_scales(a_s, layout), dev_u8(w), dev_f32(w_s), fmt,
                                         return_h=True)
    torch.cuda.synchronize()
    return host_u8(y), s.cpu().numpy(), host_bits16(h), (y, s, h)


def unfused(a_d, as_d, w_d, ws_d, fmt):
    """The same step through the separate product and gate kernels (GPU).  The
    product runs as a one-expert grouped product, which never splits K (a
    split changes the order of the fp32 additions, the fused kernel does not
    split)."""
    F_ = w_d.shape[0] // 2
    off = torch.tensor([0, a_d.shape[0]], dtype=torch.int32, device="cuda")
    h13 = ds.grouped_gemm(a_d, as_d, w_d[None], ws_d[None], off, scale_fmt=fmt)
    return ds.silu_mul_act_quant(h13[:, :F_], h13[:, F_:], fmt, return_h=True)


def assert_same(fused, ref, what):
    y, s, h = fused
    y2, s2, h2 = ref
    torch.cuda.synchronize()
    assert torch.equal(y, y2), f"{what}: e4m3 codes differ from the unfused path"
    assert torch.equal(s.contiguous().view(torch.int32), s2.contiguous().view(torch.int32)), f"{what}: scales"
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), f"{what}: h"


# ---- dense -------------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("M,F_,K", [(300, 384, 1024), (37, 256, 1024), (64, 128, 512), (65, 512, 1040)])
def test_integer_operands_exact(M, F_, K, fmt):
    a, a_s, w, w_s = int_operands(M, F_, K, seed=M)
    y, s, h, _ = run_dense(a, a_s, w[0], w_s[0], fmt)
    C, hb, _, href = oracle_gate(a, a_s, w[0], w_s[0])
    # every partial sum is exact in fp32: the kernel's h1, h3 are the oracle's
    hv, rv = F.bf16_to_f32(h).astype(np.float64), F.bf16_to_f32(href).astype(np.float64)
    diff = h != href
    assert np.all(gate_close(hv, rv)), "gate off by more than one bf16 ulp"
    assert diff.mean() < 2e-3, f"{diff.mean():.2e} of h differ from the correctly rounded value"
    yr, sr = Q.act_quant(href, ue8m0=(fmt == "ue8m0"))
    clean = ~diff.reshape(M, F_ // 128, 128).any(axis=2)
    assert clean.mean() > 0.5
    assert np.array_equal(host_f32_bits_np(s)[clean], sr.view(np.uint32)[clean])
    mask = clean[:, np.arange(F_) // 128]
    assert np.array_equal(y[mask], yr[mask])
    check_quant_of_h(y, s, h, fmt == "ue8m0", f"{M}x{F_}x{K} {fmt}")


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("M,F_,K", [(1, 128, 256), (64, 256, 7168), (65, 384, 640), (200, 256, 720),
                                    (1300, 5504, 256), (1300, 5504, 720), (300, 16640, 720),
                                    (2048, 5248, 256)])
def test_random_operands_against_oracle(M, F_, K, fmt):
    # (1300, 5504): 6 x 43 = 258 tiles of 256 x 256, the persistent kernel
    # (two workgroups take a second tile), with M and N tails; K = 720 ends
    # in a partial K-block.  On a 256-CU part the launch splits the output
    # columns when the 256-row tiles leave a partial round: (300, 16640)
    # has 2 x 130 tiles, so 128 column blocks run persistent and the last 2
    # as 64-row tiles (with a row tail); (2048, 5248) has 8 x 41 tiles, so
    # 32 blocks run persistent and the last 9 as 128-row tiles (9 x 32
    # 64-row tiles would exceed one round).
    ue = fmt == "ue8m0"
    a, a_s, w, w_s = rand_operands(M, F_, K, ue8m0=ue, seed=M)
    y, s, h, dev = run_dense(a, a_s, w[0], w_s[0], fmt)
    check_against_oracle(y, s, h, a, a_s, w[0], w_s[0], ue, f"{M}x{F_}x{K} {fmt}")
    assert_same(dev, unfused(dev_u8(a), dev_scales(a_s, "kb"), dev_u8(w[0]), dev_f32(w_s[0]), fmt), "dense")


def test_row_major_scales_and_outputs_into_views():
    M, F_, K = 100, 256, 512
    a, a_s, w, w_s = rand_operands(M, F_, K, seed=3)
    yb = torch.zeros((M, F_ + 64), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((M, 4), dtype=torch.float32, device="cuda")
    y, s = yb[:, 16:16 + F_], sb[:, 1:3]
    ds.gemm_silu_mul_act_quant(dev_u8(a), dev_scales(a_s, "row"), dev_u8(w[0]), dev_f32(w_s[0]), out=(y, s))
    ref = run_dense(a, a_s, w[0], w_s[0])
    assert np.array_equal(host_u8(y), ref[0])
    assert np.array_equal(host_f32_bits(s), host_f32_bits_np(ref[1]))
    # nothing outside the views was written
    assert torch.all(yb[:, :16] == 0) and torch.all(yb[:, 16 + F_:] == 0)
    assert torch.all(sb[:, 0] == 0) and torch.all(sb[:, 3] == 0)


def test_k_zero():
    a = torch.empty((5, 0), dtype=torch.uint8, device="cuda")
    a_s = torch.empty((5, 0), dtype=torch.float32, device="cuda")
    w = torch.empty((256, 0), dtype=torch.uint8, device="cuda")
    w_s = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    y, s, h = ds.gemm_silu_mul_act_quant(a, a_s, w, w_s, return_h=True)
    torch.cuda.synchronize()
    # h1 = h3 = 0, so h = 0 and every block takes the floor scale 1e-4 / 448
    assert torch.all(y == 0) and torch.all(h.float() == 0)
    assert np.all(s.cpu().numpy() == np.float32(np.float32(1e-4) / np.float32(448.0)))


def test_unsupported_layout_raises():
    a = torch.zeros((4, 256), dtype=torch.uint8, device="cuda")
    a_s = torch.ones((4, 2), dtype=torch.float32, device="cuda")
    w = torch.zeros((400, 256), dtype=torch.uint8, device="cuda")       # F = 200
    w_s = torch.ones((4, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(ds.Dsfp8Error, match="fused form"):
        ds.gemm_silu_mul_act_quant(a, a_s, w, w_s)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("F_", [18432, 2304])
def test_dense_ffn_full_size_sampled(F_, fmt):
    """The dense feed-forward up-projection (4096 x 2*18432 x 7168), and one
    rank's share of it under 8-way tensor parallelism (F = 2304: 288 tiles of
    256 x 256, whose launch splits the output columns on a 256-CU part), with
    device-drawn inputs: bit-identical to the unfused path everywhere, and
    against the oracle on sampled rows and output blocks, with fp32 and with
    power-of-two (ue8m0) scales."""
    M, K = 4096, 7168
    ue = fmt == "ue8m0"
    xf = I.device_normal((M, K), seed=80, std=1.0, device="cuda", dtype=torch.bfloat16)
    wf = I.device_normal((2 * F_, K), seed=81, std=0.02, device="cuda")
    a, a_s = ds.act_quant(xf, fmt)
    w, w_s = ds.weight_quant(wf, fmt)
    fused = ds.gemm_silu_mul_act_quant(a, a_s, w, w_s, fmt, return_h=True)
    assert_same(fused, unfused(a, a_s, w, w_s, fmt), "dense FFN size")
    y, s, h = fused
    rows = np.sort(np.random.default_rng(80).choice(M, 24, replace=False))
    rows[-1] = M - 1
    blocks = sorted({0, F_ // 128 - 1, *np.random.default_rng(81).choice(F_ // 128, 3, replace=False).tolist()})
    rt = torch.from_numpy(rows).cuda()
    xr = xf[rt].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    ar, asr = Q.act_quant(xr, ue8m0=ue)
    assert np.array_equal(host_u8(a[rt]), ar)
    for j in blocks:
        sel = np.r_[j * 128:(j + 1) * 128, F_ + j * 128:F_ + (j + 1) * 128]
        wr = wf[torch.from_numpy(sel).cuda()].cpu().numpy()
        wq, wsq = Q.weight_quant(wr, ue8m0=ue)
        # the GPU's weight quantiser agrees on these blocks (both halves)
        assert np.array_equal(host_u8(w[torch.from_numpy(sel).cuda()]), wq)
        cols = slice(j * 128, (j + 1) * 128)
        check_against_oracle(host_u8(y[rt, cols]), s[rt, j:j + 1].cpu().numpy(), host_bits16(h[rt, cols]),
                             ar, asr, wq, wsq, ue, f"dense FFN block {j} {fmt}")


# ---- grouped ------------------------------------------------------------------------------

def run_grouped(a, a_s, w, w_s, counts, fmt="fp32"):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    offd = torch.from_numpy(off).cuda()
    ad, asd, wd, wsd = dev_u8(a), dev_scales(a_s, "kb"), dev_u8(w), dev_f32(w_s)
    fused = ds.grouped_gemm_silu_mul_act_quant(ad, asd, wd, wsd, offd, fmt, return_h=True)
    F_ = w.shape[1] // 2
    h13 = ds.grouped_gemm(ad, asd, wd, wsd, offd, scale_fmt=fmt)
    ref = ds.silu_mul_act_quant(h13[:, :F_], h13[:, F_:], fmt, return_h=True)
    assert_same(fused, ref, "grouped")
    y, s, h = fused
    return off, host_u8(y), s.cpu().numpy(), host_bits16(h)


# Row counts that exercise the three tile heights (<= 64, 65..128, > 128 rows),
# remainders past whole 256-row tiles that run in the 64-row class (257, 300),
# the 128-row class (400) or a padded 256-row tile (450), empty experts and
# single rows.
GROUP_COUNTS = [0, 3, 64, 65, 128, 0, 129, 300, 1, 257, 400, 450]


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_grouped_against_oracle(fmt):
    ue = fmt == "ue8m0"
    counts = GROUP_COUNTS
    M, F_, K = sum(counts), 256, 640
    a, a_s, w, w_s = rand_operands(M, F_, K, E=len(counts), ue8m0=ue, seed=11)
    off, y, s, h = run_grouped(a, a_s, w, w_s, counts, fmt)
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            check_against_oracle(y[lo:hi], s[lo:hi], h[lo:hi], a[lo:hi], a_s[lo:hi], w[e], w_s[e], ue,
                                 f"expert {e} ({hi - lo} rows) {fmt}")


def test_grouped_integer_operands_exact():
    counts = [5, 0, 70, 140]
    M, F_, K = sum(counts), 128, 1024
    a, a_s, w, w_s = int_operands(M, F_, K, E=len(counts), seed=7)
    off, y, s, h = run_grouped(a, a_s, w, w_s, counts)
    for e in range(len(counts)):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        _, _, _, href = oracle_gate(a[lo:hi], a_s[lo:hi], w[e], w_s[e])
        diff = h[lo:hi] != href
        rv = F.bf16_to_f32(href).astype(np.float64)
        assert np.all(gate_close(F.bf16_to_f32(h[lo:hi]).astype(np.float64), rv))
        yr, sr = Q.act_quant(href)
        clean = ~diff.reshape(hi - lo, 1, 128).any(axis=2)
        assert np.array_equal(host_f32_bits_np(s[lo:hi])[clean], sr.view(np.uint32)[clean])
        mask = clean[:, np.zeros(F_, int)]
        assert np.array_equal(y[lo:hi][mask], yr[mask])
        check_quant_of_h(y[lo:hi], s[lo:hi], h[lo:hi], False, f"expert {e}")


def test_routed_expert_size_sampled():
    """The routed-expert up-projection at its full size (4096 tokens x top-8 of
    256 experts, dim 7168, inter 2048) with device-drawn weights: fused equals
    unfused everywhere; sampled rows of a few experts against the oracle."""
    d = I.WORKLOADS["moe"].dims
    T, E, k, D, F_ = d["tokens"], d["experts"], d["topk"], d["dim"], d["inter"]
    idx, _ = I.zipf_topk(T, E, k, d["zipf_s"])
    offsets, row_token, _, _ = moe.route(idx, E)
    x = I.device_normal((T, D), seed=90, std=1.0, device="cuda", dtype=torch.bfloat16)
    rt = torch.from_numpy(row_token.astype(np.int32)).cuda()
    a, a_s = ds.act_quant_rows(x, rt)
    w = torch.empty((E, 2 * F_, D), dtype=torch.uint8, device="cuda")
    w_s = torch.empty((E, 2 * F_ // 128, D // 128), dtype=torch.float32, device="cuda")

    def source(e):
        return I.device_normal((2 * F_, D), seed=1000 + e, std=0.02, device="cuda")

    for e in range(E):
        q, sc = ds.weight_quant(source(e))
        w[e].copy_(q)
        w_s[e].copy_(sc)
    offd = torch.from_numpy(offsets.astype(np.int32)).cuda()
    fused = ds.grouped_gemm_silu_mul_act_quant(a, a_s, w, w_s, offd, return_h=True)
    h13 = ds.grouped_gemm(a, a_s, w, w_s, offd)
    assert_same(fused, ds.silu_mul_act_quant(h13[:, :F_], h13[:, F_:], return_h=True), "routed-expert size")
    del h13
    # The per-token quantised input read through the row index gives the same
    # bytes (act_quant is row-local, so it commutes with the row selection).
    xq, xs = ds.act_quant(x)
    gathered = ds.grouped_gemm_silu_mul_act_quant(xq, xs, w, w_s, offd, return_h=True, rows=rt)
    assert_same(gathered, fused, "routed-expert size, rows read through the index")
    del gathered
    y, s, h = fused
    counts = np.diff(offsets)
    picks = [int(np.argmax(counts)), int(np.argmin(np.where(counts > 0, counts, 1 << 30))),
             int(np.nonzero((counts > 64) & (counts <= 128))[0][0])]
    g = np.random.default_rng(91)
    for e in picks:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = np.unique(np.r_[lo, hi - 1, g.integers(lo, hi, 6)])
        rd = torch.from_numpy(rows).cuda()
        xr = x[torch.from_numpy(row_token[rows]).cuda()].contiguous().view(torch.int16).cpu().numpy()
        ar, asr = Q.act_quant(xr.view(np.uint16))
        assert np.array_equal(host_u8(a[rd]), ar)
        blk = int(g.integers(0, F_ // 128))
        sel = np.r_[blk * 128:(blk + 1) * 128, F_ + blk * 128:F_ + (blk + 1) * 128]
        # the oracle quantises the same source rows; the GPU's bytes must agree
        wq, wsq = Q.weight_quant(source(e)[torch.from_numpy(sel).cuda()].cpu().numpy())
        assert np.array_equal(host_u8(w[e][torch.from_numpy(sel).cuda()]), wq)
        cols = slice(blk * 128, (blk + 1) * 128)
        check_against_oracle(host_u8(y[rd, cols]), s[rd, blk:blk + 1].cpu().numpy(), host_bits16(h[rd, cols]),
                             ar, asr, wq, wsq, False, f"expert {e} ({hi - lo} rows) block {blk}")


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_grouped_gather_equals_gathered_copy(fmt):
    """Rows read through an index (with entries outside [0, T), which clamp)
    equal the product of the explicitly gathered, quantised rows."""
    counts = GROUP_COUNTS
    M, F_, K, T = sum(counts), 256, 640, 300
    g = np.random.default_rng(12)
    x = dev_bf16(I.activations((T, K), I.MOE, 70))
    idx = g.integers(0, T, M).astype(np.int32)
    idx[[0, 7, M - 1]] = [-3, T + 5, T - 1]
    rows = torch.from_numpy(idx).cuda()
    _, _, w, w_s = rand_operands(8, F_, K, E=len(counts), ue8m0=fmt == "ue8m0", seed=13)
    wd, wsd = dev_u8(w), dev_f32(w_s)
    offd = torch.from_numpy(np.r_[0, np.cumsum(counts)].astype(np.int32)).cuda()
    a, a_s = ds.act_quant_rows(x, rows, fmt)
    ref = ds.grouped_gemm_silu_mul_act_quant(a, a_s, wd, wsd, offd, fmt, return_h=True)
    xq, xs = ds.act_quant(x, fmt)
    got = ds.grouped_gemm_silu_mul_act_quant(xq, xs, wd, wsd, offd, fmt, return_h=True, rows=rows)
    assert_same(got, ref, f"gathered rows {fmt}")
    # and the row-major scale layout of the token scales
    xs_rm = xs.contiguous()
    got = ds.grouped_gemm_silu_mul_act_quant(xq, xs_rm, wd, wsd, offd, fmt, return_h=True, rows=rows)
    assert_same(got, ref, f"gathered rows {fmt}, row-major scales")

"""GPU parity of the grouped block-scaled product over per-expert row ranges.

The oracle is the per-expert loop (Admin Guide 6.4 / 8.4) of the fp64
block-scaled product; tolerance as in gpu_helpers.  Cases: empty experts,
one expert (equal, bit for bit, to the dense kernel), ragged N/K, a single
row per expert, and the routed-expert workload at full size (256 experts,
Zipf(1.1) top-8 routing of 4096 tokens, up- and down-projection shapes) on
sampled experts, rows and columns.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import gemm as G
from oracle import moe
from oracle import quant as Q

from gpu_helpers import check_product, dev_f32, dev_scales, dev_u8, host_bits16, host_u8

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


def _run(a, a_s, b, b_s, off, layout="kb", scale_fmt="fp32"):
    c = ds.grouped_gemm(dev_u8(a), dev_scales(a_s, layout), dev_u8(b), dev_f32(b_s), torch.from_numpy(off).cuda(),
                        scale_fmt=scale_fmt)
    torch.cuda.synchronize()
    return host_bits16(c)


def _check_all(C, a, a_s, b, b_s, off, what):
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        A_hat = G.dequant_act(a[lo:hi], a_s[lo:hi])
        W_hat = G.dequant_weight(b[e], b_s[e])
        check_product(C[lo:hi], A_hat @ W_hat.T, A_hat, W_hat, f"{what} expert {e}")


@pytest.mark.parametrize("counts,N,K", [
    ([5, 0, 17, 1, 0, 300, 9], 140, 300),
    ([1] * 20, 256, 512),
    ([0, 0, 129, 0], 64, 1000),
    ([130, 127, 128, 1, 255], 384, 256),
    ([70, 3, 300, 0, 129], 256, 272),  # partial last K-block on the direct-to-LDS path
    # experts above 256 rows whose rows past the last whole 256-row tile run
    # in the 64-row class (257, 320), the 128-row class (321, 356, 640), or
    # a padded 256-row tile (700); 512 has no remainder
    ([257, 320, 321, 356, 512, 640, 700, 5], 256, 256),
])
@pytest.mark.parametrize("layout", ["kb", "row"])
def test_grouped_small(counts, N, K, layout):
    a, a_s, b, b_s, off = _case(counts, N, K, len(counts))
    C = _run(a, a_s, b, b_s, off, layout)
    _check_all(C, a, a_s, b, b_s, off, f"{counts}")


@pytest.mark.parametrize("counts,N,K", [
    ([5, 0, 17, 1, 0, 300, 9], 256, 512),
    ([70, 3, 300, 0, 129], 256, 272),
])
def test_grouped_ue8m0(counts, N, K):
    a, a_s, b, b_s, off = _case(counts, N, K, len(counts), ue8m0=True)
    C = _run(a, a_s, b, b_s, off, scale_fmt="ue8m0")
    _check_all(C, a, a_s, b, b_s, off, f"ue8m0 {counts}")


def test_many_experts():
    """More experts than the tile schedule takes in one step (1024): the
    per-class tile counts carry across steps; tiles of all three heights."""
    g = np.random.default_rng(17)
    counts = g.choice([0, 1, 2, 3, 5], size=1500)
    counts[[3, 700, 1030, 1499]] = [70, 130, 300, 257]
    a, a_s, b, b_s, off = _case(counts, 128, 256, 21)
    C = _run(a, a_s, b, b_s, off)
    _check_all(C, a, a_s, b, b_s, off, "1500 experts")


def test_single_expert_equals_dense():
    # 9 x 16 output tiles: enough that the dense product does not split K, so
    # both run the same tile code in the same accumulation order.
    a, a_s, b, b_s, off = _case([1100], 2000, 1000, 3)
    C = _run(a, a_s, b, b_s, off)
    Cd = ds.gemm(dev_u8(a), dev_scales(a_s, "kb"), dev_u8(b[0]), dev_f32(b_s[0]))
    torch.cuda.synchronize()
    assert np.array_equal(C, host_bits16(Cd))


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_rows_past_the_last_expert(fmt):
    """Row buffers sized for more rows than the experts own (one rank's share
    under expert parallelism: sized for every routed pair, only the local
    experts' rows counted by the offsets): the owned rows are bit for bit
    the product over exactly those rows, and the rows past offsets[E] are
    left as they were, for the plain and the gated-and-gathered forms."""
    ue = fmt == "ue8m0"
    counts = [5, 0, 300, 70, 129, 1]
    a, a_s, b, b_s, off = _case(counts, 256, 384, 31, ue8m0=ue)
    R = int(off[-1])
    extra = 700
    g = np.random.default_rng(31)
    a_big = np.concatenate([a, g.integers(0, 126, (extra, a.shape[1])).astype(np.uint8)])
    as_big = np.concatenate([a_s, np.full((extra, a_s.shape[1]), 0.5, np.float32)])
    offd = torch.from_numpy(off).cuda()
    sentinel = 0x3F80  # bf16 1.0
    c = torch.full((R + extra, 256), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ds.grouped_gemm(dev_u8(a_big), dev_scales(as_big, "kb"), dev_u8(b), dev_f32(b_s), offd, out=c, scale_fmt=fmt)
    want = _run(a, a_s, b, b_s, off, scale_fmt=fmt)
    got = host_bits16(c)
    assert np.array_equal(got[:R], want), "owned rows differ from the product over exactly those rows"
    assert np.all(got[R:] == sentinel), "rows past the last expert were written"

    # gated form, rows read through an index as in the routed step
    F_ = 128
    q13 = np.stack([Q.weight_quant(I.weights_f32((2 * F_, 384), I.MOE, 77 + e), ue8m0=ue)[0]
                    for e in range(len(counts))])
    s13 = np.stack([Q.weight_quant(I.weights_f32((2 * F_, 384), I.MOE, 77 + e), ue8m0=ue)[1]
                    for e in range(len(counts))])
    src = g.permutation(R + extra).astype(np.int32)  # product row r reads row src[r] of a_big
    rows_big = torch.from_numpy(src).cuda()
    y = torch.full((R + extra, F_), 0x5A, dtype=torch.uint8, device="cuda")
    sc = ds.new_scales(R + extra, 1, "cuda").fill_(-1.0)
    ds.grouped_gemm_silu_mul_act_quant(dev_u8(a_big), dev_scales(as_big, "kb"), dev_u8(q13), dev_f32(s13), offd, fmt,
                                       out=(y, sc), rows=rows_big)
    y_ref, s_ref = ds.grouped_gemm_silu_mul_act_quant(dev_u8(a_big), dev_scales(as_big, "kb"), dev_u8(q13),
                                                      dev_f32(s13), offd, fmt, rows=rows_big[:R].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y[:R], y_ref) and torch.equal(sc[:R].contiguous(), s_ref.contiguous()), "gated owned rows"
    assert torch.all(y[R:] == 0x5A) and torch.all(sc[R:] == -1.0), "gated rows past the last expert were written"


def test_all_rows_in_last_expert():
    a, a_s, b, b_s, off = _case([0, 0, 0, 200], 128, 384, 4)
    C = _run(a, a_s, b, b_s, off)
    _check_all(C, a, a_s, b, b_s, off, "last")


@pytest.mark.parametrize("proj", ["up", "down"])
def test_routed_experts_full_size_sampled(proj):
    dims = I.WORKLOADS["moe"].dims
    E, dim, inter = dims["experts"], dims["dim"], dims["inter"]
    N, K = (2 * inter, dim) if proj == "up" else (dim, inter)
    idx, _ = I.zipf_topk(dims["tokens"], E, dims["topk"], dims["zipf_s"])
    off, tok, _, _ = moe.route(idx, E)
    off = off.astype(np.int32)
    counts = np.diff(off)
    M = int(off[-1])
    # activations: the routed rows (token gathered per row), drawn on the device
    xt = I.device_normal((dims["tokens"], K), seed=900, std=1.0, device="cuda", dtype=torch.bfloat16)
    x = xt[torch.from_numpy(tok).cuda()]
    a, a_s = ds.act_quant(x)
    # expert weights drawn per expert on the device and quantised there
    b = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
    b_s = torch.empty((E, (N + 127) // 128, (K + 127) // 128), dtype=torch.float32, device="cuda")
    seeds = 5000 + np.arange(E)
    for e in range(E):
        w = I.device_normal((N, K), seed=int(seeds[e]), std=0.02, device="cuda")
        q, s = ds.weight_quant(w)
        b[e].copy_(q)
        b_s[e].copy_(s)
        del w
    c = ds.grouped_gemm(a, a_s, b, b_s, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    g = np.random.default_rng(7)
    big = int(np.argmax(counts))
    small = [int(e) for e in np.argsort(counts)[:2]]
    experts = sorted({big, *small, *g.choice(E, 3, replace=False).tolist()})
    nb = (N + 127) // 128
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], g.integers(lo, hi, min(32, hi - lo))]))
        xr = x[torch.from_numpy(rows).cuda()].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        ar, asr = Q.act_quant(xr)
        assert np.array_equal(host_u8(a[torch.from_numpy(rows).cuda()]), ar)
        A_hat = G.dequant_act(ar, asr)
        for bi in sorted({0, nb - 1, int(g.integers(0, nb))}):
            n0, n1 = bi * 128, min(N, bi * 128 + 128)
            w = I.device_normal((N, K), seed=int(seeds[e]), std=0.02, device="cuda")[n0:n1].cpu().numpy()
            br, bsr = Q.weight_quant(w)
            assert np.array_equal(host_u8(b[e, n0:n1]), br)
            W_hat = G.dequant_weight(br, bsr)
            Cg = host_bits16(c[torch.from_numpy(rows).cuda(), n0:n1])
            check_product(Cg, A_hat @ W_hat.T, A_hat, W_hat, f"{proj} expert {e} block {bi}")


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
@pytest.mark.parametrize("K", [512, 560])
def test_tile_plan_and_id_mapping_agree(fmt, K):
    """With a 16-byte aligned workspace the merged grouped launch reads every
    workgroup's tile from the plan written ahead of it; with a workspace that
    is only 4-byte aligned each workgroup maps its id to its tile itself.  The
    two must give the same bytes, for the plain, the gated and the gathered
    gated product, on experts of every tile height (64-, 128- and 256-row
    classes, a large expert's remainder tiles, empty experts) and with a
    partial last K-block."""
    dev = "cuda"
    counts = np.array([0, 3, 64, 65, 128, 129, 300, 0, 520, 37, 700, 1, 256, 384])
    E, M = len(counts), int(counts.sum())
    N, F = 640, 256
    kb = lambda n: (n + 127) // 128
    off = torch.from_numpy(np.r_[0, np.cumsum(counts)].astype(np.int32)).to(dev)
    x = I.device_normal((M, K), seed=91, std=1.0, device=dev, dtype=torch.bfloat16)
    a, a_s = ds.act_quant(x, fmt)
    w = torch.empty((E, N, K), dtype=torch.uint8, device=dev)
    w_s = torch.empty((E, kb(N), kb(K)), dtype=torch.float32, device=dev)
    w13 = torch.empty((E, 2 * F, K), dtype=torch.uint8, device=dev)
    w13_s = torch.empty((E, kb(2 * F), kb(K)), dtype=torch.float32, device=dev)
    for e in range(E):
        q, s = ds.weight_quant(I.device_normal((N, K), seed=500 + e, std=0.02, device=dev), fmt)
        w[e].copy_(q)
        w_s[e].copy_(s)
        q, s = ds.weight_quant(I.device_normal((2 * F, K), seed=700 + e, std=0.02, device=dev), fmt)
        w13[e].copy_(q)
        w13_s[e].copy_(s)
    rows = torch.from_numpy(np.random.default_rng(5).integers(0, M, M).astype(np.int32)).to(dev)
    lib = ds._lib.load()
    need = max(lib.dsfp8_grouped_gemm_workspace_bytes(E, M, N, K), lib.dsfp8_grouped_gemm_workspace_bytes(E, M, 2 * F, K))
    big = torch.empty(need + 64, dtype=torch.uint8, device=dev)
    planned, unplanned = big[:need], big[4:4 + need]
    assert planned.data_ptr() % 16 == 0 and unplanned.data_ptr() % 16 == 4

    def outputs(ws):
        c = ds.grouped_gemm(a, a_s, w, w_s, off, workspace=ws, scale_fmt=fmt)
        g = ds.grouped_gemm_silu_mul_act_quant(a, a_s, w13, w13_s, off, fmt, return_h=True, workspace=ws)
        r = ds.grouped_gemm_silu_mul_act_quant(a, a_s, w13, w13_s, off, fmt, return_h=True, workspace=ws, rows=rows)
        torch.cuda.synchronize()
        return [t.contiguous().view(torch.uint8).cpu() for t in (c, *g, *r)]

    for name, p, q in zip(["plain", "y", "s", "h", "gathered y", "gathered s", "gathered h"], outputs(planned),
                          outputs(unplanned)):
        assert torch.equal(p, q), f"{name}: tile plan and per-workgroup mapping differ"


def test_k_zero_writes_zeros():
    """K = 0: every row of every expert, in all three tile classes, is an
    empty sum; the plain product writes zeros over a sentinel, the gated one
    h = 0, zero codes and the floor scale 1e-4 / 448."""
    dev = "cuda"
    counts = np.array([0, 7, 100, 300, 0, 64])
    E, M, N, F = len(counts), int(counts.sum()), 384, 256
    off = torch.from_numpy(np.r_[0, np.cumsum(counts)].astype(np.int32)).to(dev)
    a = torch.empty((M, 0), dtype=torch.uint8, device=dev)
    a_s = torch.empty((M, 0), dtype=torch.float32, device=dev)
    c = torch.full((M, N), 0x7fff, dtype=torch.int16, device=dev).view(torch.bfloat16)
    out = ds.grouped_gemm(a, a_s, torch.empty((E, N, 0), dtype=torch.uint8, device=dev),
                          torch.empty((E, (N + 127) // 128, 0), dtype=torch.float32, device=dev), off, out=c)
    y, s, h = ds.grouped_gemm_silu_mul_act_quant(a, a_s, torch.empty((E, 2 * F, 0), dtype=torch.uint8, device=dev),
                                                 torch.empty((E, 2 * F // 128, 0), dtype=torch.float32, device=dev),
                                                 off, return_h=True)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0)
    assert torch.all(y == 0) and torch.all(h.view(torch.int16) == 0)
    assert np.all(s.cpu().numpy() == np.float32(np.float32(1e-4) / np.float32(448.0)))

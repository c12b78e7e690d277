"""The feed-forward steps captured into a HIP graph and replayed.

None of the library's kernels allocates, clears memory with a runtime memset
or synchronises the host, so a whole step (act_quant, the gated
up-projection, the down-projection; for the routed experts also routing,
the up-projection reading its rows through the routing index, and
combining) can be captured once and replayed.  A replay
must read the buffers as they are at replay time and write exactly what the
eager calls write.  Each test replays several times, with new inputs written
into the captured buffers, the eager step run and the host synchronised
between replays, and checks every replay against the eager step bit for bit;
the first replay's output is also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import moe
from oracle import quant as Q

from gpu_helpers import dev_bf16, dev_f32, dev_u8, host_bits16

pytestmark = pytest.mark.gpu

REPLAYS = 4


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _bits(t):
    return t.contiguous().view(-1).view(torch.uint8).clone()


def _replay_matches_eager(g, step, outs, refill):
    """For each replay: new inputs, the eager step, then the graph; the graph's
    outputs must equal the eager outputs byte for byte."""
    firsts = None
    for r in range(REPLAYS):
        refill(r)
        step()
        torch.cuda.synchronize()
        want = [_bits(o) for o in outs]
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(_bits(o), w), f"replay {r}: output {i} differs from the eager step"
        if firsts is None:
            firsts = [o.clone() for o in outs]
    return firsts


def _capture(step):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_dense_step_graph(fmt):
    M, D, Fi = 300, 768, 384
    ue = fmt == "ue8m0"
    xs_host = [I.activations((M, D), I.DENSE_FFN, 900 + r) for r in range(REPLAYS)]
    w13 = I.weights_f32((2 * Fi, D), I.DENSE_FFN, 910)
    w2 = I.weights_f32((D, Fi), I.DENSE_FFN, 911)
    q13, s13 = Q.weight_quant(w13, ue8m0=ue)
    q2, s2 = Q.weight_quant(w2, ue8m0=ue)
    q13d, s13d, q2d, s2d = dev_u8(q13), dev_f32(s13), dev_u8(q2), dev_f32(s2)
    x = dev_bf16(xs_host[0])
    xq = torch.empty((M, D), dtype=torch.uint8, device="cuda")
    xsc = ds.new_scales(M, ds.kblocks(D), "cuda")
    hq = torch.empty((M, Fi), dtype=torch.uint8, device="cuda")
    hsc = ds.new_scales(M, ds.kblocks(Fi), "cuda")
    out = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")

    def step():
        ds.act_quant(x, fmt, out=(xq, xsc))
        ds.gemm_silu_mul_act_quant(xq, xsc, q13d, s13d, fmt, out=(hq, hsc))
        ds.gemm(hq, hsc, q2d, s2d, out=out, scale_fmt=fmt)

    step()
    g = _capture(step)

    def refill(r):
        x.copy_(dev_bf16(xs_host[r]))

    first = _replay_matches_eager(g, step, [xq, xsc, hq, hsc, out], refill)

    # The first replay (input xs_host[0]) against the oracle's feed-forward.
    ref = F.bf16_to_f32(moe.expert_ffn(xs_host[0], q13, s13, q2, s2, ue8m0=ue)).astype(np.float64)
    got = F.bf16_to_f32(host_bits16(first[4])).astype(np.float64)
    fro = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert fro <= 2e-2, f"relative Frobenius error {fro:.3e}"


def test_dense_step_graph_persistent_products():
    """A dense step large enough that both products run the persistent kernel
    (6 x 43 = 258 tiles of 256 x 256 each, M, N and K tails): the replays
    equal the eager step byte for byte (the products' parity against the
    oracle at these paths is checked in the product tests)."""
    M, D, Fi = 1300, 11008, 5504
    g = torch.Generator(device="cuda").manual_seed(5)
    x = (torch.randn((M, D), device="cuda", generator=g)).to(torch.bfloat16)
    q13, s13 = ds.weight_quant(torch.randn((2 * Fi, D), device="cuda", generator=g) * 0.02)
    q2, s2 = ds.weight_quant(torch.randn((D, Fi), device="cuda", generator=g) * 0.02)
    xq = torch.empty((M, D), dtype=torch.uint8, device="cuda")
    xsc = ds.new_scales(M, ds.kblocks(D), "cuda")
    hq = torch.empty((M, Fi), dtype=torch.uint8, device="cuda")
    hsc = ds.new_scales(M, ds.kblocks(Fi), "cuda")
    out = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")

    def step():
        ds.act_quant(x, out=(xq, xsc))
        ds.gemm_silu_mul_act_quant(xq, xsc, q13, s13, out=(hq, hsc))
        ds.gemm(hq, hsc, q2, s2, out=out)

    step()
    gr = _capture(step)
    seeds = [11, 12, 13, 14]

    def refill(r):
        gg = torch.Generator(device="cuda").manual_seed(seeds[r])
        x.copy_(torch.randn((M, D), device="cuda", generator=gg).to(torch.bfloat16))

    _replay_matches_eager(gr, step, [xq, xsc, hq, hsc, out], refill)


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_routed_step_graph(fmt):
    T, D, Fi, E, k = 160, 512, 256, 8, 2
    ue = fmt == "ue8m0"
    lib = ds._lib.load()
    xs_host = [I.activations((T, D), I.MOE, 950 + r) for r in range(REPLAYS)]
    routes = [I.zipf_topk(T, E, k, 1.1, seed=960 + r) for r in range(REPLAYS)]
    q13, s13, q2, s2 = [], [], [], []
    for e in range(E):
        a, b = Q.weight_quant(I.weights_f32((2 * Fi, D), I.MOE, 970 + e), ue8m0=ue)
        c, d = Q.weight_quant(I.weights_f32((D, Fi), I.MOE, 990 + e), ue8m0=ue)
        q13.append(a); s13.append(b); q2.append(c); s2.append(d)
    q13, s13, q2, s2 = map(np.stack, (q13, s13, q2, s2))
    q13d, s13d, q2d, s2d = dev_u8(q13), dev_f32(s13), dev_u8(q2), dev_f32(s2)

    M = T * k
    x = dev_bf16(xs_host[0])
    idx = dev_i32(routes[0][0])
    wts = dev_bf16(routes[0][1])
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_token = torch.empty(M, dtype=torch.int32, device="cuda")
    token_rows = torch.empty((T, k), dtype=torch.int32, device="cuda")
    rws = torch.empty(max(lib.dsfp8_moe_route_workspace_bytes(T, k, E), 4), dtype=torch.uint8, device="cuda")
    xq = torch.empty((T, D), dtype=torch.uint8, device="cuda")
    xsc = ds.new_scales(T, ds.kblocks(D), "cuda")
    hq = torch.empty((M, Fi), dtype=torch.uint8, device="cuda")
    hsc = ds.new_scales(M, ds.kblocks(Fi), "cuda")
    yr = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, D), dtype=torch.bfloat16, device="cuda")
    gws = torch.empty(max(lib.dsfp8_grouped_gemm_workspace_bytes(E, M, 2 * Fi, D),
                          lib.dsfp8_grouped_gemm_workspace_bytes(E, M, D, Fi), 4), dtype=torch.uint8, device="cuda")

    def step():
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.dsfp8_moe_route(idx.data_ptr(), T, k, k, E, off.data_ptr(), row_token.data_ptr(),
                                 token_rows.data_ptr(), rws.data_ptr(), rws.numel(), stream)
        assert st == 0, ds.status_string(st)
        ds.act_quant(x, fmt, out=(xq, xsc))
        ds.grouped_gemm_silu_mul_act_quant(xq, xsc, q13d, s13d, off, fmt, out=(hq, hsc), workspace=gws, rows=row_token)
        ds.grouped_gemm(hq, hsc, q2d, s2d, off, out=yr, workspace=gws, scale_fmt=fmt)
        ds.moe_combine(yr, idx, wts, token_rows, out=y)

    step()
    g = _capture(step)

    def refill(r):
        x.copy_(dev_bf16(xs_host[r]))
        idx.copy_(dev_i32(routes[r][0]))
        wts.copy_(dev_bf16(routes[r][1]))

    first = _replay_matches_eager(g, step, [off, row_token, token_rows, xq, xsc, hq, hsc, yr, y], refill)

    idx0, w0 = routes[0]
    ref = F.bf16_to_f32(moe.moe_forward(xs_host[0], idx0, w0, q13, s13, q2, s2, ue8m0=ue)).astype(np.float64)
    got = F.bf16_to_f32(host_bits16(first[8])).astype(np.float64)
    fro = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert fro <= 2e-2, f"relative Frobenius error {fro:.3e}"

"""Benchmark of the block-scaled FP8 linear layer on one MI355X.

Headline workload: the dense FFN at prefill (4096 tokens, dim 7168, inter
18432).  One step is the whole hot path of one FFN layer with every input
already resident in HBM:

    act_quant(x [4096, 7168])                          -> e4m3 + scales
    gemm_silu_mul_act_quant(x_q, [w1; w3] e4m3 [36864, 7168])
                                                       -> e4m3 [4096, 18432] + scales
        (the up-projection with the SiLU gate and the next act_quant in
        its epilogue)
    gemm(h_q, w2 e4m3 [7168, 18432])                   -> bf16 [4096, 7168]

``value`` is the step's GEMM work (3 x 2*4096*18432*7168 flop) divided by the
step time, in TFLOP/s.  Every kernel launch is bracketed by HIP events on the
launch stream, which gives each kernel's average duration; ``roofline``
reports the dominant kernel (the gated up-projection) against the FP8 dense
MFMA peak.  The same step with the product, gate and quantisation as
separate kernels is reported under ``other_workloads`` for comparison.  The other workloads (routed experts, weight dequantisation, the
decode projection, the ragged ue8m0 case) are timed the same way and reported
under ``other_workloads``.  ``cpu_baseline`` times the CPU oracle on a bounded
sample of the same step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_scaled_fp8_act_amd as ds  # noqa: E402
from block_scaled_fp8_act_amd import inputs as I  # noqa: E402

METRIC = "block-scaled FP8 GEMM TFLOP/s & % of MI355X FP8 MFMA peak; act_quant GB/s"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)


def kb(n):
    return (n + 127) // 128


class Timer:
    """Per-kernel HIP-event timing on the current (launch) stream."""

    def __init__(self):
        self.samples = {}
        self.pending = []

    def run(self, name, fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pending.append((name, e0, e1))

    def collect(self):
        torch.cuda.synchronize()
        for name, e0, e1 in self.pending:
            self.samples.setdefault(name, []).append(e0.elapsed_time(e1) * 1e3)  # us
        self.pending = []

    def avg_us(self, name):
        return float(np.mean(self.samples[name]))

    def spread(self, name):
        """Median and minimum of a kernel's launches (us), beside the mean."""
        v = self.samples[name]
        return {"us_median": round(float(np.median(v)), 1), "us_min": round(float(np.min(v)), 1), "launches": len(v)}

    def reset(self):
        self.samples = {}
        self.pending = []


# ---- dense FFN step ---------------------------------------------------------------------

def setup_dense(dev, fmt="fp32", unfused=False, inter=None):
    d = I.WORKLOADS["dense_ffn"].dims
    M, D, F = d["M"], d["dim"], inter if inter is not None else d["inter"]
    x = I.device_normal((M, D), seed=301, std=1.0, device=dev, dtype=torch.bfloat16)
    w13 = I.device_normal((2 * F, D), seed=302, std=0.02, device=dev)
    q13, s13 = ds.weight_quant(w13, fmt)
    del w13
    w2 = I.device_normal((D, F), seed=303, std=0.02, device=dev)
    q2, s2 = ds.weight_quant(w2, fmt)
    del w2
    bufs = dict(
        x=x, q13=q13, s13=s13, q2=q2, s2=s2,
        xq=torch.empty((M, D), dtype=torch.uint8, device=dev),
        xs=ds.new_scales(M, kb(D), dev),
        h13=torch.empty((M, 2 * F), dtype=torch.bfloat16, device=dev) if unfused else None,
        hq=torch.empty((M, F), dtype=torch.uint8, device=dev),
        hs=ds.new_scales(M, kb(F), dev),
        out=torch.empty((M, D), dtype=torch.bfloat16, device=dev),
    )
    torch.cuda.synchronize()
    return dict(M=M, D=D, F=F, b=bufs, fmt=fmt, unfused=unfused)


def dense_step(st, T):
    b, F, fmt = st["b"], st["F"], st["fmt"]
    T.run("act_quant", lambda: ds.act_quant(b["x"], fmt, out=(b["xq"], b["xs"])))
    if st["unfused"]:
        T.run("gemm_up", lambda: ds.gemm(b["xq"], b["xs"], b["q13"], b["s13"], out=b["h13"], scale_fmt=fmt))
        T.run("silu_mul_act_quant",
              lambda: ds.silu_mul_act_quant(b["h13"][:, :F], b["h13"][:, F:], fmt, out=(b["hq"], b["hs"])))
    else:
        T.run("gemm_up_gate",
              lambda: ds.gemm_silu_mul_act_quant(b["xq"], b["xs"], b["q13"], b["s13"], fmt, out=(b["hq"], b["hs"])))
    T.run("gemm_down", lambda: ds.gemm(b["hq"], b["hs"], b["q2"], b["s2"], out=b["out"], scale_fmt=fmt))


def run_dense(st, steps, warmup):
    """Time `steps` dense FFN steps after `warmup`; returns (ms per step, Timer)."""
    T = Timer()
    for _ in range(warmup):
        dense_step(st, T)
    T.collect()
    T.reset()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        dense_step(st, T)
    s1.record()
    T.collect()
    torch.cuda.synchronize()
    return s0.elapsed_time(s1) / steps, T


class NoTimer:
    """Stand-in for Timer inside graph capture (no events in the graph)."""

    def run(self, name, fn):
        fn()


def capture(step_fn):
    """One step captured into a HIP graph (the step only enqueues device work)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_fn()
    return g


def _bits(t):
    return t.contiguous().view(-1).view(torch.uint8)


def check_replays(g, eager_step, outs, replays=3):
    """Replay the graph `replays` times with the eager step in between; every
    replay must reproduce the eager step's outputs bit for bit."""
    for _ in range(replays):
        eager_step()
        torch.cuda.synchronize()
        want = [o.clone() for o in outs]
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            if not torch.equal(_bits(o), _bits(w)):
                raise RuntimeError("graph replay differs from the eager step")


def time_graph(g, steps, warmup):
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        g.replay()
    s1.record()
    torch.cuda.synchronize()
    return s0.elapsed_time(s1) / steps


def dense_kernels(st, T):
    M, D, F = st["M"], st["D"], st["F"]
    k = {}
    up = "gemm_up" if st["unfused"] else "gemm_up_gate"
    for name, fl in ((up, 2.0 * M * 2 * F * D), ("gemm_down", 2.0 * M * D * F)):
        us = T.avg_us(name)
        k[name] = {"shape": [M, 2 * F if name == up else D, D if name == up else F],
                   "us": round(us, 1), "tflops": round(fl / us / 1e6, 1),
                   "frac_of_fp8_peak": round(fl / us / 1e6 / PEAK_FP8_TFLOPS, 4), **T.spread(name)}
    mem = [("act_quant", aq_bytes(M, D))]
    if st["unfused"]:
        mem.append(("silu_mul_act_quant", aq_bytes(M, F, 2)))
    for name, by in mem:
        us = T.avg_us(name)
        k[name] = {"us": round(us, 1), "gbs": round(by / us / 1e3, 1),
                   "frac_of_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 4), **T.spread(name)}
    return k


def bench_bf16_path(dev, steps):
    """The pages' default (bf16) path for the same dense FFN step, as a
    comparison: each linear dequantises its e4m3 weight with weight_dequant
    and multiplies in bf16 (the vendor library's GEMM through
    torch.mm, a two-dimensional product); the gate is SiLU(w1 x) * (w3 x) in bf16."""
    st = setup_dense(dev, unfused=True)
    b, M, D, F = st["b"], st["M"], st["D"], st["F"]
    w13 = torch.empty((2 * F, D), dtype=torch.bfloat16, device=dev)
    w2 = torch.empty((D, F), dtype=torch.bfloat16, device=dev)
    T = Timer()

    def step():
        T.run("dequant_w13", lambda: ds.weight_dequant(b["q13"], b["s13"], out=w13))
        T.run("gemm_up_bf16", lambda: torch.mm(b["x"], w13.t(), out=b["h13"]))
        h = torch.nn.functional.silu(b["h13"][:, :F]) * b["h13"][:, F:]
        T.run("dequant_w2", lambda: ds.weight_dequant(b["q2"], b["s2"], out=w2))
        T.run("gemm_down_bf16", lambda: torch.mm(h, w2.t(), out=b["out"]))

    for _ in range(3):
        step()
    T.collect()
    T.reset()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        step()
    s1.record()
    T.collect()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / steps
    flop = 2.0 * M * 2 * F * D + 2.0 * M * D * F
    out = {"workload": "dense FFN prefill, bf16 path (weight_dequant + bf16 GEMM per linear)",
           "ms_per_step": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    for name, fl in (("gemm_up_bf16", 2.0 * M * 2 * F * D), ("gemm_down_bf16", 2.0 * M * D * F)):
        us = T.avg_us(name)
        out[name] = {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1)}
    for name in ("dequant_w13", "dequant_w2"):
        out[name] = {"us": round(T.avg_us(name), 1)}
    return out


def bench_dense_ue8m0(dev, steps):
    """The dense step with power-of-two (ue8m0) scales throughout: the
    products apply the scales inside the matrix instruction."""
    st = setup_dense(dev, "ue8m0")
    ms, T = run_dense(st, steps, 3)
    M, D, F = st["M"], st["D"], st["F"]
    flop = 2.0 * M * 2 * F * D + 2.0 * M * D * F
    return {"workload": "dense FFN prefill with ue8m0 scales (same shapes)", "ms_per_step": round(ms, 4),
            "tflops": round(flop / (ms * 1e-3) / 1e12, 1), "kernels": dense_kernels(st, T)}


def bench_dense_unfused(dev, steps):
    """The dense step with the product, the SiLU gate and the quantisation of
    h as three kernels (bf16 [4096, 36864] written and read back between
    them), for comparison with the gated product."""
    st = setup_dense(dev, unfused=True)
    ms, T = run_dense(st, steps, 3)
    M, D, F = st["M"], st["D"], st["F"]
    flop = 2.0 * M * 2 * F * D + 2.0 * M * D * F
    return {"workload": "dense FFN prefill, up-projection, gate and quantisation as separate kernels",
            "ms_per_step": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
            "kernels": dense_kernels(st, T)}


def bench_dense_tp_shard(dev, steps, ranks=8):
    """One rank's share of the dense FFN step under `ranks`-way tensor
    parallelism ("DeepSeek-V3 Administrator & Developer Guide" 1.2, the
    column- and row-parallel linears, and 5.3, multi-GPU tensor-parallel
    inference): w1 and w3 split by output rows ([inter/ranks, dim] each),
    w2 by input columns ([dim, inter/ranks]); every rank quantises the full
    activations and produces a partial [M, dim] that an all-reduce (not
    timed here: one GPU) would sum.  Timed as one captured graph per step,
    like the headline."""
    F = I.WORKLOADS["dense_ffn"].dims["inter"] // ranks
    st = setup_dense(dev, inter=F)
    _, T = run_dense(st, steps, 3)
    g = capture(lambda: dense_step(st, NoTimer()))
    b = st["b"]
    check_replays(g, lambda: dense_step(st, NoTimer()), [b[n] for n in ("xq", "xs", "hq", "hs", "out")])
    ms = time_graph(g, steps, 3)
    M, D = st["M"], st["D"]
    flop = 2.0 * M * 2 * F * D + 2.0 * M * D * F
    return {"workload": f"dense FFN prefill, one rank of {ranks}-way tensor parallelism: act_quant [{M},{D}] -> "
                        f"gemm [w1;w3] {M}x{2 * F}x{D} with SiLU gate + act_quant -> gemm w2 {M}x{D}x{F}",
            "ms_per_step": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 1),
            "kernels": dense_kernels(st, T)}


def gemm_bytes(M, N, K):
    return M * K + N * K + 4 * (M * kb(K) + kb(N) * kb(K)) + 2 * M * N


def aq_bytes(M, K, inputs=1):
    return inputs * 2 * M * K + M * K + 4 * M * kb(K)


# ---- other workloads ----------------------------------------------------------------------

def bench_moe(dev, iters, ranks=1):
    """The routed-expert step on the device: routing of the gate's top-k
    choice, act_quant of the routed rows (gathered in the kernel), the grouped
    [w1;w3] product with the SiLU gate and act_quant in its epilogue, the
    grouped w2 product and the weighted bf16 combine into the token outputs.

    ranks > 1: one rank's share under expert parallelism with the experts
    assigned to ranks contiguously, as the checkpoint conversion shards them
    by expert index ("DeepSeek-V3 Administrator & Developer Guide" 1.1;
    rank 0 holds the first 256 / ranks): the
    same routing draw over all experts, routed with the local expert count,
    so pairs that chose another rank's expert get no row and are skipped by
    the combine (the all-reduce of the per-rank outputs is not timed: one
    GPU)."""
    d = I.WORKLOADS["moe"].dims
    E_all, D, F, Tk, k = d["experts"], d["dim"], d["inter"], d["tokens"], d["topk"]
    E = E_all // ranks
    idx_h, w_h = I.zipf_topk(Tk, E_all, k, d["zipf_s"])
    idx = torch.from_numpy(idx_h).to(dev)
    wts = torch.from_numpy(w_h.view(np.int16)).to(dev).view(torch.bfloat16)
    counts = np.bincount(idx_h.ravel(), minlength=E_all)[:E]
    M = Tk * k            # row buffers: at most every pair
    rows = int(counts.sum())  # rows routed to this rank's experts
    x = I.device_normal((Tk, D), seed=401, std=1.0, device=dev, dtype=torch.bfloat16)
    q13 = torch.empty((E, 2 * F, D), dtype=torch.uint8, device=dev)
    s13 = torch.empty((E, kb(2 * F), kb(D)), dtype=torch.float32, device=dev)
    q2 = torch.empty((E, D, F), dtype=torch.uint8, device=dev)
    s2 = torch.empty((E, kb(D), kb(F)), dtype=torch.float32, device=dev)
    for e in range(E):
        w = I.device_normal((2 * F, D), seed=10_000 + e, std=0.02, device=dev)
        q, s = ds.weight_quant(w)
        q13[e].copy_(q)
        s13[e].copy_(s)
        w = I.device_normal((D, F), seed=20_000 + e, std=0.02, device=dev)
        q, s = ds.weight_quant(w)
        q2[e].copy_(q)
        s2[e].copy_(s)
    del w, q, s
    lib = ds._lib.load()
    offd = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.zeros(M, dtype=torch.int32, device=dev)
    token_rows = torch.empty((Tk, k), dtype=torch.int32, device=dev)
    rws = torch.empty(lib.dsfp8_moe_route_workspace_bytes(Tk, k, E), dtype=torch.uint8, device=dev)
    xq = torch.empty((Tk, D), dtype=torch.uint8, device=dev)
    xs = ds.new_scales(Tk, kb(D), dev)
    # zero-filled: with ranks > 1 the rows past this rank's are never written
    hq = torch.zeros((M, F), dtype=torch.uint8, device=dev)
    hs = ds.new_scales(M, kb(F), dev).zero_()
    yr = torch.zeros((M, D), dtype=torch.bfloat16, device=dev)
    y = torch.empty((Tk, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(lib.dsfp8_grouped_gemm_workspace_bytes(E, M, D, D), dtype=torch.uint8, device=dev)
    T = Timer()

    def route():
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.dsfp8_moe_route(idx.data_ptr(), Tk, k, k, E, offd.data_ptr(), row_token.data_ptr(),
                                 token_rows.data_ptr(), rws.data_ptr(), rws.numel(), stream)
        assert st == 0, st

    def step(T=T):
        T.run("route", route)
        # The token rows are quantised once; the up-projection reads each
        # expert row through row_token.
        T.run("act_quant", lambda: ds.act_quant(x, out=(xq, xs)))
        T.run("grouped_up_gate",
              lambda: ds.grouped_gemm_silu_mul_act_quant(xq, xs, q13, s13, offd, out=(hq, hs), workspace=ws,
                                                         rows=row_token))
        T.run("grouped_down", lambda: ds.grouped_gemm(hq, hs, q2, s2, offd, out=yr, workspace=ws))
        T.run("combine", lambda: ds.moe_combine(yr, idx, wts, token_rows, out=y))

    for _ in range(2):
        step()
    T.collect()
    T.reset()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(iters):
        step()
    s1.record()
    T.collect()
    torch.cuda.synchronize()
    R = rows
    flop_up, flop_dn = 2.0 * R * 2 * F * D, 2.0 * R * D * F
    by_up = R * D + E * 2 * F * D + 4 * (R * kb(D) + E * kb(2 * F) * kb(D)) + R * F + 4 * R * kb(F)
    by_dn = R * F + E * D * F + 4 * (R * kb(F) + E * kb(D) * kb(F)) + 2 * R * D
    desc = I.WORKLOADS["moe"].desc
    if ranks > 1:
        desc += f"; one rank of {ranks}-way expert parallelism ({E} local experts)"
    res = {"workload": desc, "rows": R,
           "expert_rows": {"min": int(counts.min()), "median": float(np.median(counts)),
                           "max": int(counts.max())}}
    for name, fl, by in (("grouped_up_gate", flop_up, by_up), ("grouped_down", flop_dn, by_dn)):
        us = T.avg_us(name)
        roof_us = max(fl / (PEAK_FP8_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9)) * 1e6
        res[name] = {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1), "gbs": round(by / us / 1e3, 1),
                     "roofline_us": round(roof_us, 1), "frac_of_roofline": round(roof_us / us, 3), **T.spread(name)}
    # act_quant reads the token rows of x (2 B), writes e4m3 and scales;
    # combine reads the expert outputs and writes the token outputs (bf16).
    for name, by in (("act_quant", aq_bytes(Tk, D)), ("combine", 2 * R * D + 2 * Tk * D + Tk * k * 10)):
        us = T.avg_us(name)
        res[name] = {"us": round(us, 1), "gbs": round(by / us / 1e3, 1),
                     "frac_of_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 3), **T.spread(name)}
    res["route"] = {"us": round(T.avg_us("route"), 1), **T.spread("route")}
    res["step_us_eager"] = round(s0.elapsed_time(s1) * 1e3 / iters, 1)
    g = capture(lambda: step(NoTimer()))
    check_replays(g, lambda: step(NoTimer()), [offd, row_token, token_rows, xq, xs, hq, hs, yr, y])
    res["step_us"] = round(time_graph(g, iters, 2) * 1e3, 1)
    res["step_timing"] = "one captured HIP graph per step, replayed back to back"
    del g
    del q13, q2
    return res


def graph_time(fn, iters, reps=5):
    """GPU time per call of fn(i, stream) (which must only enqueue work on
    `stream`): `iters` calls are captured once into a HIP graph, and the graph
    is replayed `reps` times between one event pair, so host-side launch cost
    does not count."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stream = torch.cuda.current_stream().cuda_stream
        for i in range(iters):
            fn(i, stream)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * iters)


def bench_act_quant(dev, iters):
    """act_quant alone at the workloads' activation shapes: `iters` launches
    back to back from a captured graph (the kernel's steady-state rate; the
    per-launch event pair inside the step adds a few microseconds), rotating
    input/output sets of more than 512 MB in all (at most 64 sets) so the
    256 MB Infinity Cache cannot serve the large shapes' repeats."""
    lib = ds._lib.load()
    res = {}
    # the second quantisation of each FFN ([4096, 18432] dense, [32768, 2048]
    # routed) runs in the gated product's epilogue in the timed steps; the
    # plain kernel's rate at those shapes is listed as well
    for name, (M, K, fmt) in {"dense_ffn_input [4096,7168]": (4096, 7168, "fp32"),
                              "dense_ffn_hidden [4096,18432]": (4096, 18432, "fp32"),
                              "routed_rows [32768,7168]": (32768, 7168, "fp32"),
                              "routed_hidden [32768,2048]": (32768, 2048, "fp32"),
                              "decode [32,7168]": (32, 7168, "fp32"),
                              "ragged_ue8m0 [333,1000]": (333, 1000, "ue8m0")}.items():
        by = aq_bytes(M, K)
        nsets = int(min(64, max(1, np.ceil(600e6 / by))))
        sets = []
        for i in range(nsets):
            x = I.device_normal((M, K), seed=801 + i, std=1.0, device=dev, dtype=torch.bfloat16)
            sets.append((x, torch.empty((M, K), dtype=torch.uint8, device=dev), ds.new_scales(M, kb(K), dev)))
        code = 1 if fmt == "ue8m0" else 0

        def call(i, stream, sets=sets, M=M, K=K, code=code):
            x, y, s = sets[i % len(sets)]
            st = lib.dsfp8_act_quant(x.data_ptr(), M, K, K, y.data_ptr(), K, s.data_ptr(), s.stride(0), s.stride(1),
                                     code, stream)
            assert st == 0, st

        us = graph_time(call, max(iters, 2 * nsets))
        res[name] = {"us": round(us, 2), "gbs": round(by / us / 1e3, 1),
                     "frac_of_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 3), "buffer_sets_rotated": nsets}
        del sets
    return res


def bench_dequant(dev, iters):
    """weight_dequant of one [18432, 7168] weight per call, back to back from
    a captured graph, rotating four weight/output sets (1.6 GB) so the 256 MB
    Infinity Cache cannot serve repeats.  The fp32 and ue8m0 sets are
    allocated side by side and timed alternately, three times each (the
    median is reported), so that neither format inherits a different memory
    state from the other."""
    N, K = 18432, 7168
    res = {"workload": "weight_dequant e4m3 [18432, 7168] -> bf16", "buffer_sets_rotated": 4}
    lib = ds._lib.load()
    sets = {}
    for fmt in ("fp32", "ue8m0"):
        sets[fmt] = []
        for i in range(4):
            w = I.device_normal((N, K), seed=501 + i, std=0.02, device=dev)
            q, S = ds.weight_quant(w, fmt)
            del w
            sets[fmt].append((q, S, torch.empty((N, K), dtype=torch.bfloat16, device=dev)))

    def call(i, stream, fmt):
        q, S, out = sets[fmt][i % 4]
        st = lib.dsfp8_weight_dequant(q.data_ptr(), N, K, K, S.data_ptr(), S.stride(0), out.data_ptr(), K, stream)
        assert st == 0, st

    times = {"fp32": [], "ue8m0": []}
    for _ in range(3):
        for fmt in ("fp32", "ue8m0"):
            times[fmt].append(graph_time(lambda i, stream, fmt=fmt: call(i, stream, fmt), max(iters, 8)))
    del sets
    by = N * K * 3 + 4 * kb(N) * kb(K)
    for fmt in ("fp32", "ue8m0"):
        us = float(np.median(times[fmt]))
        res[fmt] = {"us": round(us, 1), "gbs": round(by / us / 1e3, 1),
                    "frac_of_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 3),
                    "us_runs": [round(t, 1) for t in times[fmt]]}
    return res


def bench_small_gemm(dev, iters, name, M, N, K, fmt, outlier):
    """act_quant + gemm on a small shape, rotating weight copies (> 512 MB in
    total) so that neither the L2 nor the 256 MB Infinity Cache serves them."""
    x = I.device_normal((M, K), seed=601, std=1.0, device=dev, dtype=torch.bfloat16)
    if outlier:
        cols = torch.from_numpy(np.random.default_rng(0).choice(K, int(round(0.01 * K)), replace=False)).to(dev)
        x[:, cols] *= 20
    copies = max(2, int(np.ceil(600e6 / (N * K))))
    ws = []
    for i in range(copies):
        w = I.device_normal((N, K), seed=700 + i, std=0.02, device=dev)
        ws.append(ds.weight_quant(w, fmt))
    del w
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = ds.new_scales(M, kb(K), dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for i in range(copies + 3):
        ds.act_quant(x, fmt, out=(xq, xs))
        ds.gemm(xq, xs, *ws[i % copies], out=out, scale_fmt=fmt)
    torch.cuda.synchronize()

    # Kernels this short run faster than the host can launch them through the
    # binding, so `iters` launches (through the C ABI, preallocated buffers,
    # weight copies rotated) are captured once into a HIP graph and the graph
    # is replayed between one event pair: the time is the GPU's.
    lib = ds._lib.load()
    code = 1 if fmt == "ue8m0" else 0
    wsb = lib.dsfp8_gemm_workspace_bytes(M, N, K)
    wsbuf = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)  # zero-filled once (arrival counters)
    srs, sks = xs.stride(0), xs.stride(1)

    def aq_call(i, stream):
        st = lib.dsfp8_act_quant(x.data_ptr(), M, K, K, xq.data_ptr(), K, xs.data_ptr(), srs, sks, code, stream)
        assert st == 0, st

    def gemm_call(i, stream):
        q, S = ws[i % copies]
        st = lib.dsfp8_gemm(xq.data_ptr(), K, xs.data_ptr(), srs, sks, q.data_ptr(), K, S.data_ptr(), S.stride(0),
                            out.data_ptr(), N, M, N, K, code, wsbuf.data_ptr() if wsb else None, wsb, stream)
        assert st == 0, st

    def timed(fn):
        return graph_time(fn, iters)

    a_us = timed(aq_call)
    g_us = timed(gemm_call)
    fl, by = 2.0 * M * N * K, gemm_bytes(M, N, K)
    roof_us = max(fl / (PEAK_FP8_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9)) * 1e6
    return {"workload": name, "gemm": {"us": round(g_us, 2), "tflops": round(fl / g_us / 1e6, 2),
                                       "gbs": round(by / g_us / 1e3, 1), "roofline_us": round(roof_us, 2),
                                       "frac_of_roofline": round(roof_us / g_us, 3)},
            "act_quant": {"us": round(a_us, 2), "gbs": round(aq_bytes(M, K) / a_us / 1e3, 1)},
            "weight_copies_rotated": copies, "timing": "HIP graph of back-to-back launches"}


def bench_grouped_classes(dev, reps):
    """The routed-expert products (dim 7168, inter 2048, fp32 scales) with
    uniform expert sizes that each fill one tile class of the grouped kernel:
    256 experts of 41 rows (64-row tiles), 256 of 100 rows (128-row tiles)
    and 32 of 1024 rows (256-row tiles).  Per launch: time, FP8 rate and the
    rate at which the experts' weights stream; for per-class counters."""
    d = I.WORKLOADS["moe"].dims
    D, F = d["dim"], d["inter"]
    cfgs = [("64-row tiles: 256 experts x 41 rows", 256, 41), ("128-row tiles: 256 experts x 100 rows", 256, 100),
            ("256-row tiles: 32 experts x 1024 rows", 32, 1024)]
    EM = max(E for _, E, _ in cfgs)
    q13 = torch.empty((EM, 2 * F, D), dtype=torch.uint8, device=dev)
    s13 = torch.empty((EM, kb(2 * F), kb(D)), dtype=torch.float32, device=dev)
    q2 = torch.empty((EM, D, F), dtype=torch.uint8, device=dev)
    s2 = torch.empty((EM, kb(D), kb(F)), dtype=torch.float32, device=dev)
    for e in range(EM):
        q, s = ds.weight_quant(I.device_normal((2 * F, D), seed=10_000 + e, std=0.02, device=dev))
        q13[e].copy_(q)
        s13[e].copy_(s)
        q, s = ds.weight_quant(I.device_normal((D, F), seed=20_000 + e, std=0.02, device=dev))
        q2[e].copy_(q)
        s2[e].copy_(s)
    del q, s
    res = {}
    for name, E, r in cfgs:
        M = E * r
        xq, xs = ds.act_quant(I.device_normal((M, D), seed=401, std=1.0, device=dev, dtype=torch.bfloat16))
        offd = (torch.arange(E + 1, dtype=torch.int32, device=dev) * r).contiguous()
        hq = torch.empty((M, F), dtype=torch.uint8, device=dev)
        hs = ds.new_scales(M, kb(F), dev)
        yr = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
        lib = ds._lib.load()
        ws = torch.empty(lib.dsfp8_grouped_gemm_workspace_bytes(E, M, D, D), dtype=torch.uint8, device=dev)
        T = Timer()
        a13, a2 = q13[:E], q2[:E]
        for it in range(reps + 1):
            T.run("up", lambda: ds.grouped_gemm_silu_mul_act_quant(xq, xs, a13, s13[:E], offd, out=(hq, hs),
                                                                   workspace=ws))
            T.run("down", lambda: ds.grouped_gemm(hq, hs, a2, s2[:E], offd, out=yr, workspace=ws))
            T.collect()
            if it == 0:
                T.reset()
        out = {}
        for k, fl, wb in (("up", 2.0 * M * 2 * F * D, E * 2 * F * D), ("down", 2.0 * M * D * F, E * D * F)):
            us = T.avg_us(k)
            out[k] = {"us": round(us, 1), "tflops": round(fl / us / 1e6, 1), "weight_gbs": round(wb / us / 1e3, 1)}
        res[name] = out
        del xq, xs, hq, hs, yr, ws
    return res


# ---- CPU baseline ---------------------------------------------------------------------------

def cpu_baseline(budget_s=15.0):
    """The CPU oracle on a bounded sample of the dense FFN step.

    Sample: chunks of 128 token rows (eight distinct chunks, cycled); 1536
    rows each of w1 and w3 (3072 outputs of the up-projection) over the full
    K = 7168; SiLU gate; 1536 rows of w2 over the first 1536 of its K columns.
    Weights and activations are drawn and quantised on the host before
    timing; each timed chunk runs act_quant, the up product, the gate,
    act_quant of h and the down product, all in the oracle.  Chunks run until
    ``budget_s`` seconds of oracle time have passed.  Reported as the sample's
    GEMM flop per second.  ``cores`` is the number of threads the oracle
    actually used (the BLAS pool that runs its fp64 products; its quantisers
    are single-threaded NumPy); ``affinity_cpus`` is the number of host CPUs
    the process may run on.
    """
    import threadpoolctl
    from oracle import gemm as G
    from oracle import glue
    from oracle import quant as Q
    from oracle.formats import f32_to_bf16

    Ms, D, Fs, n_chunks = 128, 7168, 1536, 8
    xs = [I.activations((Ms, D), I.DENSE_FFN, 900 + c) for c in range(n_chunks)]
    w13 = Q.weight_quant(I.weights_f32((2 * Fs, D), I.DENSE_FFN, 901))
    w2 = Q.weight_quant(I.weights_f32((Fs, Fs), I.DENSE_FFN, 902))
    dt, done = 0.0, 0
    while dt < budget_s:
        x = xs[done % n_chunks]
        t0 = time.perf_counter()
        a, a_s = Q.act_quant(x)
        h13 = f32_to_bf16(G.gemm(a, a_s, *w13))
        h = glue.silu_mul(h13[:, :Fs], h13[:, Fs:])
        hq, hs = Q.act_quant(h)
        _ = G.gemm(hq, hs, *w2)
        dt += time.perf_counter() - t0
        done += 1
    flop = done * (2.0 * Ms * 2 * Fs * D + 2.0 * Ms * Fs * Fs)
    try:
        blas = threadpoolctl.threadpool_info()
        threads = max([b.get("num_threads", 1) for b in blas] + [1])
    except Exception:
        threads = 1
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "blas_threads": int(threads), "affinity_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": round(dt, 2), "chunks": done,
            "sample": f"dense FFN step on {done} chunks of 128 tokens x (3072 up-projection outputs, K=7168) "
                      "+ SiLU gate + (1536 down outputs, K=1536); fp64 products through NumPy BLAS, "
                      "quantisers in NumPy"}


# ---- traffic (from the committed rocprofv3 counter summary) -----------------------------------

def gemm_source_digest():
    h = hashlib.sha256()
    for f in ("gemm.hip", "device.h"):
        with open(os.path.join(ROOT, "block_scaled_fp8_act_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the gated up-projection, from the counter summary
    in profiles/, or None if it was taken on a different GEMM source."""
    path = os.path.join(ROOT, "profiles", "gemm_dense_ffn_up_gate_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_digest:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != gemm_source_digest():
        return None
    return float(t.group(1))


# ---- main --------------------------------------------------------------------------------------

def only(kernel, reps, dev, fmt="fp32"):
    """Run one kernel of the dense step `reps` times (for counter collection),
    with fp32 or ue8m0 scales throughout."""
    if kernel == "dense_tp8_rank":
        print(json.dumps({"only": kernel, "reps": reps, "result": bench_dense_tp_shard(dev, reps)}))
        return
    if kernel == "routed_experts":
        print(json.dumps({"only": kernel, "reps": reps, "result": bench_moe(dev, reps)}))
        return
    if kernel == "routed_experts_ep8_rank":
        print(json.dumps({"only": kernel, "reps": reps, "result": bench_moe(dev, reps, ranks=8)}))
        return
    if kernel == "grouped_classes":
        print(json.dumps({"only": kernel, "reps": reps, "result": bench_grouped_classes(dev, reps)}))
        return
    if kernel == "small_products":
        res = {"decode_qa": bench_small_gemm(dev, reps, "decode MLA q_a: 32x1536x7168", 32, 1536, 7168, "fp32", True),
               "ragged_ue8m0": bench_small_gemm(dev, reps, "ragged ue8m0: 333x2500x1000", 333, 2500, 1000, "ue8m0",
                                                False)}
        print(json.dumps({"only": kernel, "reps": reps, "result": res}))
        return
    if kernel == "copy":
        # calibration: a plain 1 GiB device-to-device copy (1 GiB read, 1 GiB written)
        src = torch.ones(256 * 1024 * 1024, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(reps):
            dst.copy_(src)
    else:
        st = setup_dense(dev, fmt, unfused=kernel in ("gemm_up", "silu_mul_act_quant"))
        T = Timer()
        b, F = st["b"], st["F"]
        fns = {
            "act_quant": lambda: ds.act_quant(b["x"], fmt, out=(b["xq"], b["xs"])),
            "gemm_up_gate": lambda: ds.gemm_silu_mul_act_quant(b["xq"], b["xs"], b["q13"], b["s13"], fmt,
                                                               out=(b["hq"], b["hs"])),
            "gemm_up": lambda: ds.gemm(b["xq"], b["xs"], b["q13"], b["s13"], out=b["h13"], scale_fmt=fmt),
            "silu_mul_act_quant": lambda: ds.silu_mul_act_quant(b["h13"][:, :F], b["h13"][:, F:], fmt,
                                                                out=(b["hq"], b["hs"])),
            "gemm_down": lambda: ds.gemm(b["hq"], b["hs"], b["q2"], b["s2"], out=b["out"], scale_fmt=fmt),
        }
        if kernel == "weight_dequant":
            # w1 of the dense FFN, [18432, 7168] (the first F rows of the stacked [w1; w3])
            dq = torch.empty((F, b["q13"].shape[1]), dtype=torch.bfloat16, device=dev)
            fns[kernel] = lambda: ds.weight_dequant(b["q13"][:F], b["s13"][:F // 128], out=dq)
        dense_step(st, T)  # produce valid inputs for every stage
        torch.cuda.synchronize()
        for _ in range(reps):
            fns[kernel]()
    torch.cuda.synchronize()
    print(json.dumps({"only": kernel, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline step only (no other workloads, no CPU baseline)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["act_quant", "weight_dequant", "gemm_up_gate", "gemm_up", "silu_mul_act_quant", "gemm_down",
                                       "copy", "routed_experts", "small_products", "grouped_classes", "dense_tp8_rank",
                                       "routed_experts_ep8_rank"],
                    help="run one kernel of the dense step (or the routed-expert step) --reps times and exit "
                         "(for rocprofv3)")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--fmt", choices=["fp32", "ue8m0"], default="fp32", help="scale format for --only")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X).", file=sys.stderr)
        sys.exit(2)
    ds._lib.load()
    dev = torch.device("cuda:0")
    if args.only:
        only(args.only, args.reps, dev, args.fmt)
        return
    props = torch.cuda.get_device_properties(dev)

    st = setup_dense(dev)
    eager_ms, T = run_dense(st, args.steps, args.warmup)
    # The step as one captured graph (same kernels, no host launch gaps),
    # checked against the eager step before it is timed.
    g = capture(lambda: dense_step(st, NoTimer()))
    b = st["b"]
    check_replays(g, lambda: dense_step(st, NoTimer()), [b[n] for n in ("xq", "xs", "hq", "hs", "out")])
    step_ms = time_graph(g, args.steps, args.warmup)

    M, D, F = st["M"], st["D"], st["F"]
    fl_up, fl_dn = 2.0 * M * 2 * F * D, 2.0 * M * D * F
    total_flop = fl_up + fl_dn
    value = total_flop / (step_ms * 1e-3) / 1e12
    k = dense_kernels(st, T)
    up_us = T.avg_us("gemm_up_gate")
    achieved = fl_up / up_us / 1e6
    traffic = recorded_traffic()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "ms_per_step_eager": round(eager_ms, 4),
        "step_timing": "one captured HIP graph per step, replayed back to back (eager launches: ms_per_step_eager)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights quantised to e4m3 with 128x128 scales)",
        "config": {"workload": "dense FFN prefill: act_quant [4096,7168] -> gemm [w1;w3] 4096x36864x7168 with "
                               "SiLU gate + act_quant epilogue -> gemm w2 4096x7168x18432",
                   "tokens": M, "dim": D, "inter": F, "block": 128},
        "roofline": {"bound": "mfma", "kernel": "gemm_up_gate 4096x36864x7168 (gated epilogue)",
                     "achieved": round(achieved, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic, "avg_launch_us": round(up_us, 1)},
        "kernels": k,
        "act_quant_gbs": None,
        "act_quant_gbs_in_step": k["act_quant"]["gbs"],
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    aq = bench_act_quant(dev, 50)
    line["act_quant"] = aq
    line["act_quant_gbs"] = aq["dense_ffn_input [4096,7168]"]["gbs"]
    if not args.quick:
        others = {}
        del st
        torch.cuda.empty_cache()
        others["dense_ffn_ue8m0"] = bench_dense_ue8m0(dev, 20)
        torch.cuda.empty_cache()
        others["dense_ffn_unfused"] = bench_dense_unfused(dev, 20)
        torch.cuda.empty_cache()
        others["dense_ffn_bf16_path"] = bench_bf16_path(dev, 10)
        torch.cuda.empty_cache()
        others["dense_ffn_tp8_rank"] = bench_dense_tp_shard(dev, 20)
        torch.cuda.empty_cache()
        others["routed_experts"] = bench_moe(dev, 10)
        others["routed_experts_ep8_rank"] = bench_moe(dev, 10, ranks=8)
        others["weight_dequant"] = bench_dequant(dev, 20)
        others["decode_qa"] = bench_small_gemm(dev, 50, "decode MLA q_a: 32x1536x7168", 32, 1536, 7168, "fp32", True)
        others["ragged_ue8m0"] = bench_small_gemm(dev, 50, "ragged ue8m0: 333x2500x1000", 333, 2500, 1000,
                                                  "ue8m0", False)
        others["decode_one_token"] = bench_small_gemm(dev, 20, "one-token decode of the dense FFN's w1: 1x18432x7168",
                                                      1, 18432, 7168, "fp32", False)
        line["other_workloads"] = others
    if not args.quick and not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))


if __name__ == "__main__":
    main()

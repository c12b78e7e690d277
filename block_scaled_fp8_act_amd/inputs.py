"""Seeded synthetic inputs for the FP8 linear layer workloads.

This module draws random numbers and arranges them into the shapes of the
DeepSeek-V3 projections; it contains none of the quantisation or product
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
it.  Every generator is keyed by ``(seed, config id, tensor id)`` through
``numpy.random.SeedSequence``.

Activations are N(0, 1) in fp32 rounded to bf16 by torch's own cast; weights
are N(0, 0.02) in fp32 (they become e4m3 + block scales through the weight
quantiser).  Expert routing for the routed-expert workload draws, for every
token, 8 distinct experts out of 256 with probabilities proportional to
rank^-1.1 (Gumbel top-k over log-probabilities, i.e. weighted sampling without
replacement), the ranks being assigned to experts by a seeded permutation.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

SEED = 0

# Config ids (used as the second SeedSequence word).
TINY, DECODE_QA, DENSE_FFN, MOE, RAGGED = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    cid: int
    desc: str
    dims: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", TINY, "x bf16 [16,512], W e4m3 [256,512]", dict(M=16, K=512, N=256)),
    "decode_qa": Workload("decode_qa", DECODE_QA,
                          "MLA q_a projection at decode: x bf16 [32,7168] with 1% outlier channels x20, "
                          "W e4m3 [1536,7168]", dict(M=32, K=7168, N=1536, outlier_frac=0.01, outlier_scale=20.0)),
    "dense_ffn": Workload("dense_ffn", DENSE_FFN,
                          "dense FFN prefill: x bf16 [4096,7168], w1/w3 [18432,7168], w2 [7168,18432]",
                          dict(M=4096, dim=7168, inter=18432)),
    "moe": Workload("moe", MOE,
                    "routed experts: 4096 tokens top-8 of 256 experts (Zipf 1.1), dim 7168, inter 2048",
                    dict(tokens=4096, topk=8, experts=256, dim=7168, inter=2048, zipf_s=1.1)),
    "ragged": Workload("ragged", RAGGED,
                       "ragged ue8m0: x bf16 [333,1000], W e4m3 [2500,1000]; dequant of [18432,7168]",
                       dict(M=333, K=1000, N=2500, dqN=18432, dqK=7168)),
}


def rng(cid, tensor, seed=SEED):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, tensor])))


def to_bf16_bits(x32):
    """bf16 bit patterns (uint16) of fp32 values, rounded by torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def activations(shape, cid, tensor, std=1.0, outlier_frac=0.0, outlier_scale=20.0, seed=SEED):
    """bf16 activations (uint16 bits): N(0, std^2), optionally with a random
    ``outlier_frac`` of the channels (last dim) scaled by ``outlier_scale``
    before rounding."""
    g = rng(cid, tensor, seed)
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outlier_frac > 0:
        C = shape[-1]
        n_out = int(round(outlier_frac * C))
        cols = g.choice(C, size=n_out, replace=False)
        x[..., cols] *= np.float32(outlier_scale)
    return to_bf16_bits(x)


def weights_f32(shape, cid, tensor, std=0.02, seed=SEED):
    """Real-valued weights, N(0, std^2) in fp32."""
    g = rng(cid, tensor, seed)
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def device_normal(shape, seed, std, device, dtype=torch.float32):
    """N(0, std^2) drawn on the device by torch's seeded generator (used for
    inputs too large to draw on the host, e.g. 11 GB of expert weights)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def zipf_topk(tokens, experts, topk, s, cid=MOE, seed=SEED):
    """Synthetic gate output: per token, ``topk`` distinct experts drawn with
    Zipf(s) popularity (Gumbel top-k over log-popularity), and positive routing
    weights (uniform draws normalised to sum 1 per token, times 2.5, the
    routing scale of the 671B configuration) rounded to bf16.

    Returns ``(indices int32 [tokens, topk], weights_bits uint16 [tokens, topk])``.
    """
    g = rng(cid, 100, seed)
    perm = g.permutation(experts)                  # expert perm[r] has rank r+1
    logp = np.empty(experts, dtype=np.float64)
    logp[perm] = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(g.random((tokens, experts))))
    keys = logp[None, :] + gumbel
    choice = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]   # distinct experts per token
    w = g.uniform(0.05, 1.0, (tokens, topk))
    w = 2.5 * w / w.sum(axis=1, keepdims=True)
    return choice.astype(np.int32), to_bf16_bits(w.astype(np.float32))


def random_offsets(total, experts, cid, tensor, empty_frac=0.25, seed=SEED):
    """Random non-decreasing expert offsets with some empty experts (tests)."""
    g = rng(cid, tensor, seed)
    w = g.random(experts)
    w[g.random(experts) < empty_frac] = 0.0
    if w.sum() == 0:
        w[0] = 1.0
    counts = np.floor(w / w.sum() * total).astype(np.int64)
    counts[int(np.argmax(w))] += total - counts.sum()
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets

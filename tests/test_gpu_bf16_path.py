"""GPU parity of the pages' default bf16 path for a linear layer
("DeepSeek-V3 Administrator & Developer Guide" 6.3: with the default
gemm_impl, each FP8 weight is dequantised to bf16 with weight_dequant and the
layer runs as a bf16 product; 6.6 contrasts it with the FP8 product).

The step is the one bench.py times as its comparison: dsfp8_weight_dequant
into a bf16 buffer, then the vendor bf16 GEMM through torch.mm with the
weight's transposed view, C = x W_hat^T in bf16.  The oracle is the fp64
product of the same bf16 x and the oracle's weight_dequant (bit-exact bf16
weights): the only differences are the GEMM's fp32 accumulation and its bf16
output rounding, so each element must lie within

    |C - C_ref| <= ulp_bf16(C_ref) + 1e-4 * (|x| |W_hat|^T)

(one bf16 unit covers the output rounding with room for a tie on the
other side; 1e-4 |x||W|^T is far above what fp32 accumulation over
K <= 18432 can lose, about K * 2^-24 < 1.1e-3 in the worst case, 2^-24
times sqrt(K) typically), together with the product tolerance of the FP8
path (gpu_helpers).  Shapes: the tiny linear, the decode q_a projection
with outlier channels, the ragged shape with ue8m0 weight scales, and the
dense FFN's stacked [w1; w3] at full size on sampled rows and columns.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import quant as Q

from gpu_helpers import check_product, dev_bf16, dev_f32, dev_u8, host_bits16

pytestmark = pytest.mark.gpu


def bf16_ulp(v):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def bf16_linear(x_d, q_d, S_d, w_buf=None, out=None):
    """The comparison step: weight_dequant, then a bf16 product with W^T."""
    w = ds.weight_dequant(q_d, S_d, out=w_buf)
    if out is None:
        return torch.mm(x_d, w.t())
    return torch.mm(x_d, w.t(), out=out)


def check_elementwise(C_bits, x_bits, w_bits, what):
    X = F.bf16_to_f32(x_bits).astype(np.float64)
    W = F.bf16_to_f32(w_bits).astype(np.float64)
    ref = X @ W.T
    C = F.bf16_to_f32(C_bits).astype(np.float64)
    bound = bf16_ulp(ref) + 1e-4 * (np.abs(X) @ np.abs(W).T)
    bad = np.abs(C - ref) > bound
    assert not bad.any(), f"{what}: outside the bf16 bound at {np.argwhere(bad)[:5].tolist()}"
    check_product(C_bits, ref, X, W, what)


@pytest.mark.parametrize("M,N,K,ue8m0,outliers", [
    (16, 256, 512, False, False),      # tiny linear
    (32, 1536, 7168, False, True),     # decode MLA q_a projection, 1% outlier channels x20
    (333, 2500, 1000, True, False),    # ragged, ue8m0 weight scales, partial blocks
])
def test_bf16_linear(M, N, K, ue8m0, outliers):
    cid = I.DECODE_QA if outliers else (I.RAGGED if ue8m0 else I.TINY)
    x = I.activations((M, K), cid, 7, outlier_frac=0.01 if outliers else 0.0)
    q, S = Q.weight_quant(I.weights_f32((N, K), cid, 8), ue8m0=ue8m0)
    C = bf16_linear(dev_bf16(x), dev_u8(q), dev_f32(S))
    torch.cuda.synchronize()
    check_elementwise(host_bits16(C), x, Q.weight_dequant(q, S), f"{M}x{N}x{K}")


def test_bf16_linear_dense_ffn_size_sampled():
    """The dense FFN's stacked [w1; w3] (36864 x 7168) on 4096 tokens, with
    device-drawn inputs, as bench.py runs it (preallocated weight buffer and
    output): sampled rows against the oracle on sampled 128-column blocks,
    and the dequantised weight bit-exact on those blocks."""
    M, K, N = 4096, 7168, 2 * 18432
    xf = I.device_normal((M, K), seed=70, std=1.0, device="cuda", dtype=torch.bfloat16)
    wf = I.device_normal((N, K), seed=71, std=0.02, device="cuda")
    q, S = ds.weight_quant(wf)
    del wf
    w_buf = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    bf16_linear(xf, q, S, w_buf=w_buf, out=out)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(70).choice(M, 32, replace=False))
    rows[-1] = M - 1
    blocks = sorted({0, N // 128 - 1, *np.random.default_rng(71).choice(N // 128, 4, replace=False).tolist()})
    rt = torch.from_numpy(rows).cuda()
    xr = xf[rt].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    for j in blocks:
        sel = slice(j * 128, (j + 1) * 128)
        qj = q[sel].cpu().numpy()
        Sj = S[j:j + 1].cpu().numpy()
        wj = Q.weight_dequant(qj, Sj)
        assert np.array_equal(host_bits16(w_buf[sel]), wj), f"weight_dequant block {j}"
        check_elementwise(host_bits16(out[rt, sel]), xr, wj, f"dense FFN block {j}")

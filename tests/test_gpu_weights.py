"""GPU parity of the weight block quantiser and of weight_dequant (bit-exact).

weight_dequant: Admin Guide 8.5.2 (fp32 product, then bf16); the stored format
with its zero padding: DocSearch item 3.  Shapes: ragged [2500, 1000] with
ue8m0 scales, odd edges, the [18432, 7168] weight of the dense FFN with fp32
and with ue8m0 scales (sampled rows plus a full [2048, 7168] slice), and
strided / unaligned storage.
"""

import numpy as np
import pytest
import torch

import block_scaled_fp8_act_amd as ds
from block_scaled_fp8_act_amd import inputs as I
from oracle import formats as F
from oracle import quant as Q

from gpu_helpers import dev_f32, dev_u8, host_bits16, host_f32_bits, host_u8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,fmt", [(256, 512, "fp32"), (2500, 1000, "ue8m0"), (300, 260, "fp32"),
                                     (1, 1, "fp32"), (129, 7, "ue8m0")])
def test_weight_quant_fp32_input(N, K, fmt):
    w = I.weights_f32((N, K), I.RAGGED, N + K)
    q, S = ds.weight_quant(dev_f32(w), fmt)
    torch.cuda.synchronize()
    qr, Sr = Q.weight_quant(w, ue8m0=(fmt == "ue8m0"))
    assert np.array_equal(host_f32_bits(S), Sr.view(np.uint32))
    assert np.array_equal(host_u8(q), qr)


def test_weight_quant_bf16_input():
    wb = I.activations((384, 640), I.TINY, 9, std=0.02)
    wd = torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).cuda()
    q, S = ds.weight_quant(wd)
    torch.cuda.synchronize()
    qr, Sr = Q.weight_quant(F.bf16_to_f32(wb))
    assert np.array_equal(host_f32_bits(S), Sr.view(np.uint32))
    assert np.array_equal(host_u8(q), qr)


def test_weight_quant_zero_block():
    w = I.weights_f32((256, 256), I.TINY, 3)
    w[128:, :128] = 0.0
    q, S = ds.weight_quant(dev_f32(w))
    torch.cuda.synchronize()
    qr, Sr = Q.weight_quant(w)
    assert np.array_equal(host_f32_bits(S), Sr.view(np.uint32))
    assert np.array_equal(host_u8(q), qr)


def _stored_weight(N, K, fmt, seed):
    return Q.weight_quant(I.weights_f32((N, K), I.RAGGED, seed), ue8m0=(fmt == "ue8m0"))


@pytest.mark.parametrize("N,K,fmt", [(2500, 1000, "ue8m0"), (260, 300, "fp32"), (2048, 7168, "fp32"),
                                     (2048, 7168, "ue8m0"), (1, 1, "fp32"), (130, 16, "fp32"),
                                     # workgroups fitted to K: 128 threads, 144 (last one partial), 240 x 5
                                     (100, 2048, "fp32"), (300, 4112, "fp32"), (200, 18432, "ue8m0")])
def test_weight_dequant(N, K, fmt):
    q, S = _stored_weight(N, K, fmt, 40 + N)
    out = ds.weight_dequant(dev_u8(q), dev_f32(S))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits16(out), Q.weight_dequant(q, S))


@pytest.mark.parametrize("fmt", ["fp32", "ue8m0"])
def test_weight_dequant_full_size_sampled(fmt):
    # The [18432, 7168] weight, quantised on the GPU from fp32 drawn on the
    # device; sampled block-rows of the quantised weight, of its scales and of
    # the dequantised output are checked against the oracle run on the same
    # fp32 source rows.
    N, K = 18432, 7168
    w = I.device_normal((N, K), seed=1234, std=0.02, device="cuda")
    q, S = ds.weight_quant(w, fmt)
    out = ds.weight_dequant(q, S)
    torch.cuda.synchronize()
    for bi in (0, 77, 143):
        rows = slice(bi * 128, (bi + 1) * 128)
        wr = w[rows].cpu().numpy()
        qr, Sr = Q.weight_quant(wr, ue8m0=(fmt == "ue8m0"))
        assert np.array_equal(host_u8(q[rows]), qr)
        assert np.array_equal(host_f32_bits(S[bi:bi + 1]), Sr.view(np.uint32))
        assert np.array_equal(host_bits16(out[rows]), Q.weight_dequant(qr, Sr))


def test_weight_dequant_strided_and_unaligned():
    q, S = _stored_weight(300, 512, "fp32", 5)
    big = np.zeros((300, 600), np.uint8)
    big[:, 8:520] = q
    qd = dev_u8(big)[:, 8:520]              # ld 600, 8-byte aligned start: scalar path
    out = ds.weight_dequant(qd, dev_f32(S))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits16(out), Q.weight_dequant(q, S))

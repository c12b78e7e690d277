"""The seeded input generators: determinism, shapes and routing structure (CPU only)."""

import numpy as np

from block_scaled_fp8_act_amd import inputs as I


def test_deterministic_and_keyed():
    a = I.activations((8, 256), I.TINY, 0)
    b = I.activations((8, 256), I.TINY, 0)
    c = I.activations((8, 256), I.TINY, 1)
    assert a.dtype == np.uint16 and np.array_equal(a, b) and not np.array_equal(a, c)


def test_outlier_channels():
    x = I.activations((32, 7168), I.DECODE_QA, 0, outlier_frac=0.01, outlier_scale=20.0)
    v = (x.astype(np.uint32) << 16).view(np.float32)
    col_rms = np.sqrt((v.astype(np.float64) ** 2).mean(axis=0))
    assert np.sum(col_rms > 8) == 72


def test_zipf_topk_structure():
    idx, w = I.zipf_topk(4096, 256, 8, 1.1)
    assert idx.shape == (4096, 8) and idx.dtype == np.int32 and w.shape == (4096, 8) and w.dtype == np.uint16
    assert idx.min() >= 0 and idx.max() < 256
    # each token picks 8 distinct experts
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])
    # skewed popularity: the largest expert is far above the median
    counts = np.bincount(idx.ravel(), minlength=256)
    assert counts.sum() == 32768 and counts.max() > 20 * np.median(counts)
    # positive bf16 weights summing to about 2.5 per token
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(wf > 0) and np.allclose(wf.sum(axis=1), 2.5, rtol=2e-2)


def test_random_offsets():
    off = I.random_offsets(1000, 12, 9, 0)
    assert off[0] == 0 and off[-1] == 1000 and np.all(np.diff(off) >= 0)

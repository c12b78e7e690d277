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


def test_zipf_routing_structure():
    tok, off, counts = I.zipf_routing(4096, 256, 8, 1.1)
    assert off[0] == 0 and off[-1] == 4096 * 8 and np.all(np.diff(off) >= 0)
    assert counts.max() <= 4096 and counts.sum() == 32768
    # each token picks 8 distinct experts
    pairs = set()
    for e in range(256):
        for t in tok[off[e]:off[e + 1]]:
            assert (t, e) not in pairs
            pairs.add((t, e))
    assert len(pairs) == 32768
    # skewed popularity: the largest expert is far above the median
    assert counts.max() > 20 * np.median(counts)


def test_random_offsets():
    off = I.random_offsets(1000, 12, 9, 0)
    assert off[0] == 0 and off[-1] == 1000 and np.all(np.diff(off) >= 0)

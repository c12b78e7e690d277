"""The grouped products' workspace bound, on the host (no GPU).

The merged grouped launch sizes its grid, and its tile plan in the workspace,
from E, M and N alone, since the per-expert row counts live on the device.
The workspace query returns the schedule (3(E+1) int32, rounded up to 256
bytes) followed by one 16-byte plan entry per workgroup, so the number of
workgroups it provides for can be read back from it.  Here that number is
checked against the workgroups the launch actually needs for many expert-size
lists: each expert's rows split into tiles of 64, 128 or 256 rows (a large
expert's remainder of at most 128 rows goes to the smaller class of its own
height), each class's tiles times the column tiles rounded up to chunks of 8.
"""

import numpy as np
import pytest

from block_scaled_fp8_act_amd import _lib

H0, H1, H2 = 64, 128, 256


def class_tiles(n):
    """Row tiles of each class for an expert of n rows."""
    t = [0, 0, 0]
    if n == 0:
        return t
    if n <= H0:
        t[0] = 1
    elif n <= H1:
        t[1] = 1
    else:
        full, rem = divmod(n, H2)
        if full > 0 and 0 < rem <= H1:
            t[2] = full
            t[0 if rem <= H0 else 1] = 1
        else:
            t[2] = -(-n // H2)
    return t


def workgroups_needed(counts, tn):
    t = np.zeros(3, np.int64)
    for n in counts:
        t += class_tiles(int(n))
    return 8 * sum((int(x) * tn + 7) // 8 for x in t)


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(_lib.LIB_PATH):
        from block_scaled_fp8_act_amd import build
        build.build()
    return _lib.load()


def provided(lib, E, M, N):
    sched = (3 * (E + 1) * 4 + 255) // 256 * 256
    total = lib.dsfp8_grouped_gemm_workspace_bytes(E, M, N, 128)
    assert (total - sched) % 16 == 0
    return (total - sched) // 16


def test_class_split_examples():
    assert class_tiles(0) == [0, 0, 0]
    assert class_tiles(64) == [1, 0, 0] and class_tiles(65) == [0, 1, 0]
    assert class_tiles(129) == [0, 0, 1] and class_tiles(256) == [0, 0, 1]
    assert class_tiles(300) == [1, 0, 1] and class_tiles(384) == [0, 1, 1]
    assert class_tiles(385) == [0, 0, 2] and class_tiles(512) == [0, 0, 2]


def test_bound_covers_every_expert_size_list(lib):
    rng = np.random.default_rng(0)
    tight = 0
    for trial in range(4000):
        E = int(rng.integers(1, 300))
        N = 256 * int(rng.integers(1, 40)) - int(rng.integers(0, 2)) * int(rng.integers(0, 255))
        tn = -(-N // 256)
        kind = trial % 5
        if kind == 0:
            counts = rng.integers(0, 400, E)
        elif kind == 1:
            counts = rng.choice([0, 1, 64, 65, 128, 129, 256, 257, 384, 385, 512, 513], E)
        elif kind == 2:
            counts = np.full(E, int(rng.integers(0, 1000)))
        elif kind == 3:
            counts = rng.zipf(1.3, E).clip(0, 5000)
        else:
            counts = rng.choice([129, 130, 385, 641], E)   # the fewest rows per 256-row tile
        M = int(counts.sum())
        need, have = workgroups_needed(counts, tn), provided(lib, E, M, N)
        assert need <= have, (E, M, N, need, have)
        tight += need == have
    assert tight > 0   # the bound is reached: every expert of 129 rows


def test_routed_expert_workload(lib):
    # 4096 tokens x top-8 of 256 experts, as the benchmark routes them
    from block_scaled_fp8_act_amd import inputs as I
    d = I.WORKLOADS["moe"].dims
    idx, _ = I.zipf_topk(d["tokens"], d["experts"], d["topk"], d["zipf_s"])
    counts = np.bincount(idx.reshape(-1), minlength=d["experts"])
    M = int(counts.sum())
    for N in (d["dim"], 2 * d["inter"]):
        assert workgroups_needed(counts, -(-N // 256)) <= provided(lib, d["experts"], M, N)

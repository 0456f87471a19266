"""GPU segment builder vs the oracle's stable counting sort: bit-exact.

Covers the ids of the five named workloads, random batches (ragged sizes, 1..16384
adapters, both sides of the 960-adapter switch between the two builder kernels), the
degenerate cases (one row, all rows base-only, all rows one adapter, one
adapter in the pool) and out-of-range ids (counted in meta[2], treated as base-only).
"""

import zlib

import numpy as np
import pytest

import oracle
from synth import make_workload

from .gpu_util import gpu_segments, log

pytestmark = pytest.mark.gpu

TILE = 16


def _expected(ids: np.ndarray, n: int):
    bad = (ids < -1) | (ids >= n)
    clean = np.where(bad, -1, ids).astype(np.int32)
    ref = oracle.build_segments(clean, n, TILE)
    ref["meta"] = ref["meta"].copy()
    ref["meta"][2] = int(bad.sum())
    return ref


def _check(ids: np.ndarray, n: int, what: str):
    log(f"segments: {what} M={len(ids)} n={n}")
    got, _, _ = gpu_segments(ids, n)
    ref = _expected(ids, n)
    for key in ("perm", "offsets", "seg_adapter", "tiles", "meta"):
        assert np.array_equal(got[key], ref[key]), (what, key)
    again, _, _ = gpu_segments(ids, n)
    for key in got:
        assert np.array_equal(got[key], again[key]), (what, "not deterministic", key)


@pytest.mark.parametrize("config", [1, 2, 3, 4, 5])
def test_named_workloads(workload_cache, config):
    w = workload_cache(config)
    _check(w.ids, w.n_adapters, f"config {config}")


CASES = [
    ("one row", np.array([3], np.int32), 8),
    ("one row base", np.array([-1], np.int32), 8),
    ("all base", np.full(300, -1, np.int32), 5),
    ("all one adapter", np.full(1000, 7, np.int32), 8),
    ("all one adapter, 313 tiles", np.full(5000, 3, np.int32), 8),
    ("single-slot pool", np.zeros(77, np.int32), 1),
    ("ragged 65", None, 3),
    ("ragged 1023", None, 40),
    ("ragged 1025", None, 1024),
    ("large 5000", None, 16384),
    ("large 20000 zipf-like", None, 300),
    ("edge 3000", None, 959),
    ("edge 2100", None, 960),
    ("long 100000", None, 600),
    ("contiguous 4096 runs", np.repeat(np.arange(8, dtype=np.int32), 512), 8),
]


@pytest.mark.parametrize("name,ids,n", CASES, ids=[c[0] for c in CASES])
def test_cases(name, ids, n):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if ids is None:
        M = int(name.split()[1])
        if "zipf" in name:
            p = np.arange(1, n + 1, dtype=np.float64) ** -1.1
            ids = rng.choice(n, size=M, p=p / p.sum()).astype(np.int32)
        else:
            ids = rng.integers(-1, n, size=M).astype(np.int32)
    _check(ids, n, name)


def test_invalid_ids_are_counted_and_base_only():
    rng = np.random.default_rng(5)
    ids = rng.integers(-1, 6, size=500).astype(np.int32)
    ids[[3, 50, 499]] = [6, -5, 1 << 30]
    _check(ids, 6, "invalid ids")

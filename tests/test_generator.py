"""The seeded input generator: reproducible, bf16 rounding, padding, id distributions.  CPU only."""

import numpy as np
import pytest
import torch

from synth import (CONFIGS, bf16_bits_to_f32, compact_pool, f32_to_bf16_bits, make_workload,
                   random_case, zipf_probs)


def test_bf16_rounding_matches_torch():
    """Round-half-to-even on the bit pattern agrees with torch's float32 -> bfloat16 cast."""
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30,
                                  -2.5e-38, 3.0e38], np.float32)])
    # ties: exactly halfway between two bf16 values, both parities of the kept bit
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    v = np.concatenate([v, ties.view(np.float32)])
    ours = f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_bits_to_f32(ours), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_reproducible_bits():
    a, b = make_workload(1), make_workload(1)
    for pa, pb in zip(a.projections, b.projections):
        for k in ("x", "W", "A", "B"):
            assert np.array_equal(getattr(pa, k), getattr(pb, k))
    assert np.array_equal(a.ids, b.ids)
    c = make_workload(1, seed=7)
    assert not np.array_equal(a.projections[0].x, c.projections[0].x)


def test_config1_shapes_and_ids():
    w = make_workload(1)
    p = w.projections[0]
    assert w.storage == "f32" and p.x.dtype == np.float32
    assert p.x.shape == (16, 256) and p.W.shape == (256, 256)
    assert p.A.shape == (4, 256, 8) and p.B.shape == (4, 8, 256)
    assert set(np.unique(w.ids)).issubset({-1, 0, 1, 2, 3})
    assert np.all(w.alpha / w.ranks == 2.0)
    wb = w.as_bf16()
    assert wb.projections[0].x.dtype == np.uint16
    assert np.array_equal(wb.projections[0].W, f32_to_bf16_bits(p.W))


def test_config3_base_rows_and_padding():
    w = make_workload(3)
    assert w.M == 256 and int((w.ids == -1).sum()) == 26
    assert set(np.unique(w.ranks)).issubset({8, 16, 32, 64})
    assert np.all(w.alpha == 2 * w.ranks)
    p = w.projections[0]
    for i, r in enumerate(w.ranks):
        assert not np.any(p.A[i, :, r:]) and not np.any(p.B[i, r:, :])
        assert np.all(p.A[i, :, :r].any(axis=0)) and np.all(p.B[i, :r, :].any(axis=1))


def test_config4_blocks():
    spec = CONFIGS[4]
    assert spec["M"] == 4096
    # ids only (avoid drawing the 4096^2 tensors twice)
    ids = np.repeat(np.arange(8), 512)
    w = make_workload(4)
    assert np.array_equal(w.ids, ids)


def test_zipf():
    p = zipf_probs(1024, 1.1)
    assert p[0] == pytest.approx(0.1789, abs=2e-3)
    assert np.all(np.diff(p) < 0) and p.sum() == pytest.approx(1.0)


def test_value_scale():
    w = make_workload(2)
    p = w.as_f32().projections[0]
    assert p.x.std() == pytest.approx(1.0, rel=0.01)
    assert p.W.std() == pytest.approx(0.02, rel=0.01)
    assert p.A.std() == pytest.approx(0.02, rel=0.01)


def test_random_case_padding():
    w = random_case(5, 33, 40, 24, 7, 16)
    p = w.projections[0]
    for i, r in enumerate(w.ranks):
        assert 1 <= r <= 16
        assert not np.any(p.A[i, :, r:]) and not np.any(p.B[i, r:, :])


def test_compact_pool_is_the_padded_pool_at_true_rank():
    """The rank-compact layout holds exactly the unpadded part of every adapter: its size is
    sum r_i (d_in + d_out) elements (the per-adapter count of the pages' adapter-size
    formula, at each adapter's own rank), and every block maps back to A[i, :, :r_i] and
    B[i, :r_i, :]."""
    w = make_workload(3)
    p = w.projections[0]
    A_c, B_c, off, rows = compact_pool(p.A, p.B, w.ranks)
    n, d_in, r_max = p.A.shape
    d_out = p.B.shape[2]
    assert rows == int(w.ranks.sum())
    assert A_c.size + B_c.size == sum(int(r) * (d_in + d_out) for r in w.ranks)
    assert off[0] == 0 and np.all(np.diff(off) == w.ranks[:-1])
    for i in range(n):
        o, r = int(off[i]), int(w.ranks[i])
        assert np.array_equal(A_c[o * d_in:(o + r) * d_in].reshape(d_in, r), p.A[i, :, :r])
        assert np.array_equal(B_c[o:o + r], p.B[i, :r, :])
        assert not np.any(p.A[i, :, r:]) and not np.any(p.B[i, r:, :])  # nothing dropped
    # every rank of this workload is a multiple of 8: no adapter needs rows of zeros


def test_compact_pool_rounds_each_adapter_up_to_8_rows():
    """Ranks that are not multiples of 8 occupy round_up(r, 8) rank rows, the extra rows
    zero, so that every k row of A_i starts 16-byte aligned."""
    w = random_case(5, 8, 64, 40, 6, 24, ranks=[1, 8, 12, 17, 24, 3])
    p = w.projections[0]
    A_c, B_c, off, rows = compact_pool(p.A, p.B, w.ranks)
    widths = [8, 8, 16, 24, 24, 8]
    assert rows == sum(widths) and list(off) == list(np.cumsum([0] + widths[:-1]))
    for i, (r, wd) in enumerate(zip(w.ranks, widths)):
        o = int(off[i])
        blk = A_c[o * 64:(o + wd) * 64].reshape(64, wd)
        assert np.array_equal(blk[:, :r], p.A[i, :, :r]) and not np.any(blk[:, r:])
        assert np.array_equal(B_c[o:o + r], p.B[i, :r, :]) and not np.any(B_c[o + r:o + wd])

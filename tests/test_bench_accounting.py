"""The algorithmic bytes and flops bench.py charges each kernel, checked against figures worked
out by hand from the workloads' definitions.  CPU only: nothing here touches a GPU.

The roofline fractions the bench reports divide these figures by measured durations, so an
error here would misstate every fraction.
"""

import numpy as np

import bench
from synth import make_workload


def test_headline_decode_gemm_bytes():
    """Decode q_proj, 64 rows: W (4096 x 4096 bf16) + x (64 x 4096 bf16) + the A of every
    adapter the seeded ids touch, at rank 16 (28 of 32 adapters)."""
    w = make_workload(2).as_bf16()
    touched = np.unique(w.ids[w.ids >= 0])
    assert len(touched) == 28
    work = bench.algorithmic_work(w, 4096, 4096, prefill=False)
    expect = 4096 * 4096 * 2 + 64 * 4096 * 2 + 28 * 16 * 4096 * 2
    assert expect == 37_748_736
    assert work["decode_gemm_lora"]["bytes"] == expect
    # the reduction: B of the touched adapters, t of every row, y written once
    assert work["decode_reduce_lora"]["bytes"] == 28 * 16 * 4096 * 2 + 64 * 16 * 4 + 64 * 4096 * 2


def test_prefill_flops():
    """Prefill, 4096 rows: 2 M d_in d_out of base plus 2 r d_out per row of expand (all rows
    have a rank-16 adapter) in the GEMM's epilogue: 137.44 + 0.54 GFLOP."""
    w = make_workload(4).as_bf16()
    work = bench.algorithmic_work(w, 4096, 4096, prefill=True)
    base = 2.0 * 4096 * 4096 * 4096
    assert work["gemm_prefill_lora"]["flops"] == base + 2.0 * 4096 * 16 * 4096
    assert abs(work["call_flops"] - (base + 2.0 * 4096 * 16 * (4096 + 4096))) < 1.0


def test_heterogeneous_adapters_count_at_true_rank():
    """Adapters of the heterogeneous workload are charged at their own rank, not at the
    r_max = 64 they are padded to, and only when a row uses them."""
    w = make_workload(3).as_bf16()
    used = np.unique(w.ids[w.ids >= 0])
    work = bench.algorithmic_work(w, 4096, 4096, prefill=False)
    a_true = int(w.ranks[used].sum()) * 4096 * 2
    lora_rows = int((w.ids >= 0).sum())
    r_rows = int(w.ranks[w.ids[w.ids >= 0]].sum())
    assert work["shrink"]["bytes"] == a_true + lora_rows * 4096 * 2 + r_rows * 4
    assert a_true < len(used) * 64 * 4096 * 2  # below the padded bytes


def test_merged_call_kernels_split_between_projections():
    """A lora_linear_multi call over two projections: launches shared by the group (the merged
    shrink, GEMM and reduction) are charged half to each projection; launches made once per
    projection (the call ran projection by projection) go to the projections in order."""
    merged = [("shrink", 16.0), ("gemm_decode", 100.0), ("decode_reduce_lora", 50.0)]
    a, b = bench.split_group_kernels(merged, 2)
    assert a == b == [("shrink", 8.0), ("gemm_decode", 50.0), ("decode_reduce_lora", 25.0)]
    looped = [("shrink", 9.0), ("gemm_decode", 60.0), ("shrink", 10.0), ("gemm_decode", 61.0)]
    a, b = bench.split_group_kernels(looped, 2)
    assert a == [("shrink", 9.0), ("gemm_decode", 60.0)]
    assert b == [("shrink", 10.0), ("gemm_decode", 61.0)]
    # the per-projection lists add back to the call's total
    for ks in (merged, looped):
        a, b = bench.split_group_kernels(ks, 2)
        assert abs(sum(ms for _, ms in a + b) - sum(ms for _, ms in ks)) < 1e-9

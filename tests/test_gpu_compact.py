"""lora_linear_compact (adapters stored at their own rank, no padding to r_max) vs the CPU
oracle, through the C ABI, on every launch path of the layer.

The compact pool is a storage layout of the same adapters: the oracle computes y from the
padded pool it was cut from.  The compact call takes the same launches as lora_linear on the
padded pool (small decode batches included: the fused GEMM's adapter tiles read each compact
adapter at its own row width), so the two outputs are also compared bit for bit.  The parity
rule is that of test_gpu_parity.
"""

import numpy as np
import pytest

import oracle
from synth import compact_pool, random_case

from .gpu_util import assert_parity, bf16_dev, bf16_host, gpu_linear, log, to_device

pytestmark = pytest.mark.gpu

DECODE, PREFILL = 1, 2


def oracle_y(w, pi=0, rows=None):
    p = w.projections[pi]
    return oracle.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids, rows=rows)


def to_compact(w, pi=0, pool_rows=None):
    """Device copies of the compact pool of projection pi (bf16 bits) and its offsets."""
    import torch

    p = w.projections[pi]
    A_c, B_c, off, rows = compact_pool(p.A, p.B, w.ranks)
    if pool_rows is not None:  # a pool cut short: the adapters past it must add nothing
        A_c, B_c, rows = A_c[:pool_rows * p.d_in], B_c[:pool_rows], pool_rows
    return bf16_dev(A_c), bf16_dev(B_c), torch.from_numpy(off).cuda(), rows


def gpu_compact(dw, comp, mode, y_f32=False, ids=None, ranks=None):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    A_c, B_c, off, rows = comp
    p = dw.projs[0]
    M = dw.M
    y = torch.empty((M, p.d_out), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    ws, nbytes = L.workspace(M, p.d_in, p.d_out, dw.w.r_max, dw.n)
    L.lora_linear_compact(p.x, p.W, A_c, B_c, dw.scale, dw.ranks if ranks is None else ranks, off,
                          rows, dw.ids if ids is None else ids, M, p.d_in, p.d_out, dw.w.r_max,
                          dw.n, None, y, L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws, nbytes)
    torch.cuda.synchronize()
    return y.cpu().numpy() if y_f32 else bf16_host(y)


def ranks8(seed, n, r_max):
    """Ranks drawn from the multiples of 8 up to r_max (ranks of any value are covered by
    test_gpu_boundary)."""
    rng = np.random.default_rng(seed + 1000)
    return (8 * rng.integers(1, r_max // 8 + 1, size=n)).astype(np.int32)


CASES = [
    # seed, M, d_in, d_out, n, r_max, base_frac, mode, path
    (41, 64, 1024, 520, 40, 64, 0.2, DECODE, "small batch (fused)"),
    (48, 33, 512, 264, 70, 16, 0.1, DECODE, "small batch (fused), pool larger than the batch"),
    (42, 200, 1024, 520, 40, 32, 0.1, DECODE, "medium"),
    (43, 300, 4096, 2056, 50, 64, 0.1, DECODE, "stream-K"),
    (44, 1500, 256, 512, 5, 16, 0.1, DECODE, "split-K GEMM + expand"),
    (45, 640, 2048, 256, 200, 32, 0.0, PREFILL, "prefill epilogue"),
    (46, 100, 264, 1032, 600, 8, 0.1, DECODE, "segment path, d_in % 32 != 0"),
    (47, 17, 136, 264, 3, 64, 0.2, PREFILL, "prefill, ragged"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-M{c[1]}-{c[8]}" for c in CASES])
@pytest.mark.parametrize("y_f32", [False, True], ids=["bf16", "f32"])
def test_compact_matches_oracle(case, y_f32):
    seed, M, d_in, d_out, n, r_max, base_frac, mode, path = case
    log(f"compact: {case} y_f32={y_f32}")
    w = random_case(seed, M, d_in, d_out, n, r_max, ranks=ranks8(seed, n, r_max),
                    base_frac=base_frac)
    dw = to_device(w)
    y = gpu_compact(dw, to_compact(w.as_bf16()), mode, y_f32=y_f32)
    assert_parity(y, oracle_y(w), f"compact {case}")
    y_pad = gpu_linear(dw, 0, mode, y_f32=y_f32)  # the same launches on the padded pool
    assert np.array_equal(y, y_pad), f"compact {case}: differs from the padded pool's bits"


@pytest.mark.parametrize("mode", [DECODE, PREFILL])
def test_compact_heterogeneous_workload(workload_cache, mode):
    """The heterogeneous-rank decode workload (256 x 4096, 128 adapters, ranks 8..64 padded
    to 64) served from its compact pool."""
    w = workload_cache(3).as_bf16()
    log(f"compact: decode heterogeneous, mode {mode}")
    dw = to_device(w)
    y = gpu_compact(dw, to_compact(w), mode)
    assert_parity(y, oracle_y(w), f"compact heterogeneous mode {mode}")
    assert np.array_equal(y, gpu_linear(dw, 0, mode))

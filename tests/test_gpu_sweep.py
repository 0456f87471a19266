"""A seeded sweep of random layer shapes through the C ABI, against the CPU oracle.

Ninety-six cases are drawn once from a fixed generator, so every run sees the same ones.
They vary:
  * the batch, from one row to past the stream-K range;
  * d_in and d_out at each alignment the launch paths branch on (multiples of 8, 32 and 128);
  * r_max from 1 to 64, on a rank bucket or not;
  * the pool, smaller or larger than the batch;
  * the ids, from every row base-only to no base row;
  * the mode (decode, prefill, automatic);
  * the output (bf16, fp32) and the pool layout (padded, rank-compact).
Adapter sizes are capped so that the pool stays small on the host.

Each case logs its parameters before its GPU calls.  The parity rule is test_gpu_parity's.
A rank-compact case is checked against the oracle too.  Its bits are also compared with the
padded pool it was cut from, except where the two calls take different launches: a decode
batch of at most 128 rows (d_in % 32 == 0) whose r_max is no rank bucket runs the medium
sequence on the padded pool and the fused one on the compact pool.
"""

import numpy as np
import pytest

import oracle
from synth import compact_pool, random_case

from .gpu_util import assert_parity, bf16_dev, bf16_host, gpu_linear, log, to_device

pytestmark = pytest.mark.gpu

AUTO, DECODE, PREFILL = 0, 1, 2


def _draw_cases(n_cases: int = 96, seed: int = 20261203):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n_cases):
        # batch size: every launch path (fused <= 128, medium <= 256, stream-K <= 1024, beyond)
        lo, hi = [(1, 16), (17, 128), (129, 256), (257, 1024), (1025, 1600)][int(rng.choice(5, p=[0.15, 0.3, 0.2, 0.25, 0.1]))]
        M = int(rng.integers(lo, hi + 1))
        # d_in: a multiple of 128, of 32 only, or of 8 only
        align = [128, 32, 8][int(rng.choice(3, p=[0.45, 0.3, 0.25]))]
        d_in = int(align * rng.integers(max(1, 16 // align), 4160 // align + 1))
        if align < 128 and d_in % (2 * align) == 0:
            d_in += align  # keep the stated alignment exact
        d_out = int(8 * rng.integers(1, 3072 // 8 + 1))
        r_max = int(rng.choice([8, 16, 32, 64])) if rng.random() < 0.5 else int(rng.integers(1, 65))
        n = int(np.exp(rng.uniform(0.0, np.log(1200.0))))
        # host pool size: n x d_in x r_max and n x r_max x d_out elements, at most 2e7 each
        n = max(1, min(n, int(2e7 // (d_in * r_max)), int(2e7 // (r_max * d_out))))
        base_frac = float(rng.choice([0.0, 0.1, 0.3, 1.0], p=[0.3, 0.4, 0.2, 0.1]))
        mode = int(rng.choice([DECODE, PREFILL, AUTO], p=[0.5, 0.3, 0.2]))
        y_f32 = bool(rng.random() < 0.3)
        compact = bool(rng.random() < 0.25)
        cases.append((1000 + i, M, d_in, d_out, n, r_max, base_frac, mode, y_f32, compact))
    return cases


CASES = _draw_cases()


def _compact_call(dw, w, mode, y_f32):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    p = w.projections[0]
    A_c, B_c, off, rows = compact_pool(p.A, p.B, w.ranks)
    dp = dw.projs[0]
    M = dw.M
    y = torch.empty((M, dp.d_out), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    ws, nbytes = L.workspace(M, dp.d_in, dp.d_out, w.r_max, dw.n)
    L.lora_linear_compact(dp.x, dp.W, bf16_dev(A_c), bf16_dev(B_c), dw.scale, dw.ranks,
                          torch.from_numpy(off).cuda(), rows, dw.ids, M, dp.d_in, dp.d_out,
                          w.r_max, dw.n, None, y, L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws,
                          nbytes)
    torch.cuda.synchronize()
    return y.cpu().numpy() if y_f32 else bf16_host(y)


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}-M{c[1]}-{c[2]}x{c[3]}-n{c[4]}-r{c[5]}" for c in CASES])
def test_sweep(case):
    seed, M, d_in, d_out, n, r_max, base_frac, mode, y_f32, compact = case
    log(f"sweep: seed={seed} M={M} d_in={d_in} d_out={d_out} n={n} r_max={r_max} "
        f"base={base_frac} mode={mode} y_f32={y_f32} compact={compact}")
    w = random_case(seed, M, d_in, d_out, n, r_max, base_frac=base_frac).as_bf16()
    p = w.projections[0]
    ref = oracle.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    dw = to_device(w)
    y = gpu_linear(dw, 0, mode, y_f32=y_f32)
    assert_parity(y, ref, f"sweep {case}")
    if compact:
        yc = _compact_call(dw, w, mode, y_f32)
        assert_parity(yc, ref, f"sweep {case} (compact)")
        from rank_adapter_gemm_sgmv_amd import lora as L

        decode = mode == DECODE or (mode == AUTO and M < L.LORA_PREFILL_MIN_ROWS)
        fused_only_compact = decode and M <= 128 and d_in % 32 == 0 and r_max not in (8, 16, 32, 64)
        if not fused_only_compact:
            assert np.array_equal(yc, y), f"sweep {case}: the compact pool's bits differ"

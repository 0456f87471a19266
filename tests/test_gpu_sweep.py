"""Seeded sweeps of random layer shapes through the C ABI, against the CPU oracle: the layer
(lora_linear and lora_linear_compact), the fp8 base (lora_linear_fp8w) and the MoE layer
(lora_moe_linear).

The layer:

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

The fp8 base: 32 cases over 1-256 rows, d_in a multiple of 32 (at least 128), any d_out, r_max
1-64, pools smaller and larger than the batch, bf16 and fp32 outputs.  The MoE layer: 32 cases
over 1-300 tokens, top_k 1-8 of 1-64 experts, empty slots, skewed routing, r_max a multiple of
8, tokens without an adapter; empty slots must be zero rows.

Each case logs its parameters before its GPU calls.  The parity rule is test_gpu_parity's.
A rank-compact case is checked against the oracle too.  Its bits are also compared with the
padded pool it was cut from, except where the two calls take different launches: a decode
batch of at most 128 rows (d_in % 32 == 0) whose r_max is not a multiple of 8 runs the medium
sequence on the padded pool and the fused one on the compact pool.
"""

import numpy as np
import pytest

import oracle
from synth import compact_pool, fp8_base, moe_case, random_case

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
        fused_only_compact = decode and M <= 128 and d_in % 32 == 0 and r_max % 8 != 0
        if not fused_only_compact:
            assert np.array_equal(yc, y), f"sweep {case}: the compact pool's bits differ"


def _draw_fp8_cases(n_cases: int = 32, seed: int = 20261204):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n_cases):
        M = int(rng.integers(1, 257))
        d_in = int(32 * rng.integers(4, 4160 // 32 + 1))
        d_out = int(8 * rng.integers(1, 3072 // 8 + 1))
        r_max = int(rng.choice([8, 16, 32, 64])) if rng.random() < 0.5 else int(rng.integers(1, 65))
        n = int(np.exp(rng.uniform(0.0, np.log(600.0))))
        n = max(1, min(n, int(2e7 // (d_in * r_max)), int(2e7 // (r_max * d_out))))
        base_frac = float(rng.choice([0.0, 0.1, 0.3, 1.0], p=[0.3, 0.4, 0.2, 0.1]))
        y_f32 = bool(rng.random() < 0.3)
        cases.append((2000 + i, M, d_in, d_out, n, r_max, base_frac, y_f32))
    return cases


FP8_CASES = _draw_fp8_cases()


@pytest.mark.parametrize("case", FP8_CASES, ids=[f"s{c[0]}-M{c[1]}-{c[2]}x{c[3]}-n{c[4]}-r{c[5]}" for c in FP8_CASES])
def test_sweep_fp8(case):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    seed, M, d_in, d_out, n, r_max, base_frac, y_f32 = case
    log(f"sweep fp8: seed={seed} M={M} d_in={d_in} d_out={d_out} n={n} r_max={r_max} "
        f"base={base_frac} y_f32={y_f32}")
    w = random_case(seed, M, d_in, d_out, n, r_max, base_frac=base_frac).as_bf16()
    W8, w_scale = fp8_base(seed, d_in, d_out)
    p = w.projections[0]
    ref = oracle.lora_linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, w.ids)
    dw = to_device(w)
    dp = dw.projs[0]
    y = torch.empty((M, d_out), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    ws, nb = L.workspace(M, d_in, d_out, r_max, n)
    L.lora_linear_fp8w(dp.x, torch.from_numpy(np.ascontiguousarray(W8)).cuda(),
                       torch.from_numpy(w_scale).cuda(), dp.A, dp.B, dw.scale, dw.ranks, dw.ids, M,
                       d_in, d_out, r_max, n, None, y, L.LORA_F32 if y_f32 else L.LORA_BF16,
                       L.LORA_MODE_DECODE, ws, nb)
    torch.cuda.synchronize()
    assert_parity(y.cpu().numpy() if y_f32 else bf16_host(y), ref, f"sweep fp8 {case}")


def _draw_moe_cases(n_cases: int = 32, seed: int = 20261205):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n_cases):
        M = int(rng.integers(1, 301))
        E = int(rng.integers(1, 65))
        top_k = int(rng.integers(1, min(8, E) + 1))
        d_in = int(32 * rng.integers(4, 2048 // 32 + 1))
        d_out = int(8 * rng.integers(1, 1536 // 8 + 1))
        d_out = max(8, min(d_out, int(5e7 // (E * d_in)) // 8 * 8))  # E x d_in x d_out <= 5e7
        r_max = int(8 * rng.integers(1, 9))
        n = int(np.exp(rng.uniform(0.0, np.log(400.0))))
        # host pool size: n x E x d_in x r_max elements (and B's), at most 3e7 each
        n = max(1, min(n, int(3e7 // (E * d_in * r_max)), int(3e7 // (E * r_max * d_out))))
        empty = float(rng.choice([0.0, 0.1, 0.4]))
        zipf = float(rng.choice([0.0, 0.0, 1.2]))
        y_f32 = bool(rng.random() < 0.3)
        cases.append((3000 + i, M, top_k, E, d_in, d_out, n, r_max, empty, zipf, y_f32))
    return cases


MOE_CASES = _draw_moe_cases()


@pytest.mark.parametrize("case", MOE_CASES, ids=[f"s{c[0]}-M{c[1]}k{c[2]}E{c[3]}-{c[4]}x{c[5]}-r{c[7]}" for c in MOE_CASES])
def test_sweep_moe(case):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    seed, M, top_k, E, d_in, d_out, n, r_max, empty, zipf, y_f32 = case
    log(f"sweep moe: seed={seed} M={M} top_k={top_k} E={E} d_in={d_in} d_out={d_out} n={n} "
        f"r_max={r_max} empty={empty} zipf={zipf} y_f32={y_f32}")
    w = moe_case(seed, M, top_k, E, d_in, d_out, n, r_max, base_frac=0.2, empty_frac=empty,
                 zipf_s=zipf)
    ref = oracle.moe_lora_linear(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids, w.topk_w)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    scale = (w.alpha.astype(np.float32) / w.ranks.astype(np.float32)).astype(np.float32)
    y = torch.empty((M, top_k, d_out), dtype=torch.float32 if y_f32 else torch.bfloat16,
                    device="cuda")
    ws = L.moe_workspace(M, top_k, E, d_in, d_out, r_max, n)
    L.lora_moe_linear(bf(w.x), bf(w.W), bf(w.A), bf(w.B), torch.from_numpy(scale).cuda(),
                      torch.from_numpy(w.ranks.astype(np.int32)).cuda(),
                      torch.from_numpy(w.ids.astype(np.int32)).cuda(),
                      torch.from_numpy(w.topk_ids.astype(np.int32)).cuda(),
                      torch.from_numpy(w.topk_w.astype(np.float32)).cuda(), M, top_k, E, d_in,
                      d_out, r_max, n, y, L.LORA_F32 if y_f32 else L.LORA_BF16, 1, ws[0], ws[1])
    torch.cuda.synchronize()
    got = y.cpu().numpy() if y_f32 else bf16_host(y)
    assert_parity(got, ref, f"sweep moe {case}")
    assert not np.any(got[w.topk_ids < 0]), "empty slots must be zero rows"

"""The C ABI at the edges of its contract, on the GPU, against the CPU oracle:

- r_max anywhere in [1, 64] (the kernels run at the rank bucket 8/16/32/64; a padded pool of
  any r_max is stored at that stride), on every launch path of lora_linear: small decode
  batches take the fused GEMM when r_max is a multiple of 8 (each adapter's rows read at the
  pool's stride; rank-8 pools in 16-wide slots), the medium sequence otherwise;
- rank-compact pools whose ranks are any value in [1, r_max] (not only multiples of 8);
- lora_shrink / lora_expand with such an r_max (t is [M, r_max]) and their compact variants;
- LORA_MODE_CHECKED: a bad id, rank or compact offset is reported and nothing is enqueued;
  valid tables give the unchecked result bit for bit.

The parity rule is that of test_gpu_parity (every row, max|y_ref| over the whole output).
"""

import numpy as np
import pytest

import oracle
from synth import compact_pool, random_case

from .gpu_util import assert_parity, bf16_dev, bf16_host, gpu_linear, log, to_device

pytestmark = pytest.mark.gpu

DECODE, PREFILL = 1, 2


def oracle_y(w, ids=None):
    p = w.projections[0]
    return oracle.lora_linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids if ids is None else ids)


ANY_RANK = [
    # seed, M, d_in, d_out, n, r_max, base_frac, mode, path
    (201, 64, 1024, 520, 9, 12, 0.2, DECODE, "small batch -> medium"),
    (202, 200, 1024, 520, 40, 5, 0.1, DECODE, "medium"),
    (203, 300, 4096, 2056, 50, 24, 0.1, DECODE, "stream-K"),
    (204, 1500, 256, 512, 5, 40, 0.1, DECODE, "split-K GEMM + expand"),
    (205, 640, 2048, 256, 200, 3, 0.0, PREFILL, "prefill epilogue"),
    (206, 100, 264, 1032, 60, 1, 0.1, DECODE, "segment path, rank 1"),
    (207, 17, 136, 264, 3, 63, 0.2, PREFILL, "prefill, ragged"),
    (208, 96, 2048, 768, 12, 48, 0.1, DECODE, "small batch (fused), stride 48"),
    (209, 64, 1024, 520, 30, 8, 0.1, DECODE, "small batch (fused), rank 8 in 16-wide slots"),
    (210, 40, 512, 264, 90, 40, 0.2, DECODE, "small batch (fused), stride 40, pool > batch"),
    (218, 128, 4096, 1032, 33, 24, 0.0, DECODE, "small batch (fused), stride 24, 128 rows"),
]


@pytest.mark.parametrize("case", ANY_RANK, ids=[f"r{c[5]}-M{c[1]}-{c[8]}" for c in ANY_RANK])
@pytest.mark.parametrize("y_f32", [False, True], ids=["bf16", "f32"])
def test_any_r_max(case, y_f32):
    seed, M, d_in, d_out, n, r_max, base_frac, mode, path = case
    log(f"boundary: r_max {r_max} {case} y_f32={y_f32}")
    w = random_case(seed, M, d_in, d_out, n, r_max, base_frac=base_frac)
    y = gpu_linear(to_device(w), 0, mode, y_f32=y_f32)
    assert_parity(y, oracle_y(w), f"r_max {r_max} {path}")


def to_compact(w):
    import torch

    p = w.as_bf16().projections[0]
    A_c, B_c, off, rows = compact_pool(p.A, p.B, w.ranks)
    return bf16_dev(A_c), bf16_dev(B_c), torch.from_numpy(off).cuda(), rows


def gpu_compact(dw, comp, mode, y_f32=False, ranks=None, check=False):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    A_c, B_c, off, rows = comp
    p = dw.projs[0]
    M = dw.M
    y = torch.empty((M, p.d_out), dtype=torch.float32 if y_f32 else torch.bfloat16, device="cuda")
    ws, nbytes = L.workspace(M, p.d_in, p.d_out, dw.w.r_max, dw.n)
    L.lora_linear_compact(p.x, p.W, A_c, B_c, dw.scale, dw.ranks if ranks is None else ranks, off,
                          rows, dw.ids, M, p.d_in, p.d_out, dw.w.r_max, dw.n, None, y,
                          L.LORA_F32 if y_f32 else L.LORA_BF16,
                          mode | (L.LORA_MODE_CHECKED if check else 0), ws, nbytes)
    torch.cuda.synchronize()
    return y.cpu().numpy() if y_f32 else bf16_host(y)


COMPACT_ANY = [
    # seed, M, d_in, d_out, n, r_max, base_frac, mode, path
    (211, 64, 1024, 520, 40, 64, 0.2, DECODE, "small batch (fused)"),
    (212, 200, 1024, 520, 40, 32, 0.1, DECODE, "medium"),
    (213, 300, 4096, 2056, 50, 64, 0.1, DECODE, "stream-K"),
    (214, 1500, 256, 512, 5, 16, 0.1, DECODE, "split-K GEMM + expand"),
    (215, 640, 2048, 256, 200, 32, 0.0, PREFILL, "prefill epilogue"),
    (216, 100, 264, 1032, 600, 13, 0.1, DECODE, "segment path"),
    (217, 17, 136, 264, 3, 64, 0.2, PREFILL, "prefill, ragged"),
]


@pytest.mark.parametrize("case", COMPACT_ANY, ids=[f"s{c[0]}-M{c[1]}-{c[8]}" for c in COMPACT_ANY])
def test_compact_any_rank(case):
    """Ranks drawn from [1, r_max] (mostly not multiples of 8), stored at their own rank."""
    seed, M, d_in, d_out, n, r_max, base_frac, mode, path = case
    log(f"boundary: compact, ranks 1..{r_max}, {case}")
    w = random_case(seed, M, d_in, d_out, n, r_max, base_frac=base_frac)
    assert (w.ranks % 8 != 0).any()
    dw = to_device(w)
    y = gpu_compact(dw, to_compact(w), mode, y_f32=True)
    assert_parity(y, oracle_y(w), f"compact any rank {path}")
    if same_launches(M, d_in, r_max, mode):  # as the padded pool: the same bits
        assert np.array_equal(y, gpu_linear(dw, 0, mode, y_f32=True))


def same_launches(M, d_in, r_max, mode):
    """A compact call takes the padded pool's launches, except for decode batches of at most
    128 rows (d_in % 32 == 0) whose padded r_max is not a multiple of 8: the padded pool then
    takes the medium path (its adapters' rows cannot be read in 16-byte groups), the compact
    one the fused path."""
    return not (mode == DECODE and M <= 128 and d_in % 32 == 0 and r_max % 8 != 0)


@pytest.mark.parametrize("M", [300, 96], ids=["M300", "M96-fused"])
def test_compact_adapter_outside_the_pool_adds_nothing(M):
    """An adapter whose rows leave the pool (the last one, cut off) leaves its rows
    base-only; the others are unaffected.  The checked mode reports it.  At 96 rows the
    adapter tiles of the fused GEMM read such an adapter at a stride of zero."""
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    n, r_max = 12, 32
    w = random_case(48, M, 1024, 264, n, r_max, base_frac=0.1)
    dw = to_device(w)
    A_c, B_c, off, rows = to_compact(w)
    cut = rows - int(w.ranks[-1])
    comp = (A_c[: cut * 1024], B_c[:cut], off, cut)
    for mode in (DECODE, PREFILL):
        y = gpu_compact(dw, comp, mode, y_f32=True)
        dropped = w.ids == n - 1
        ids_base = w.ids.copy()
        ids_base[dropped] = -1
        y_base = gpu_linear(dw, 0, mode, y_f32=True, ids=torch.from_numpy(ids_base).cuda())
        assert dropped.any()
        assert np.array_equal(y[dropped], y_base[dropped])
        assert_parity(y[~dropped], oracle_y(w)[~dropped], "compact, kept rows")
        with pytest.raises(L.LoraError) as e:
            gpu_compact(dw, comp, mode, check=True)
        assert e.value.status == 10  # LORA_ERR_POOL


@pytest.mark.parametrize("r_max", [5, 12, 24, 64])
def test_shrink_expand_any_rank(r_max):
    """lora_shrink and lora_expand at any r_max (t is [M, r_max]), and their compact
    variants on the same adapters stored at their own rank."""
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    log(f"boundary: shrink / expand, r_max {r_max}")
    w = random_case(220 + r_max, 97, 1032, 776, 11, r_max, base_frac=0.2)
    dw = to_device(w)
    p = w.projections[0]
    M, n = w.M, w.n_adapters
    seg = L.Segments(M, n)
    L.lora_build_segments(dw.ids, M, n, seg)
    ws, nbytes = L.workspace(M, p.d_in, 8, r_max, n)
    t_ref = oracle.lora_shrink(p.x, p.A, w.ids)
    A_c, B_c, off, rows = to_compact(w)
    y0 = np.random.default_rng(r_max).standard_normal((M, p.d_out)).astype(np.float32)
    y_ref = oracle.lora_expand(t_ref, p.B, w.alpha, w.ranks, w.ids, y0)
    base = w.ids == -1
    for compact in (False, True):
        t = torch.full((M, r_max), 7.0, dtype=torch.float32, device="cuda")
        if compact:
            L.lora_shrink_compact(dw.projs[0].x, A_c, dw.ranks, off, rows, M, p.d_in, r_max, n, seg,
                                  t, ws, nbytes)
        else:
            L.lora_shrink(dw.projs[0].x, dw.projs[0].A, dw.ranks, M, p.d_in, r_max, n, seg, t, ws,
                          nbytes)
        torch.cuda.synchronize()
        tg = t.cpu().numpy()
        assert_parity(tg, t_ref, f"shrink r_max {r_max} compact={compact}", max_rel=1e-4,
                      mean_rel=1e-5)
        assert not np.any(tg[base])
        for m in np.flatnonzero(~base):
            assert not np.any(tg[m, w.ranks[w.ids[m]]:])
        yd = torch.from_numpy(y0.copy()).cuda()
        td = torch.from_numpy(t_ref).cuda()
        if compact:
            L.lora_expand_compact(td, B_c, dw.scale, dw.ranks, off, rows, M, p.d_out, r_max, n, seg,
                                  yd, L.LORA_F32)
        else:
            L.lora_expand(td, dw.projs[0].B, dw.scale, dw.ranks, M, p.d_out, r_max, n, seg, yd,
                          L.LORA_F32)
        torch.cuda.synchronize()
        yg = yd.cpu().numpy()
        assert np.array_equal(yg[base], y0[base])
        assert_parity((yg - y0)[~base], (y_ref - y0)[~base], f"expand r_max {r_max} compact={compact}")


def test_checked_mode():
    """LORA_MODE_CHECKED: a bad id (LORA_ERR_BAD_ID) or rank (LORA_ERR_RANK) is reported
    before anything is enqueued (y keeps its contents); valid tables give the unchecked
    result bit for bit, on the small-batch, medium and prefill paths."""
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    for M, mode in ((64, DECODE), (200, DECODE), (300, PREFILL)):
        log(f"boundary: checked mode M={M} mode={mode}")
        w = random_case(230 + M, M, 512, 264, 7, 16, base_frac=0.1)
        dw = to_device(w)
        p = dw.projs[0]
        ws, nbytes = L.workspace(M, p.d_in, p.d_out, 16, 7)

        def call(ids=None, ranks=None, checked=True):
            y = torch.full((M, p.d_out), 3.0, dtype=torch.float32, device="cuda")
            L.lora_linear(p.x, p.W, p.A, p.B, dw.scale, dw.ranks if ranks is None else ranks,
                          dw.ids if ids is None else ids, M, p.d_in, p.d_out, 16, 7, None, y,
                          L.LORA_F32, mode | (L.LORA_MODE_CHECKED if checked else 0), ws, nbytes)
            torch.cuda.synchronize()
            return y

        assert torch.equal(call(), call(checked=False))
        bad = w.ids.copy()
        bad[M // 2] = 7
        for ids_bad in (bad, np.where(np.arange(M) == 3, -2, w.ids)):
            y = torch.full((M, p.d_out), 3.0, dtype=torch.float32, device="cuda")
            with pytest.raises(L.LoraError) as e:
                L.lora_linear(p.x, p.W, p.A, p.B, dw.scale, dw.ranks,
                              torch.from_numpy(ids_bad.astype(np.int32)).cuda(), M, p.d_in,
                              p.d_out, 16, 7, None, y, L.LORA_F32, mode | L.LORA_MODE_CHECKED, ws,
                              nbytes)
            assert e.value.status == 8  # LORA_ERR_BAD_ID
            torch.cuda.synchronize()
            assert bool((y == 3.0).all())  # nothing was enqueued
        for rv in (0, 17):
            r_bad = w.ranks.copy()
            r_bad[2] = rv
            with pytest.raises(L.LoraError) as e:
                call(ranks=torch.from_numpy(r_bad).cuda())
            assert e.value.status == 3  # LORA_ERR_RANK

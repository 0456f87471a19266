"""lora_linear_multi on the GPU: several projections that read the same x and the same adapter
tables, each with its own W, A and B (an MLP's gate and up projections).  Each projection's
output is checked against the oracle's layer for that projection, on every row.  Batches of
257-1024 rows run the projections' stream-K GEMMs as one launch (whole groups or, when the
merged panels would fill the chip, groups of fewer); every other batch runs lora_linear's
launches per projection and must give lora_linear's bits."""

import numpy as np
import pytest

import oracle
from synth import random_case

from .gpu_util import assert_parity, bf16_dev, bf16_host, log, scale_of

pytestmark = pytest.mark.gpu


def multi_case(seed, M, d_in, d_out, n_adapters, r_max, n_proj):
    """n_proj projections sharing x, ids, ranks and alpha (those of the first draw; bf16 bits)."""
    base = random_case(seed, M, d_in, d_out, n_adapters, r_max)
    projs = [base.projections[0]]
    for p in range(1, n_proj):
        w = random_case(seed + 1000 * p, M, d_in, d_out, n_adapters, r_max, ids=base.ids,
                        ranks=base.ranks)
        projs.append(w.projections[0])
    return base, projs


def run_multi(base, projs, mode, y_f32=False):
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    M, d_in, d_out = base.M, projs[0].d_in, projs[0].d_out
    x = bf16_dev(projs[0].x)
    Ws = [bf16_dev(p.W) for p in projs]
    As = [bf16_dev(p.A) for p in projs]
    Bs = [bf16_dev(p.B) for p in projs]
    ids = torch.from_numpy(base.ids.astype(np.int32)).cuda()
    ranks = torch.from_numpy(base.ranks.astype(np.int32)).cuda()
    scale = torch.from_numpy(scale_of(base)).cuda()
    dt = torch.float32 if y_f32 else torch.bfloat16
    ys = [torch.empty((M, d_out), dtype=dt, device="cuda") for _ in projs]
    nb = L.lora_workspace_bytes_multi(M, d_in, d_out, base.r_max, base.n_adapters, len(projs))
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
    L.lora_linear_multi(x, Ws, As, Bs, scale, ranks, ids, M, d_in, d_out, base.r_max,
                        base.n_adapters, None, ys, L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws, nb)
    torch.cuda.synchronize()
    out = [y.cpu().numpy() if y_f32 else bf16_host(y) for y in ys]
    singles = []
    n1 = L.lora_workspace_bytes(M, d_in, d_out, base.r_max, base.n_adapters)
    ws1 = torch.empty(max(n1, 256), dtype=torch.uint8, device="cuda")
    for W, A, B in zip(Ws, As, Bs):
        y = torch.empty((M, d_out), dtype=dt, device="cuda")
        L.lora_linear(x, W, A, B, scale, ranks, ids, M, d_in, d_out, base.r_max, base.n_adapters,
                      None, y, L.LORA_F32 if y_f32 else L.LORA_BF16, mode, ws1, n1)
        torch.cuda.synchronize()
        singles.append(y.cpu().numpy() if y_f32 else bf16_host(y))
    return out, singles


def refs(base, projs):
    x = projs[0].x
    return [oracle.lora_linear(x, p.W, p.A, p.B, base.alpha, base.ranks, base.ids) for p in projs]


# (seed, M, d_in, d_out, n_adapters, r_max, n_proj): 257-1024 rows with few 256 x 256 tiles
# take the merged stream-K launch: 2-4 projections in one group; 3 projections in groups of
# 2 + 1 (3 x 33 panels x 2 row tiles would fill the chip); a ragged last panel (d_out 1000);
# 3 and 4 row tiles; ranks up to 64
MERGED = [
    (501, 300, 4096, 2048, 24, 16, 2),
    (502, 300, 4096, 2048, 24, 16, 4),
    (503, 512, 4096, 2048, 96, 32, 3),
    (504, 260, 4096, 8200, 16, 16, 3),
    (505, 1000, 4096, 1000, 40, 64, 2),
    (506, 700, 4096, 1536, 8, 8, 2),
]


@pytest.mark.parametrize("case", MERGED, ids=[f"c{c[0]}-M{c[1]}-N{c[3]}-p{c[6]}" for c in MERGED])
def test_multi_merged_stream_k(case):
    from rank_adapter_gemm_sgmv_amd import lora as L

    seed, M, d_in, d_out, n, r_max, n_proj = case
    log(f"multi merged: seed {seed} M={M} {d_in}x{d_out} n={n} r_max={r_max} projections {n_proj}")
    base, projs = multi_case(seed, M, d_in, d_out, n, r_max, n_proj)
    out, singles = run_multi(base, projs, L.LORA_MODE_DECODE)
    for p, (y, y1, ref) in enumerate(zip(out, singles, refs(base, projs))):
        assert_parity(y, ref, f"projection {p}")
        assert_parity(y1, ref, f"projection {p}, lora_linear")


def test_multi_merged_f32_and_deterministic():
    from rank_adapter_gemm_sgmv_amd import lora as L

    base, projs = multi_case(511, 400, 4096, 2048, 32, 16, 2)
    log("multi merged: M=400 f32 output, two calls")
    a, _ = run_multi(base, projs, L.LORA_MODE_DECODE, y_f32=True)
    b, _ = run_multi(base, projs, L.LORA_MODE_DECODE, y_f32=True)
    for p, (ya, yb, ref) in enumerate(zip(a, b, refs(base, projs))):
        assert_parity(ya, ref, f"projection {p}, f32")
        assert np.array_equal(ya, yb), f"projection {p}: two calls differ"


# batches outside the stream-K range: lora_linear's sequence per projection, same bits
SEPARATE = [
    (521, 64, 1024, 1024, 16, 16, 2, "decode"),     # small-batch fused GEMM
    (522, 200, 1024, 768, 40, 32, 3, "decode"),     # medium decode path
    (523, 384, 1024, 1024, 16, 16, 2, "prefill"),   # prefill GEMM with the LoRA epilogue
    (524, 1200, 512, 512, 16, 8, 2, "decode"),      # above 1024 rows
    (525, 800, 2048, 6144, 16, 16, 2, "decode"),    # stream-K, but 2 x 24 panels x 4 row tiles
                                                    # would fill the chip: no merge
]


@pytest.mark.parametrize("case", SEPARATE, ids=[f"c{c[0]}-M{c[1]}-{c[7]}" for c in SEPARATE])
def test_multi_separate_paths(case):
    from rank_adapter_gemm_sgmv_amd import lora as L

    seed, M, d_in, d_out, n, r_max, n_proj, mode = case
    log(f"multi separate: seed {seed} M={M} {d_in}x{d_out} n={n} projections {n_proj} {mode}")
    base, projs = multi_case(seed, M, d_in, d_out, n, r_max, n_proj)
    m = L.LORA_MODE_PREFILL if mode == "prefill" else L.LORA_MODE_DECODE
    out, singles = run_multi(base, projs, m)
    for p, (y, y1, ref) in enumerate(zip(out, singles, refs(base, projs))):
        assert np.array_equal(y, y1), f"projection {p}: bits differ from lora_linear"
        assert_parity(y, ref, f"projection {p}")


def test_multi_caller_segments_and_checked_mode():
    """The merged stream-K sequence on segments the caller built (no build launch) gives the
    bits of the call that builds them; LORA_MODE_CHECKED passes valid tables through
    unchanged and reports an id outside [-1, n) before enqueueing anything."""
    import torch

    from rank_adapter_gemm_sgmv_amd import lora as L

    M, d_in, d_out, n, r_max = 320, 4096, 2048, 20, 16
    log(f"multi: caller segments and checked mode, M={M}")
    base, projs = multi_case(531, M, d_in, d_out, n, r_max, 2)
    x = bf16_dev(projs[0].x)
    Ws = [bf16_dev(p.W) for p in projs]
    As = [bf16_dev(p.A) for p in projs]
    Bs = [bf16_dev(p.B) for p in projs]
    ids = torch.from_numpy(base.ids.astype(np.int32)).cuda()
    ranks = torch.from_numpy(base.ranks.astype(np.int32)).cuda()
    scale = torch.from_numpy(scale_of(base)).cuda()
    nb = L.lora_workspace_bytes_multi(M, d_in, d_out, r_max, n, 2)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def call(segs=None, mode=L.LORA_MODE_DECODE, ids_t=ids):
        ys = [torch.full((M, d_out), 3.0, dtype=torch.float32, device="cuda") for _ in range(2)]
        L.lora_linear_multi(x, Ws, As, Bs, scale, ranks, ids_t, M, d_in, d_out, r_max, n, segs,
                            ys, L.LORA_F32, mode, ws, nb)
        torch.cuda.synchronize()
        return ys

    own = call()
    segs = L.Segments(M, n)
    L.lora_build_segments(ids, M, n, segs)
    for y, y0 in zip(call(segs=segs), own):
        assert torch.equal(y, y0)
    for y, y0 in zip(call(mode=L.LORA_MODE_DECODE | L.LORA_MODE_CHECKED), own):
        assert torch.equal(y, y0)
    for y, ref in zip(own, refs(base, projs)):
        assert_parity(y.cpu().numpy(), ref, "caller segments")
    bad = base.ids.copy()
    bad[M // 3] = n
    ys = [torch.full((M, d_out), 3.0, dtype=torch.float32, device="cuda") for _ in range(2)]
    with pytest.raises(L.LoraError) as e:
        L.lora_linear_multi(x, Ws, As, Bs, scale, ranks, torch.from_numpy(bad).cuda(), M, d_in,
                            d_out, r_max, n, None, ys, L.LORA_F32,
                            L.LORA_MODE_DECODE | L.LORA_MODE_CHECKED, ws, nb)
    assert e.value.status == 8  # LORA_ERR_BAD_ID
    torch.cuda.synchronize()
    assert all(bool((y == 3.0).all()) for y in ys)  # nothing was enqueued


def _sk_group(M, K, N, n_proj):
    """Projections per merged stream-K launch (0: the batch does not take stream-K): the rule
    the library states, restated here to name what each seeded case exercises."""
    def use(g):
        if M <= 256 or M > 1024 or K % 128 or N % 8:
            return False
        n_tm, n_tn = (M + 255) // 256, g * ((N + 255) // 256)
        if n_tm * n_tn >= 192:
            return False
        return n_tn * (K // 32) >= 8 * ((256 // n_tm) // 8 * 8)
    if not use(1):
        return 0
    g = n_proj
    while g > 1 and not use(g):
        g -= 1
    return g


RANDOM_MULTI = list(range(8))


@pytest.mark.parametrize("i", RANDOM_MULTI)
def test_multi_random_shapes(i):
    """Seeded shapes across the stream-K range: 257-1024 rows, d_out any multiple of 8 from
    1800 to 3072 (ragged last panels), 2-4 projections, r_max 1-64, pools of 4-300 adapters."""
    from rank_adapter_gemm_sgmv_amd import lora as L

    rng = np.random.default_rng(600 + i)
    M = int(rng.integers(257, 1025))
    d_out = int(rng.integers(225, 385)) * 8
    n_proj = int(rng.integers(2, 5))
    r_max = int(rng.integers(1, 65))
    n = int(rng.integers(4, 301))
    g = _sk_group(M, 4096, d_out, n_proj)
    log(f"multi random {i}: M={M} d_out={d_out} projections {n_proj} r_max={r_max} n={n} group {g}")
    base, projs = multi_case(610 + i, M, 4096, d_out, n, r_max, n_proj)
    out, singles = run_multi(base, projs, L.LORA_MODE_DECODE)
    for p, (y, ref) in enumerate(zip(out, refs(base, projs))):
        assert_parity(y, ref, f"case {i} projection {p} (group {g})")

"""Pins that tie the CPU oracle to facts fixed outside it (collected by test_oracle_pins.py).

Each ``pin_*`` takes an ``Orc`` (the oracle bound to one compiled library) and raises
AssertionError on a mismatch, so the same pins run against the real oracle and against
deliberately broken copies of it (test_oracle_mutants.py).

Sources, cited by title and section:
  [P1] "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to)
  [P2] "Serving Many LoRA Adapters From One Base Model" (ai-tldr.dev)
  [P3] "Multi-LoRA Serving: Sharing One GPU Across Adapters" (cloudai.pt)

What pins what:
  * merge identity, exact: [P1] "Why can't you just merge LoRA weights into the base
    model?" and [P2] "Going deeper" state that folding the adapter into the base, W' = W + BA
    (scaled), gives the same layer.  On tiny dyadic inputs the exact rational value of
    x W'_i is computed with fractions.Fraction, and the oracle's float32 result must lie
    within the standard float32 summation bound gamma_n * sum|terms| of it.
  * integer-exact: with small integer inputs and alpha / r = 2 or 3 every float32 operation
    is exact, so the oracle must equal numpy's int64 matrix products bit for bit.
  * merged / single-adapter in float64: numpy's float64 matmul of the merged weight, or of
    the unmerged chain with one adapter for all rows, within the float32 bound.
  * base-only rows: adapter=None in [P2] "A worked example: the memory math" -- those rows
    equal numpy's float64 x W within the bound, and stay bit-identical whatever the other
    rows' ids are.
  * zero padding is storage: [P1] "Where does multi-LoRA serving actually break?" (rank
    padding) -- padding a rank-r adapter out to r_max = 64 with zeros changes no bit.
  * the scale is alpha / r: doubling alpha doubles the delta bit-exactly (W = 0); doubling
    both alpha and r changes nothing.
  * rows are independent: permuting rows permutes the output bit-exactly.
  * segments: equal to Python's stable sorted() plus numpy bincount / cumsum.
  * quantized base ([P1] "Where does multi-LoRA serving actually break?", item 4): the fp8
    E4M3 decode equals torch's float8_e4m3fn conversion on every non-NaN code and gives the
    values the OCP 8-bit floating point specification fixes for E4M3 (largest normal 448,
    smallest normal 2^-6, smallest subnormal 2^-9, NaN at S.1111.111, -0 at 0x80); with unit
    scales the fp8 layer equals the bf16 layer on the same (exactly representable) weights,
    bit for bit; a power-of-two column scale scales the base term exactly; and the fp8 layer
    agrees with numpy float64 on the dequantized weight within the float32 bound.
  * MoE-LoRA ([P3] "MoE Models Raise the Bar"): one expert, top-1, unit weights is the dense
    layer bit for bit; every routed slot is the dense layer on that expert's weights and
    adapter pair times its routing weight, bit for bit; the merged weight W_e + s A_ie B_ie
    per (expert, adapter) exactly on integer inputs; empty slots are zero rows; doubling
    the routing weights doubles the output exactly; float64 within the float32 bound.
"""

from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import Optional

import numpy as np

from synth import random_case

U32 = 2.0 ** -24  # unit roundoff of float32


def gamma(n: int) -> float:
    return n * U32 / (1.0 - n * U32)


@dataclasses.dataclass
class Orc:
    """The oracle module bound to one compiled library."""

    mod: object
    lib: Optional[object] = None

    def linear(self, *a, **k):
        return self.mod.lora_linear(*a, lib=self.lib, **k)

    def shrink(self, *a, **k):
        return self.mod.lora_shrink(*a, lib=self.lib, **k)

    def expand(self, *a, **k):
        return self.mod.lora_expand(*a, lib=self.lib, **k)

    def segments(self, *a, **k):
        return self.mod.build_segments(*a, lib=self.lib, **k)

    def linear_fp8w(self, *a, **k):
        return self.mod.lora_linear_fp8w(*a, lib=self.lib, **k)

    def fp8_decode(self, *a, **k):
        return self.mod.fp8_e4m3_decode(*a, lib=self.lib, **k)

    def moe(self, *a, **k):
        return self.mod.moe_lora_linear(*a, lib=self.lib, **k)


def _int_case(seed, M, d_in, d_out, n, r_max, scale_int=2, base_frac=0.25):
    """Small-integer inputs: every float32 product and partial sum below is exact."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, size=(M, d_in)).astype(np.float32)
    W = rng.integers(-3, 4, size=(d_in, d_out)).astype(np.float32)
    A = rng.integers(-3, 4, size=(n, d_in, r_max)).astype(np.float32)
    B = rng.integers(-3, 4, size=(n, r_max, d_out)).astype(np.float32)
    ranks = rng.integers(1, r_max + 1, size=n).astype(np.int32)
    for i, r in enumerate(ranks):
        A[i, :, r:] = 0
        B[i, r:, :] = 0
    alpha = (scale_int * ranks).astype(np.float32)
    ids = rng.integers(0, n, size=M).astype(np.int32)
    ids[rng.random(M) < base_frac] = -1
    return x, W, A, B, alpha, ranks, ids


def _abs_bound(x, W, A, B, s, ids, extra_ops):
    """gamma_{d_in + r_max + extra} * (sum_k |x W| + |s| sum_j (sum_k |x A|) |B|), float64."""
    x, W, A, B = (np.asarray(v, np.float64) for v in (x, W, A, B))
    M, d_in = x.shape
    r_max = A.shape[2]
    base = np.abs(x) @ np.abs(W)
    lora = np.zeros_like(base)
    for m in range(M):
        i = int(ids[m])
        if i >= 0:
            T = np.abs(x[m]) @ np.abs(A[i])
            lora[m] = abs(float(s[i])) * (T @ np.abs(B[i]))
    return gamma(d_in + r_max + extra_ops) * (base + lora) * 1.001 + 1e-30


# ---------------------------------------------------------------------------------------


def pin_exact_merged_rational(orc: Orc) -> None:
    """Oracle vs the exact rational value of x_m (W + s_i A_i B_i) on tiny shapes."""
    for seed in range(8):
        M, d_in, d_out = 1 + seed % 5, 2 + seed % 6, 1 + (3 * seed) % 7
        n, r_max = 1 + seed % 3, 1 + seed % 3
        w = random_case(100 + seed, M, d_in, d_out, n, r_max, storage="f32", base_frac=0.3,
                        w_std=0.5, ab_std=0.5)
        rng = np.random.default_rng(seed)
        alpha = rng.uniform(0.5, 40.0, size=n).astype(np.float32)
        p = w.projections[0]
        y = orc.linear(p.x, p.W, p.A, p.B, alpha, w.ranks, w.ids)
        s_exact = [Fraction(float(alpha[i])) / int(w.ranks[i]) for i in range(n)]
        bound = _abs_bound(p.x, p.W, p.A, p.B, alpha / w.ranks, w.ids, 4)
        for m in range(M):
            i = int(w.ids[m])
            for c in range(d_out):
                # merged weight column c, exactly: W[k][c] + s_i * sum_j A_i[k][j] B_i[j][c]
                acc = Fraction(0)
                for k in range(d_in):
                    wk = Fraction(float(p.W[k, c]))
                    if i >= 0:
                        wk += s_exact[i] * sum(Fraction(float(p.A[i, k, j])) *
                                               Fraction(float(p.B[i, j, c])) for j in range(r_max))
                    acc += Fraction(float(p.x[m, k])) * wk
                err = abs(Fraction(float(y[m, c])) - acc)
                assert err <= Fraction(float(bound[m, c])), (seed, m, c, float(err))


def pin_integer_exact(orc: Orc) -> None:
    """Integer inputs, alpha / r in {2, 3}: bit-equal to numpy int64 products."""
    for seed, scale_int in ((1, 2), (2, 3), (3, 2)):
        M, d_in, d_out, n, r_max = 40, 48, 40, 5, 8
        x, W, A, B, alpha, ranks, ids = _int_case(seed, M, d_in, d_out, n, r_max, scale_int)
        y = orc.linear(x, W, A, B, alpha, ranks, ids)
        xi, Wi, Ai, Bi = (v.astype(np.int64) for v in (x, W, A, B))
        ref = xi @ Wi
        for m in range(M):
            i = int(ids[m])
            if i >= 0:
                ref[m] += scale_int * ((xi[m] @ Ai[i]) @ Bi[i])
        assert np.array_equal(y, ref.astype(np.float32)), seed
        # the shrink alone: t = x A_i, zero rows for id -1
        t = orc.shrink(x, A, ids)
        tref = np.zeros((M, r_max), np.int64)
        for m in range(M):
            if ids[m] >= 0:
                tref[m] = xi[m] @ Ai[ids[m]]
        assert np.array_equal(t, tref.astype(np.float32)), seed
        # the expand alone on top of the base term
        y2 = orc.expand(t, B, alpha, ranks, ids, (xi @ Wi).astype(np.float32))
        assert np.array_equal(y2, ref.astype(np.float32)), seed


def pin_merged_float64(orc: Orc) -> None:
    """x_m (W + s_i A_i B_i) in float64 (numpy matmul) within the float32 bound."""
    for seed in (11, 12):
        w = random_case(seed, 32, 96, 80, 6, 16, storage="bf16", base_frac=0.2)
        rng = np.random.default_rng(seed)
        alpha = rng.uniform(1.0, 64.0, size=6).astype(np.float32)
        wf = w.as_f32()
        p = wf.projections[0]
        y = orc.linear(w.projections[0].x, w.projections[0].W, w.projections[0].A,
                       w.projections[0].B, alpha, w.ranks, w.ids)
        s = alpha.astype(np.float64) / w.ranks
        x64, W64 = p.x.astype(np.float64), p.W.astype(np.float64)
        ref = np.empty_like(y, dtype=np.float64)
        for m in range(w.M):
            i = int(w.ids[m])
            Wm = W64 if i < 0 else W64 + s[i] * (p.A[i].astype(np.float64) @ p.B[i].astype(np.float64))
            ref[m] = x64[m] @ Wm
        bound = _abs_bound(p.x, p.W, p.A, p.B, s, w.ids, 4)
        # the merged weight is itself summed in float64: allow its (tiny) rounding too
        assert np.all(np.abs(y - ref) <= bound + 1e-12 * np.abs(ref)), seed


def pin_single_adapter_float64(orc: Orc) -> None:
    """All rows on one adapter: numpy float64 x W + s (x A_i) B_i within the bound."""
    w = random_case(21, 24, 64, 48, 3, 16, ranks=[16, 5, 9], storage="f32")
    p = w.projections[0]
    for i in range(3):
        ids = np.full(w.M, i, np.int32)
        y = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, ids)
        s = float(w.alpha[i]) / float(w.ranks[i])
        x64 = p.x.astype(np.float64)
        ref = x64 @ p.W + s * ((x64 @ p.A[i]) @ p.B[i])
        bound = _abs_bound(p.x, p.W, p.A, p.B, w.alpha / w.ranks, ids, 4)
        assert np.all(np.abs(y - ref) <= bound), i


def pin_base_rows(orc: Orc) -> None:
    """id -1 rows: float64 x W within the bound, and independent of the other rows' ids."""
    w = random_case(31, 30, 72, 40, 4, 8, storage="f32", base_frac=0.4)
    p = w.projections[0]
    y = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    base = w.ids == -1
    assert base.any() and (~base).any()
    ref = p.x.astype(np.float64) @ p.W
    bound = gamma(72 + 2) * (np.abs(p.x).astype(np.float64) @ np.abs(p.W)) * 1.001
    assert np.all(np.abs(y[base] - ref[base]) <= bound[base])
    # LoRA rows must differ from the bare base (the delta is not dropped)
    assert np.all(np.abs(y[~base] - ref[~base]).max(axis=1) > 10 * bound[~base].max(axis=1))
    # other rows' adapters do not leak into base rows
    ids2 = w.ids.copy()
    ids2[~base] = (ids2[~base] + 1) % 4
    y2 = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, ids2)
    assert np.array_equal(y2[base], y[base])
    # an all-base batch (every request adapter=None)
    y3 = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, np.full(w.M, -1, np.int32))
    assert np.all(np.abs(y3 - ref) <= bound)


def pin_zero_padding(orc: Orc) -> None:
    """Rank-r adapters stored at r_max = 8 or padded with zeros to r_max = 64: same bits."""
    w = random_case(41, 20, 64, 56, 5, 8, storage="bf16", base_frac=0.2)
    p = w.projections[0]
    n = w.n_adapters
    A64 = np.zeros((n, p.d_in, 64), np.uint16)
    B64 = np.zeros((n, 64, p.d_out), np.uint16)
    A64[:, :, :8] = p.A
    B64[:, :8, :] = p.B
    y8 = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    y64 = orc.linear(p.x, p.W, A64, B64, w.alpha, w.ranks, w.ids)
    assert np.array_equal(y8, y64)
    t8 = orc.shrink(p.x, p.A, w.ids)
    t64 = orc.shrink(p.x, A64, w.ids)
    assert np.array_equal(t64[:, :8], t8) and not np.any(t64[:, 8:])


def pin_scale(orc: Orc) -> None:
    """W = 0 isolates the delta: doubling alpha doubles it; doubling alpha and r is a no-op."""
    w = random_case(51, 16, 48, 32, 3, 16, storage="f32", base_frac=0.25)
    p = w.projections[0]
    W0 = np.zeros_like(p.W)
    d1 = orc.linear(p.x, W0, p.A, p.B, w.alpha, w.ranks, w.ids)
    d2 = orc.linear(p.x, W0, p.A, p.B, 2 * w.alpha, w.ranks, w.ids)
    assert np.array_equal(d2, 2 * d1)
    d3 = orc.linear(p.x, W0, p.A, p.B, 2 * w.alpha, 2 * w.ranks, w.ids)
    assert np.array_equal(d3, d1)
    assert not np.any(d1[w.ids == -1]) and np.all(np.abs(d1[w.ids >= 0]).max(axis=1) > 0)


def pin_row_permutation(orc: Orc) -> None:
    """Permuting the rows of (x, ids) permutes y, bit for bit."""
    w = random_case(61, 28, 40, 24, 4, 8, storage="bf16", base_frac=0.2)
    p = w.projections[0]
    y = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids)
    perm = np.random.default_rng(61).permutation(w.M)
    yp = orc.linear(p.x[perm], p.W, p.A, p.B, w.alpha, w.ranks, w.ids[perm])
    assert np.array_equal(yp, y[perm])
    # computing a subset of rows gives the same bits as the full call
    rows = np.array([5, 0, 27, 5], np.int32)
    ys = orc.linear(p.x, p.W, p.A, p.B, w.alpha, w.ranks, w.ids, rows=rows)
    assert np.array_equal(ys, y[rows])


def reference_segments(ids, n_adapters: int, tile_rows: int) -> dict:
    """Python's stable sort and numpy counting, written independently of oracle.c."""
    ids = np.asarray(ids, np.int64)
    M = len(ids)
    perm = sorted(range(M), key=lambda m: (ids[m] == -1, ids[m]))
    counts = np.bincount(ids[ids >= 0], minlength=n_adapters) if M else np.zeros(n_adapters, int)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    seg_adapter = np.nonzero(counts)[0]
    tiles = [(p, a) for a in seg_adapter for p in range(offsets[a], offsets[a + 1], tile_rows)]
    meta = [len(seg_adapter), int(counts.sum()), 0, len(tiles)]
    return dict(perm=np.array(perm, np.int32), offsets=offsets.astype(np.int32),
                seg_adapter=seg_adapter.astype(np.int32),
                tiles=np.array(tiles, np.int32).reshape(-1, 2), meta=np.array(meta, np.int32))


def pin_segments(orc: Orc) -> None:
    rng = np.random.default_rng(71)
    cases = [np.array([], np.int32), np.full(5, -1, np.int32), np.full(37, 2, np.int32),
             np.array([0], np.int32)]
    for _ in range(12):
        M = int(rng.integers(1, 300))
        n = int(rng.integers(1, 70))
        ids = rng.integers(-1, n, size=M).astype(np.int32)
        cases.append(ids)
    for ids in cases:
        n = int(ids.max()) + 1 if len(ids) and ids.max() >= 0 else 3
        for tile_rows in (1, 4, 16):
            got = orc.segments(ids, n, tile_rows)
            ref = reference_segments(ids, n, tile_rows)
            for key in ("perm", "offsets", "seg_adapter", "tiles", "meta"):
                assert np.array_equal(got[key], ref[key]), (key, ids, tile_rows)


# ---------------------------------------------------------------------------------------
# quantized (fp8 E4M3) base


def _fp8_case(seed, M, d_in, d_out, n, r_max, scale=None):
    """A random case plus fp8 codes W8[d_out, d_in] (every non-NaN code drawn uniformly) and
    column scales; W8 is an input, drawn, not computed from a float weight."""
    from synth import fp8_base

    w = random_case(seed, M, d_in, d_out, n, r_max, storage="f32", base_frac=0.25)
    W8, w_scale = fp8_base(seed, d_in, d_out, uniform_codes=True)
    if scale is not None:
        w_scale = np.full(d_out, scale, np.float32)
    return w, W8, w_scale


def pin_fp8_decode(orc: Orc) -> None:
    import torch

    codes = np.arange(256, dtype=np.uint8)
    got = orc.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF] and np.all(np.isnan(got[nan]))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # values the format fixes
    fixed = {0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0xC0: -2.0, 0x00: 0.0}
    for c, v in fixed.items():
        assert got[c] == v, (hex(c), got[c], v)
    assert got[0x80] == 0.0 and np.signbit(got[0x80])
    # strictly increasing over the positive codes
    assert np.all(np.diff(got[0x00:0x7F].astype(np.float64)) > 0)


def pin_fp8_equals_bf16_layer(orc: Orc) -> None:
    """Unit scales: the fp8 layer is the bf16/fp32 layer on W[k, c] = dec(W8[c, k])."""
    for seed, (M, d_in, d_out, n, r_max) in enumerate([(9, 40, 24, 3, 8), (5, 16, 72, 2, 4)]):
        w, W8, w_scale = _fp8_case(900 + seed, M, d_in, d_out, n, r_max, scale=1.0)
        p = w.projections[0]
        W = np.ascontiguousarray(orc.fp8_decode(W8).T)
        y8 = orc.linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, w.ids)
        y = orc.linear(p.x, W, p.A, p.B, w.alpha, w.ranks, w.ids)
        assert np.array_equal(y8, y)


def pin_fp8_scale(orc: Orc) -> None:
    """A power-of-two scale on column c multiplies the base term of column c exactly."""
    w, W8, _ = _fp8_case(910, 7, 32, 20, 2, 8, scale=1.0)
    p = w.projections[0]
    base = np.full(w.M, -1, np.int32)
    y1 = orc.linear_fp8w(p.x, W8, np.ones(20, np.float32), p.A, p.B, w.alpha, w.ranks, base)
    sc = (2.0 ** np.arange(-4, 16)).astype(np.float32)
    y2 = orc.linear_fp8w(p.x, W8, sc, p.A, p.B, w.alpha, w.ranks, base)
    assert np.array_equal(y2, y1 * sc[None, :])


def pin_fp8_float64(orc: Orc) -> None:
    """The fp8 layer vs numpy float64 on the dequantized weight, within the float32 bound."""
    w, W8, w_scale = _fp8_case(920, 11, 64, 48, 4, 16)
    p = w.projections[0]
    Wd = (orc.fp8_decode(W8).astype(np.float64) * w_scale[:, None].astype(np.float64)).T
    y = orc.linear_fp8w(p.x, W8, w_scale, p.A, p.B, w.alpha, w.ranks, w.ids)
    x, A, B = (np.asarray(v, np.float64) for v in (p.x, p.A, p.B))
    s = w.alpha.astype(np.float64) / w.ranks
    ref = x @ Wd
    for m in range(w.M):
        i = int(w.ids[m])
        if i >= 0:
            ref[m] += s[i] * ((x[m] @ A[i]) @ B[i])
    bound = _abs_bound(p.x, Wd, p.A, p.B, s, w.ids, 5)
    assert np.all(np.abs(y - ref) <= bound)


# ---------------------------------------------------------------------------------------
# MoE-LoRA


def _moe(seed, M=9, top_k=2, E=4, d_in=24, d_out=20, n=3, r_max=4, empty=0.2):
    from synth import moe_case

    return moe_case(seed, M, top_k, E, d_in, d_out, n, r_max, base_frac=0.25, empty_frac=empty,
                    storage="f32")


def pin_moe_single_expert_is_dense(orc: Orc) -> None:
    from synth import moe_case

    w = moe_case(930, 11, 1, 1, 32, 24, 3, 8, base_frac=0.3, storage="f32")
    y = orc.moe(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids)
    ref = orc.linear(w.x, w.W[0], w.A[:, 0], w.B[:, 0], w.alpha, w.ranks, w.ids)
    assert np.array_equal(y[:, 0, :], ref)


def pin_moe_slots_are_dense_rows(orc: Orc) -> None:
    """y[m, j] = w[m, j] * dense(x, W_e, A[:, e], B[:, e])[m] for e = topk_ids[m, j]."""
    w = _moe(931)
    y = orc.moe(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids, w.topk_w)
    dense = [orc.linear(w.x, w.W[e], np.ascontiguousarray(w.A[:, e]), np.ascontiguousarray(w.B[:, e]),
                        w.alpha, w.ranks, w.ids) for e in range(w.n_experts)]
    for m in range(w.M):
        for j in range(w.top_k):
            e = int(w.topk_ids[m, j])
            if e < 0:
                assert not np.any(y[m, j])
            else:
                assert np.array_equal(y[m, j], w.topk_w[m, j] * dense[e][m])
    assert (w.topk_ids < 0).any() and (w.topk_ids >= 0).any()


def pin_moe_weight_linearity(orc: Orc) -> None:
    w = _moe(932)
    y1 = orc.moe(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids, w.topk_w)
    y2 = orc.moe(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids, 2 * w.topk_w)
    y0 = orc.moe(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids)
    assert np.array_equal(y2, 2 * y1)
    nz = w.topk_ids >= 0
    assert np.array_equal(y1[nz], w.topk_w[nz][:, None] * y0[nz])


def pin_moe_merged_integer(orc: Orc) -> None:
    """The merged-weight identity per (expert, adapter), exactly: small-integer inputs,
    alpha / r in {2, 3} and power-of-two routing weights make every float32 step exact, so
    y[m, j] = w[m, j] * x_m (W_e + s_i A[i, e] B[i, e]) in int64 arithmetic, bit for bit."""
    rng = np.random.default_rng(934)
    for scale_int in (2, 3):
        M, top_k, E, d_in, d_out, n, r_max = 23, 3, 5, 32, 24, 4, 8
        x = rng.integers(-3, 4, size=(M, d_in)).astype(np.float32)
        W = rng.integers(-3, 4, size=(E, d_in, d_out)).astype(np.float32)
        A = rng.integers(-3, 4, size=(n, E, d_in, r_max)).astype(np.float32)
        B = rng.integers(-3, 4, size=(n, E, r_max, d_out)).astype(np.float32)
        ranks = rng.integers(1, r_max + 1, size=n).astype(np.int32)
        for i, r in enumerate(ranks):
            A[i, :, :, r:] = 0
            B[i, :, r:, :] = 0
        alpha = (scale_int * ranks).astype(np.float32)
        ids = rng.integers(-1, n, size=M).astype(np.int32)
        topk = np.stack([rng.permutation(E)[:top_k] for _ in range(M)]).astype(np.int32)
        topk[rng.random((M, top_k)) < 0.15] = -1
        tw = (2.0 ** rng.integers(-3, 2, size=(M, top_k))).astype(np.float32)
        y = orc.moe(x, W, A, B, alpha, ranks, ids, topk, tw)
        xi, Wi, Ai, Bi = (v.astype(np.int64) for v in (x, W, A, B))
        for m in range(M):
            for j in range(top_k):
                e = int(topk[m, j])
                if e < 0:
                    assert not np.any(y[m, j])
                    continue
                i = int(ids[m])
                Wm = Wi[e] + (scale_int * (Ai[i, e] @ Bi[i, e]) if i >= 0 else 0)
                ref = (xi[m] @ Wm).astype(np.float64) * float(tw[m, j])
                assert np.array_equal(y[m, j], ref.astype(np.float32)), (scale_int, m, j)


def pin_moe_float64(orc: Orc) -> None:
    w = _moe(933, M=7, top_k=3, E=5, d_in=40, d_out=28, n=4, r_max=8, empty=0.1)
    y = orc.moe(w.x, w.W, w.A, w.B, w.alpha, w.ranks, w.ids, w.topk_ids, w.topk_w)
    x, W, A, B = (np.asarray(v, np.float64) for v in (w.x, w.W, w.A, w.B))
    s = w.alpha.astype(np.float64) / w.ranks
    for m in range(w.M):
        for j in range(w.top_k):
            e = int(w.topk_ids[m, j])
            if e < 0:
                assert not np.any(y[m, j])
                continue
            i = int(w.ids[m])
            ref = x[m] @ W[e]
            mag = np.abs(x[m]) @ np.abs(W[e])
            if i >= 0:
                ref = ref + s[i] * ((x[m] @ A[i, e]) @ B[i, e])
                mag = mag + abs(s[i]) * ((np.abs(x[m]) @ np.abs(A[i, e])) @ np.abs(B[i, e]))
            ref = ref * float(w.topk_w[m, j])
            bound = gamma(w.d_in + w.r_max + 6) * mag * abs(float(w.topk_w[m, j])) * 1.001 + 1e-30
            assert np.all(np.abs(y[m, j] - ref) <= bound)


ALL_PINS = [pin_exact_merged_rational, pin_integer_exact, pin_merged_float64,
            pin_single_adapter_float64, pin_base_rows, pin_zero_padding, pin_scale,
            pin_row_permutation, pin_segments, pin_fp8_decode, pin_fp8_equals_bf16_layer,
            pin_fp8_scale, pin_fp8_float64, pin_moe_single_expert_is_dense,
            pin_moe_slots_are_dense_rows, pin_moe_weight_linearity, pin_moe_merged_integer,
            pin_moe_float64]

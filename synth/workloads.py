"""Seeded synthetic workloads for the multi-LoRA batched linear.

The layer that consumes these inputs is y = xW + (x A_i) B_i (alpha_i / r_i), where every
row of a mixed batch names its own adapter i (or -1 for the bare base) -- described in
"Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), section "Why can't you
just merge LoRA weights into the base model?".  This module draws the inputs and nothing
else: activations x, one shared base weight W, a stacked pool of adapters padded to one
static maximum rank (same page, "What does a working multi-LoRA config look like?"), the
per-adapter rank and alpha, and the row -> adapter id vector ("How does one batch run 30
different adapters at once?").  It computes none of the layer's arithmetic; the CPU oracle
and the GPU library both receive exactly the arrays produced here.

Storage layout (row-major, what the GPU library takes):
  x  [M, d_in]                  W  [d_in, d_out]
  A  [n_adapters, d_in, r_max]  B  [n_adapters, r_max, d_out]
Entries of adapter i beyond its own rank r_i (columns of A_i, rows of B_i) are zero.

Values are drawn with numpy's PCG64 generator (seed = 1000 + config number for the five
named workloads), as float32 normals times the standard deviation, and then rounded to
bfloat16 with round-to-nearest-even on the bit pattern.  Config 1 keeps its float32
values; ``Workload.as_bf16()`` gives the rounded copy the GPU receives.

Draw order: ids, then ranks, then every x, then per projection W, A, B.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------------------
# bfloat16 bit patterns
# --------------------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round half to even) and return the uint16 bits.

    Integer method: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits.
    Only finite inputs are expected (no NaN handling).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32
    )


# --------------------------------------------------------------------------------------
# Containers
# --------------------------------------------------------------------------------------


@dataclasses.dataclass
class Projection:
    """One adapted linear: activations, shared base weight and its adapter pool."""

    name: str
    x: np.ndarray  # [M, d_in]     float32 or uint16 (bf16 bits)
    W: np.ndarray  # [d_in, d_out]
    A: np.ndarray  # [n, d_in, r_max]
    B: np.ndarray  # [n, r_max, d_out]

    @property
    def d_in(self) -> int:
        return int(self.W.shape[0])

    @property
    def d_out(self) -> int:
        return int(self.W.shape[1])


@dataclasses.dataclass
class Workload:
    """A batch of rows with their adapter ids plus one or more adapted projections."""

    name: str
    ids: np.ndarray  # int32 [M]; -1 = base only
    ranks: np.ndarray  # int32 [n]; true rank of each adapter, 1 <= r_i <= r_max
    alpha: np.ndarray  # float32 [n]
    r_max: int
    projections: List[Projection]
    storage: str  # "bf16" (uint16 bit patterns) or "f32"
    seed: int

    @property
    def M(self) -> int:
        return int(self.ids.shape[0])

    @property
    def n_adapters(self) -> int:
        return int(self.ranks.shape[0])

    def as_bf16(self) -> "Workload":
        """The same workload with every float tensor rounded to bf16 bits (no-op if bf16)."""
        if self.storage == "bf16":
            return self
        projs = [
            Projection(p.name, f32_to_bf16_bits(p.x), f32_to_bf16_bits(p.W),
                       f32_to_bf16_bits(p.A), f32_to_bf16_bits(p.B))
            for p in self.projections
        ]
        return dataclasses.replace(self, projections=projs, storage="bf16")

    def as_f32(self) -> "Workload":
        """Float32 view of every tensor (exact widening when stored as bf16)."""
        if self.storage == "f32":
            return self
        projs = [
            Projection(p.name, bf16_bits_to_f32(p.x), bf16_bits_to_f32(p.W),
                       bf16_bits_to_f32(p.A), bf16_bits_to_f32(p.B))
            for p in self.projections
        ]
        return dataclasses.replace(self, projections=projs, storage="f32")


# --------------------------------------------------------------------------------------
# Draw helpers
# --------------------------------------------------------------------------------------


def zipf_probs(n: int, s: float) -> np.ndarray:
    """Truncated Zipf law over ids 0..n-1: p(id) proportional to (id + 1) ** -s."""
    w = np.arange(1, n + 1, dtype=np.float64) ** (-float(s))
    return w / w.sum()


def _normal(rng: np.random.Generator, shape: Sequence[int], std: float, storage: str,
            chunk_rows: int = 1 << 22) -> np.ndarray:
    """float32 normals * std, rounded to bf16 bits when storage == 'bf16'.

    Drawn in chunks along the flattened array so large pools do not need a float32 copy
    of the whole tensor; the drawn stream is the same as one draw of the full size.
    """
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16 if storage == "bf16" else np.float32)
    stdf = np.float32(std)
    for s in range(0, total, chunk_rows):
        e = min(total, s + chunk_rows)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= stdf
        out[s:e] = f32_to_bf16_bits(v) if storage == "bf16" else v
    return out.reshape(shape)


def _zero_padding(A: np.ndarray, B: np.ndarray, ranks: np.ndarray) -> None:
    """Zero A[i, :, r_i:] and B[i, r_i:, :] in place (padding is storage, not values)."""
    r_max = A.shape[2]
    for i, r in enumerate(ranks.tolist()):
        if r < r_max:
            A[i, :, r:] = 0
            B[i, r:, :] = 0


def compact_pool(A: np.ndarray, B: np.ndarray, ranks: np.ndarray):
    """The same adapters stored at their own rank instead of padded to r_max: a storage
    layout, no arithmetic.  Adapter i occupies w_i = round_up(r_i, 8) rank rows (its rows
    r_i .. w_i - 1 zero).  Returns (A_c, B_c, offsets, pool_rows): A_c is flat with A_i =
    A[i, :, :w_i] (a [d_in][w_i] block, columns past r_max zero) at element offsets[i] * d_in,
    B_c is [pool_rows, d_out] with B_i = B[i, :w_i, :] at rows offsets[i] ..,
    offsets[i] = w_0 + ... + w_{i-1}."""
    n, d_in, r_max = A.shape
    d_out = B.shape[2]
    r = np.asarray(ranks, dtype=np.int64)
    w = (r + 7) // 8 * 8
    offsets = np.concatenate([[0], np.cumsum(w)[:-1]]).astype(np.int32)
    pool_rows = int(w.sum())
    A_c = np.zeros(pool_rows * d_in, dtype=A.dtype)
    B_c = np.zeros((pool_rows, d_out), dtype=B.dtype)
    for i in range(n):
        o, ri, wi = int(offsets[i]), int(r[i]), int(w[i])
        blk = np.zeros((d_in, wi), dtype=A.dtype)
        blk[:, :ri] = A[i, :, :ri]
        A_c[o * d_in:(o + wi) * d_in] = blk.reshape(-1)
        B_c[o:o + ri] = B[i, :ri, :]
    return A_c, B_c, offsets, pool_rows


def fp8_base(seed: int, d_in: int, d_out: int, uniform_codes: bool = False, std: float = 0.02):
    """A base weight stored as fp8 E4M3 codes: W8[d_out, d_in] (uint8; each output column's
    d_in codes contiguous) and per-column scales w_scale[d_out] (float32), drawn from a stream
    of their own (PCG64 seeded with [seed, 8]).  No arithmetic of the layer: the codes are an
    input.

    default: values N(0, 1) * 64 clipped to +-448, converted to E4M3 by torch's float8_e4m3fn
    cast, and scales std / 64 * U[0.75, 1.25), so the effective weight w_scale * dec(W8) has
    about the spread of the bf16 workloads' N(0, std) weights.
    uniform_codes: every code other than the two NaN codes, uniformly (subnormals, zeros and
    the largest values included).
    """
    import torch

    rng = np.random.Generator(np.random.PCG64([int(seed), 8]))
    if uniform_codes:
        valid = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        W8 = valid[rng.integers(0, len(valid), size=(d_out, d_in))]
    else:
        v = np.clip(rng.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(64.0),
                    -448.0, 448.0)
        W8 = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w_scale = (np.float32(std / 64.0) * rng.uniform(0.75, 1.25, size=d_out)).astype(np.float32)
    return np.ascontiguousarray(W8, dtype=np.uint8), w_scale


def pool_param_count(n_adapters: int, d_in: int, d_out: int, rank: int) -> int:
    """Element count of a stacked pool A[n, d_in, rank] + B[n, rank, d_out]."""
    return int(n_adapters) * int(rank) * (int(d_in) + int(d_out))


# --------------------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------------------

CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny_f32_16x256", M=16, d=[(256, 256)], n=4, rank_choices=[8], r_max=8,
            alpha_per_rank=2.0, ids="uniform_with_base", storage="f32"),
    2: dict(name="decode_qproj_64x4096_32ad_r16", M=64, d=[(4096, 4096)], n=32,
            rank_choices=[16], r_max=16, alpha_per_rank=2.0, ids="uniform", storage="bf16"),
    3: dict(name="decode_hetero_256x4096_128ad_r8-64", M=256, d=[(4096, 4096)], n=128,
            rank_choices=[8, 16, 32, 64], r_max=64, alpha_per_rank=2.0, ids="zipf",
            zipf_s=1.1, base_rows=26, storage="bf16"),
    4: dict(name="prefill_8x512x4096_8ad_r16", M=4096, d=[(4096, 4096)], n=8, rank_choices=[16],
            r_max=16, alpha_per_rank=2.0, ids="blocks", block_rows=512, storage="bf16"),
    5: dict(name="decode_mlp_512_1024ad_r16", M=512,
            d=[(4096, 11008), (4096, 11008), (11008, 4096)], proj_names=["gate", "up", "down"],
            shared_x=[0, 0, 1], n=1024, rank_choices=[16], r_max=16, alpha_per_rank=2.0,
            ids="zipf", zipf_s=1.1, storage="bf16"),
}


def make_workload(config: int, seed: Optional[int] = None) -> Workload:
    """Draw one of the five named workloads (seed defaults to 1000 + config)."""
    spec = CONFIGS[int(config)]
    seed = 1000 + int(config) if seed is None else int(seed)
    rng = np.random.Generator(np.random.PCG64(seed))
    M, n, r_max, storage = spec["M"], spec["n"], spec["r_max"], spec["storage"]

    # ids
    kind = spec["ids"]
    if kind == "uniform_with_base":
        ids = rng.integers(-1, n, size=M)
    elif kind == "uniform":
        ids = rng.integers(0, n, size=M)
    elif kind == "zipf":
        ids = rng.choice(n, size=M, p=zipf_probs(n, spec["zipf_s"]))
        nb = spec.get("base_rows", 0)
        if nb:
            ids[rng.choice(M, size=nb, replace=False)] = -1
    elif kind == "blocks":
        ids = np.repeat(np.arange(M // spec["block_rows"]), spec["block_rows"])
    else:  # pragma: no cover
        raise ValueError(kind)
    ids = ids.astype(np.int32)

    # ranks (drawn only when there is a choice) and alpha = alpha_per_rank * rank
    choices = spec["rank_choices"]
    if len(choices) > 1:
        ranks = rng.choice(np.array(choices), size=n)
    else:
        ranks = np.full(n, choices[0])
    ranks = ranks.astype(np.int32)
    alpha = (np.float32(spec["alpha_per_rank"]) * ranks.astype(np.float32)).astype(np.float32)

    # activations: one x per distinct input width (gate and up share the hidden state)
    dims = spec["d"]
    shared = spec.get("shared_x", list(range(len(dims))))
    xs: Dict[int, np.ndarray] = {}
    for p, key in enumerate(shared):
        if key not in xs:
            xs[key] = _normal(rng, (M, dims[p][0]), 1.0, storage)

    names = spec.get("proj_names", ["proj"] * len(dims))
    projs = []
    for p, (d_in, d_out) in enumerate(dims):
        W = _normal(rng, (d_in, d_out), 0.02, storage)
        A = _normal(rng, (n, d_in, r_max), 0.02, storage)
        B = _normal(rng, (n, r_max, d_out), 0.02, storage)
        _zero_padding(A, B, ranks)
        projs.append(Projection(names[p], xs[shared[p]], W, A, B))
    return Workload(spec["name"], ids, ranks, alpha, r_max, projs, storage, seed)


def random_alpha(seed: int, n_adapters: int, lo: float = 1.0, hi: float = 64.0) -> np.ndarray:
    """Per-adapter alpha_i, uniform over [lo, hi) in float32, from a stream of its own
    (PCG64 seeded with [seed, 1]), so that drawing it changes no other draw of a case.
    alpha_i / r_i is then a different, almost never power-of-two scale for every adapter."""
    rng = np.random.Generator(np.random.PCG64([int(seed), 1]))
    return rng.uniform(lo, hi, size=int(n_adapters)).astype(np.float32)


def random_case(seed: int, M: int, d_in: int, d_out: int, n_adapters: int, r_max: int,
                ranks: Optional[Sequence[int]] = None, ids: Optional[Sequence[int]] = None,
                base_frac: float = 0.2, alpha_per_rank: Optional[float] = None,
                storage: str = "bf16", x_std: float = 1.0, w_std: float = 0.02,
                ab_std: float = 0.02) -> Workload:
    """A small seeded case with free shapes, for parity sweeps and edge cases.

    ids default to uniform over adapters with a fraction ``base_frac`` of rows set to -1;
    ranks default to uniform over [1, r_max]; alpha defaults to ``random_alpha(seed, n)``
    (a distinct scale alpha_i / r_i per adapter), or alpha_per_rank * r_i when given.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if ids is None:
        ids_a = rng.integers(0, n_adapters, size=M)
        if base_frac > 0 and M > 0:
            ids_a[rng.random(M) < base_frac] = -1
    else:
        ids_a = np.asarray(ids)
    ids_a = ids_a.astype(np.int32)
    if ranks is None:
        ranks_a = rng.integers(1, r_max + 1, size=n_adapters)
    else:
        ranks_a = np.asarray(ranks)
    ranks_a = ranks_a.astype(np.int32)
    if alpha_per_rank is None:
        alpha = random_alpha(seed, n_adapters)
    else:
        alpha = (np.float32(alpha_per_rank) * ranks_a.astype(np.float32)).astype(np.float32)
    x = _normal(rng, (M, d_in), x_std, storage)
    W = _normal(rng, (d_in, d_out), w_std, storage)
    A = _normal(rng, (n_adapters, d_in, r_max), ab_std, storage)
    B = _normal(rng, (n_adapters, r_max, d_out), ab_std, storage)
    _zero_padding(A, B, ranks_a)
    return Workload(f"random_{seed}", ids_a, ranks_a, alpha, int(r_max),
                    [Projection("proj", x, W, A, B)], storage, int(seed))


# --------------------------------------------------------------------------------------
# MoE-LoRA inputs
# --------------------------------------------------------------------------------------


@dataclasses.dataclass
class MoeWorkload:
    """A routed expert projection with per-expert adapters ("Multi-LoRA Serving: Sharing One
    GPU Across Adapters", "MoE Models Raise the Bar").  Layouts (row-major):
      x [M, d_in]        W [E, d_in, d_out]          topk_ids [M, top_k] (-1: empty slot)
      A [n, E, d_in, r_max]   B [n, E, r_max, d_out]   topk_w [M, top_k] float32
    ids [M] is each token's adapter (-1: none), ranks / alpha per adapter."""

    name: str
    x: np.ndarray
    W: np.ndarray
    A: np.ndarray
    B: np.ndarray
    ids: np.ndarray
    topk_ids: np.ndarray
    topk_w: np.ndarray
    ranks: np.ndarray
    alpha: np.ndarray
    r_max: int
    seed: int

    @property
    def M(self) -> int:
        return int(self.x.shape[0])

    @property
    def top_k(self) -> int:
        return int(self.topk_ids.shape[1])

    @property
    def n_experts(self) -> int:
        return int(self.W.shape[0])

    @property
    def n_adapters(self) -> int:
        return int(self.ranks.shape[0])

    @property
    def d_in(self) -> int:
        return int(self.W.shape[1])

    @property
    def d_out(self) -> int:
        return int(self.W.shape[2])


def moe_case(seed: int, M: int, top_k: int, n_experts: int, d_in: int, d_out: int,
             n_adapters: int, r_max: int, ranks: Optional[Sequence[int]] = None,
             base_frac: float = 0.2, empty_frac: float = 0.0, zipf_s: float = 0.0,
             name: Optional[str] = None, storage: str = "bf16") -> MoeWorkload:
    """A seeded MoE-LoRA case.  Router (synthetic): each token picks top_k distinct experts,
    uniformly or with Zipf(zipf_s) popularity when zipf_s > 0, routing weights are a softmax
    of N(0, 1) logits over its picks; a fraction empty_frac of slots is left empty (-1).
    Adapter ids uniform over the pool with base_frac of tokens -1; ranks uniform over
    [1, r_max] unless given, alpha from ``random_alpha``.  Values N(0, 1) for x, N(0, 0.02)
    for W, A, B, rounded to bf16; adapter entries past the rank are zero."""
    rng = np.random.Generator(np.random.PCG64([int(seed), 9]))
    E = int(n_experts)
    p = zipf_probs(E, zipf_s) if zipf_s > 0 else np.full(E, 1.0 / E)
    topk = np.stack([rng.choice(E, size=top_k, replace=False, p=p) for _ in range(M)]).astype(np.int32) \
        if M else np.zeros((0, top_k), np.int32)
    logits = rng.standard_normal((M, top_k))
    w = np.exp(logits - logits.max(axis=1, keepdims=True)) if M else logits
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32) if M else w.astype(np.float32)
    if empty_frac > 0 and M:
        topk[rng.random((M, top_k)) < empty_frac] = -1
    ids = rng.integers(0, n_adapters, size=M)
    if base_frac > 0 and M:
        ids[rng.random(M) < base_frac] = -1
    ids = ids.astype(np.int32)
    ranks_a = (rng.integers(1, r_max + 1, size=n_adapters) if ranks is None
               else np.asarray(ranks)).astype(np.int32)
    alpha = random_alpha(seed, n_adapters)
    x = _normal(rng, (M, d_in), 1.0, storage)
    W = _normal(rng, (E, d_in, d_out), 0.02, storage)
    A = _normal(rng, (n_adapters, E, d_in, r_max), 0.02, storage)
    B = _normal(rng, (n_adapters, E, r_max, d_out), 0.02, storage)
    for i, r in enumerate(ranks_a.tolist()):
        if r < r_max:
            A[i, :, :, r:] = 0
            B[i, :, r:, :] = 0
    return MoeWorkload(name or f"moe_{seed}", x, W, A, B, ids, topk, w, ranks_a, alpha,
                       int(r_max), int(seed))


MOE_DECODE = dict(name="moe_decode_64tok_32exp_top4_2880_8ad_r16", M=64, top_k=4, n_experts=32,
                  d_in=2880, d_out=2880, n_adapters=8, r_max=16, base_frac=0.1)


def make_moe_workload(seed: int = 1006) -> MoeWorkload:
    """The MoE decode workload: 64 tokens routed top-4 over 32 experts of 2880 x 2880 (the
    expert width of the GPT-OSS 20B model the pages report MoE-LoRA results on), 8 adapters
    of rank 16 (alpha drawn per adapter), 10% of tokens without an adapter."""
    spec = dict(MOE_DECODE)
    return moe_case(seed, spec.pop("M"), spec.pop("top_k"), spec.pop("n_experts"),
                    spec.pop("d_in"), spec.pop("d_out"), spec.pop("n_adapters"),
                    spec.pop("r_max"), ranks=[16] * 8, **spec)

// shrink.hip -- t = x A_i per row, for all adapters of a mixed batch in one launch.
//
// Source: the adapter "shrink" step of "Multi-LoRA Serving: Sharing One GPU Across
// Adapters" (cloudai.pt), section "MoE Models Raise the Bar", which also names split-K for
// these skinny products; the [B, 4096] x [4096, r] product of "Multi-LoRA Serving: Why 100
// Adapters Fit on One GPU" (dev.to), "How does one batch run 30 different adapters at
// once?", memory-bound on the adapter weights.
//
// Work item = (tile, k-chunk), one workgroup each: a tile is up to LORA_TILE_ROWS (16) rows of
// one adapter a (from the segment builder), a k-chunk is kc consecutive rows of A_a (one
// contiguous block of the padded pool), and each of the four waves takes a quarter of it.
// The product x[tile rows, quarter] A_a[quarter, :] runs on v_mfma_f32_16x16x32_bf16:
// sixteen rows are exactly one MFMA row block, so a tile costs one 16 x 16 accumulator per
// 16 rank columns, and the VALU does almost nothing (a VALU version of this product is
// compute-bound at prefill sizes).  Each A_a byte is read once per tile, each x byte once per
// chunk.
//
// Wave 0 adds the four quarters in wave order (through LDS) and writes the chunk's sums to
// partial[chunk][row][0:r_max] (zero beyond the rank); the consumers add the chunks in
// ascending order, so the result does not depend on scheduling.  Summing the quarters in
// the workgroup leaves a quarter as many chunk sums to write and to read back.
#include "common.h"

namespace lora {

namespace {

constexpr int kKC = 256;           // k rows of A per wave and chunk (128 at r_max 64)
constexpr int kWavesPerBlock = 4;  // waves per workgroup, one quarter of the chunk each
constexpr int kMaxGrid = 1 << 20;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

template <int RM>
struct MfmaShrink {
    static constexpr int NB = RM >= 16 ? RM / 16 : 1;  // 16-column MFMA blocks
    static constexpr int RMP = 16 * NB;                // columns held in LDS (RM 8 -> 16)
    // k rows of A per LDS fill: at most 128, so that a workgroup's four staging areas stay small
    // enough for five workgroups per CU at r_max <= 16 (with 256 rows three fit, and a batch's
    // workgroups ran in two rounds)
    static constexpr int KS = 4096 / RMP < 128 ? 4096 / RMP : 128;
    static constexpr int STEPS = KS / 32;              // 32-deep MFMA steps per fill
    static constexpr int GR = RM / 8;                  // 16-byte groups per row of A_a
    static constexpr int AL = KS * GR / 64;            // 16-byte A loads per lane per fill
    static constexpr int LROW = RMP * 2 + 16;          // LDS bytes per k row (padded)
    static constexpr int LDS = KS * LROW;              // LDS bytes per wave
    static constexpr int KW = RM == 64 ? 128 : kKC;    // k rows per wave and chunk
    static constexpr int FILLS = KW / KS;              // LDS fills per wave and chunk
    static_assert(KS * GR % 64 == 0, "whole loads per lane");
    static_assert(KW % KS == 0 && FILLS >= 1 && FILLS <= 2, "whole fills per wave");
};

// The MFMA steps over one LDS fill: rows kb .. kb + KS of the chunk (x beyond k_hi masked),
// v_mfma_f32_16x16x32_bf16 per 16 rank columns below the rank.
template <class C, int RM>
__device__ __forceinline__ void shrink_mfma_fill(f32x4_t (&acc)[C::NB], const uint4 (&xv)[C::STEPS],
                                                 const lds_char_t *wl, int kb, int k_hi, int g,
                                                 int li, int r) {
#pragma unroll
    for (int st = 0; st < C::STEPS; ++st) {
        const uint4 xs = kb + 32 * st + 8 * g < k_hi ? xv[st] : make_uint4(0, 0, 0, 0);
        const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, xs);
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
            if (16 * b < r) {
                const lds_char_t *q = wl + (32 * st + 8 * g + (li >> 2)) * C::LROW + b * 32 + 8 * (li & 3);
                const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)q);
                const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(q + 4 * C::LROW));
                const bf16x8_t bb = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bb, acc[b], 0, 0, 0);
            }
        }
    }
}

// One workgroup per (tile, k-chunk), one wave per quarter of the chunk:
// t_part[rows of the tile, 0:RM] = x[rows, quarter] A_a[quarter, :] on v_mfma_f32_16x16x32_bf16.  The A operand (16 rows x 32 k) is the tile's x rows, each
// lane loading its 8 consecutive k straight from global memory; the B operand (32 k x 16
// columns) is the adapter's chunk, staged in this wave's own LDS rows as it lies in HBM
// ([k][columns], rows padded by 16 bytes) and read with the transposing LDS read, which
// hands each lane 4 consecutive k of one column.  Column groups at or beyond the adapter's
// rank are written to LDS as zeros.  All global loads are issued unconditionally (clamped
// addresses; out-of-range values are masked at use), so they are all in flight together.
// LAYOUT of the pool's rows of A_a:
//   kPadRM   padded at stride RM (roff and pstride not read);
//   kVarW    rows not RM wide but a multiple of 8: a rank-compact pool (roff names each
//            adapter's first rank row; an adapter of rank r occupies round_up(r, 8) rows) or a
//            padded pool whose stride pstride (< RM) is a multiple of 8;
//   kFlat    a padded pool whose stride is not a multiple of 8: its k rows cannot be read in
//            16-byte groups, so each chunk of A_a is read element by element (eight 2-byte
//            loads in flight per lane) and scattered into the zeroed LDS rows.  A separate
//            instantiation, so that the other layouts keep their registers and occupancy.
enum { kPadRM = 0, kVarW = 1, kFlat = 2 };
// Several pools of one x (lora_linear_multi): item it belongs to pool it / (tiles x chunks),
// which reads A.p[pool] and writes partial.p[pool].
struct ShrinkPools {
    const uint16_t *A[kMaxProj];
    float *partial[kMaxProj];
    int n;
};

template <int RM, int LAYOUT>
__global__ __launch_bounds__(64 * kWavesPerBlock) void shrink_mfma_kernel(
    const uint16_t *__restrict__ x, ShrinkPools pools, const int32_t *__restrict__ ranks,
    const int32_t *__restrict__ roff, int pool_rows, int pstride, int M, int d_in, int n_adapters,
    Seg seg, int n_chunks, int kc) {
    using C = MfmaShrink<RM>;
    __shared__ __attribute__((aligned(16))) char lds[kWavesPerBlock][C::LDS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    char *wg = &lds[wv][0];  // generic pointer for stores (inferred LDS)
    const lds_char_t *wl = (const lds_char_t *)(&lds[wv][0]);
    const int g = lane >> 4, li = lane & 15;
    if constexpr (RM == 8) {  // columns 8..15 of every LDS row stay zero
        for (int r = lane; r < C::KS; r += 64)
            *reinterpret_cast<uint4 *>(wg + r * C::LROW + 16) = make_uint4(0, 0, 0, 0);
    }
    // the block's waves take the four quarters of the chunk's k range; waves 1-3 hand their
    // sums to wave 0 through LDS, which adds them in wave order and writes the chunk's sums
    __shared__ float red[kWavesPerBlock - 1][16 * C::RMP];
    const int per_pool = seg.meta[3] * n_chunks;
    const int total = per_pool * pools.n;
    const int kw = kc / kWavesPerBlock;
    for (int it = blockIdx.x; it < total; it += gridDim.x) {
        const int pi = it / per_pool, ip = it - pi * per_pool;
        const uint16_t *__restrict__ A = pick_proj(pi, pools.A);
        float *__restrict__ partial = pick_proj(pi, pools.partial);
        const int tile = ip / n_chunks, c = ip % n_chunks;
        const int p0 = seg.tiles[2 * tile], a = seg.tiles[2 * tile + 1];
        // (a tile naming no adapter of the pool, possible only in segments a caller built, is
        // skipped by the whole workgroup)
        if (a < 0 || a >= n_adapters) continue;
        const int rows = min(p0 + kTileRows, seg.offsets[a + 1]) - p0;
        constexpr bool VARW = LAYOUT != kPadRM;
        // width of A_a's rows: RM, the padded stride, or (compact) the rank rounded up to 8
        const int width = !VARW ? RM : roff ? RM : pstride;
        int r = ranks ? min(max(ranks[a], 0), width) : width;
        const int row0 = adapter_row0(VARW ? roff : nullptr, pool_rows, a, VARW ? pstride : RM, r);
        // row stride of A_a: in a compact pool the groups at or beyond the rank are not
        // loaded (they are zero or belong to the next adapter)
        const int rs = !VARW ? RM : roff ? (r + 7) & ~7 : pstride;
        const int k0 = c * kc + wv * kw;
        const int k_lo = min(k0, d_in), k_hi = min(k0 + kw, d_in);
        // this lane's x row (rows beyond the tile repeat its last row; their sums are dropped)
        const int mrow = seg.perm[p0 + min(li, rows - 1)];
        const uint16_t *xr = x + (size_t)mrow * d_in;
        const uint16_t *Aa = A + (size_t)row0 * d_in;

        f32x4_t acc[C::NB];
#pragma unroll
        for (int b = 0; b < C::NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        constexpr bool flat = LAYOUT == kFlat;
        if constexpr (!flat) {
            // per LDS fill: A_a[kb .. kb+KS, 0:rank] and x; groups at or beyond the rank, and
            // rows at or beyond the range's end, are zeros instead of loads (a padded pool's
            // padding is not read above r_max 16).  Unit u = lane + 64 i is (row u / GR, group u % GR); the
            // offsets are 32-bit bytes from the adapter's block (one VGPR per address).
            const char *ab = reinterpret_cast<const char *>(Aa);
            // fill f's loads: A_a rows kb .. kb + KS (zeros past k_hi) and this lane's x
            auto load_fill = [&](int kb, uint4(&av)[C::AL], uint4(&xv)[C::STEPS]) {
#pragma unroll
                for (int i = 0; i < C::AL; ++i) {
                    const int u = lane + 64 * i, kr = kb + u / C::GR, gr = u % C::GR;
                    const uint32_t off = ((uint32_t)min(kr, d_in - 1) * (uint32_t)rs + (uint32_t)(gr * 8)) * 2u;
                    // (a padded pool at r_max <= 16 loads its padding too: its loads then need
                    // not wait for the rank, and the saving would be at most half a row)
                    const bool want = (LAYOUT == kPadRM && RM <= 16) || gr * 8 < r;
                    av[i] = want && kr < k_hi ? *reinterpret_cast<const uint4 *>(ab + off)
                                              : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int st = 0; st < C::STEPS; ++st) xv[st] = ld16(xr + min(kb + 32 * st + 8 * g, d_in - 8));
            };
            // At r_max <= 16 every fill's loads are issued before the first fill is used (one
            // round trip per chunk instead of one per fill; at r_max 16, 30 more VGPRs and four
            // workgroups per CU instead of five): prefill shrink 9.9 -> 9.4 us, the MLP's
            // 11008-deep shrink 16.0 -> 15.7 us.  Above r_max 16 the registers would cost a
            // wave per SIMD.
            constexpr bool UPFRONT = RM <= 16;
            uint4 pav[UPFRONT ? C::FILLS : 1][C::AL], pxv[UPFRONT ? C::FILLS : 1][C::STEPS];
            if constexpr (UPFRONT) {
#pragma unroll
                for (int f = 0; f < C::FILLS; ++f) load_fill(k_lo + f * C::KS, pav[f], pxv[f]);
            }
#pragma unroll
            for (int f = 0; f < C::FILLS; ++f) {
                const int kb = k_lo + f * C::KS;
                if (kb >= k_hi) break;  // uniform: the wave's range ends inside this chunk
                uint4 av[C::AL], xv[C::STEPS];
                if constexpr (UPFRONT) {
#pragma unroll
                    for (int i = 0; i < C::AL; ++i) av[i] = pav[f][i];
#pragma unroll
                    for (int st = 0; st < C::STEPS; ++st) xv[st] = pxv[f][st];
                } else {
                    load_fill(kb, av, xv);
                }
#pragma unroll
                for (int i = 0; i < C::AL; ++i) {
                    const int u = lane + 64 * i, kr = u / C::GR, gr = u % C::GR;
                    *reinterpret_cast<uint4 *>(wg + kr * C::LROW + gr * 16) = av[i];
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
                shrink_mfma_fill<C, RM>(acc, xv, wl, kb, k_hi, g, li, r);
                __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS reads done before the next fill overwrites
            }
        } else {
            for (int kb = k_lo; kb < k_hi; kb += C::KS) {
                // (kFlat) rows of a width that is not a multiple of 8: the chunk's run of rs-wide
                // rows, element by element
                {
                    // zero the wave's rows (columns at or beyond rs, rows at or beyond k_hi stay
                    // zero), wait for those writes, then place element e of the run at k row
                    // e / rs, column e % rs (rows kb .. k_hi - 1 of A_a: all inside it)
                    for (int v = lane; v < C::KS * C::LROW / 16; v += 64)
                        *reinterpret_cast<uint4 *>(wg + v * 16) = make_uint4(0, 0, 0, 0);
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    const int n_el = min(C::KS, k_hi - kb) * rs;
                    const int step_k = 64 / rs, step_j = 64 - step_k * rs;
                    const uint16_t *src = Aa + (size_t)kb * rs;
#pragma unroll 1
                    for (int e0 = 0; e0 < n_el; e0 += 64 * 8) {
                        uint16_t h[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int e = e0 + lane + 64 * q;
                            h[q] = e < n_el ? src[e] : (uint16_t)0;
                        }
                        // element e0 + lane + 64 q sits at k row kr, column j: one division per
                        // batch, then steps of 64 elements
                        int kr = (e0 + lane) / rs, j = (e0 + lane) - kr * rs;
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            if (e0 + lane + 64 * q < n_el)
                                *reinterpret_cast<uint16_t *>(wg + kr * C::LROW + j * 2) = h[q];
                            j += step_j;
                            kr += step_k;
                            if (j >= rs) { j -= rs; ++kr; }
                        }
                    }
                }
                uint4 xv[C::STEPS];
#pragma unroll
                for (int st = 0; st < C::STEPS; ++st) xv[st] = ld16(xr + min(kb + 32 * st + 8 * g, d_in - 8));
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
                shrink_mfma_fill<C, RM>(acc, xv, wl, kb, k_hi, g, li, r);
                __builtin_amdgcn_s_waitcnt(0xC07F);  // LDS reads done before the next fill overwrites
            }
        }
        // acc[b][i] = sum for tile row 4 g + i, column 16 b + li (this wave's quarter)
        if (wv > 0) {
#pragma unroll
            for (int b = 0; b < C::NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wv - 1][(4 * g + i) * C::RMP + 16 * b + li] = acc[b][i];
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = 4 * g + i;
                const int m = __shfl(mrow, tr, 64);
                if (tr < rows) {
#pragma unroll
                    for (int b = 0; b < C::NB; ++b) {
                        const int col = 16 * b + li;
                        float v = acc[b][i];
#pragma unroll
                        for (int q = 0; q < kWavesPerBlock - 1; ++q) v += red[q][tr * C::RMP + col];
                        if (col < RM) partial[((size_t)c * M + m) * RM + col] = v;
                    }
                }
            }
        }
        __syncthreads();  // wave 0 has read red before the next chunk's sums go there
    }
}

// t[m, 0:t_stride) = sum over chunks (ascending) of partial[chunk][m][:] for LoRA rows; 0 for
// base-only rows.  One thread per 4 columns of one position of perm; eight chunk loads are
// in flight at a time and added in chunk order.  Rows of t are t_stride floats apart
// (t_stride <= RM; 16-byte stores when it is a multiple of 4).
__global__ __launch_bounds__(256) void shrink_finalize_kernel(const float *__restrict__ partial,
                                                              int M, int RM, int ksplit, Seg seg,
                                                              float *__restrict__ t, int t_stride) {
    const int per_row = RM / 4;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)M * per_row) return;
    const int p = (int)(idx / per_row), j = (int)(idx % per_row) * 4;
    if (j >= t_stride) return;
    const int m = seg.perm[p];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p < seg.meta[1]) {
        const float *src = partial + (size_t)m * RM + j;
        const size_t cs = (size_t)M * RM;
        for (int c0 = 0; c0 < ksplit; c0 += 8) {
            float4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = c0 + i < ksplit ? *reinterpret_cast<const float4 *>(src + (c0 + i) * cs)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                acc.x += v[i].x; acc.y += v[i].y; acc.z += v[i].z; acc.w += v[i].w;
            }
        }
    }
    float *dst = t + (size_t)m * t_stride + j;
    if ((t_stride & 3) == 0) {
        *reinterpret_cast<float4 *>(dst) = acc;
    } else {
        const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
        for (int q = 0; q < 4 && j + q < t_stride; ++q) dst[q] = a4[q];
    }
}

}  // namespace

void shrink_plan(int d_in, int r_max, int *kc, int *ksplit) {
    *kc = (r_max == 64 ? 128 : kKC) * kWavesPerBlock;  // a workgroup's k range (MfmaShrink::KW per wave)
    *ksplit = (d_in + *kc - 1) / *kc;
}

namespace {

hipError_t launch_shrink_pools(const uint16_t *x, const ShrinkPools &pools, const int32_t *ranks,
                               const int32_t *roff, int pool_rows, int pstride, int M, int d_in,
                               int r_max, int n_adapters, Seg seg, int kc, int ksplit,
                               hipStream_t s) {
    if (roff == nullptr && (pstride < 1 || pstride > r_max)) return hipErrorInvalidValue;
    if (kc % (8 * kWavesPerBlock) != 0) return hipErrorInvalidValue;
    if (pools.n < 1 || pools.n > kMaxProj) return hipErrorInvalidValue;
    // one workgroup per item
    const long items = (long)lora_max_tiles(M, n_adapters) * ksplit * pools.n;
    const dim3 wgrid((unsigned)(items < kMaxGrid ? items : kMaxGrid));
    const dim3 wblock(64 * kWavesPerBlock);
    const int layout = roff != nullptr       ? kVarW
                       : pstride == r_max    ? kPadRM
                       : (pstride & 7) != 0  ? kFlat
                                             : kVarW;
#define LORA_SHRINK_ONE(RMV, LAY)                                                                \
    launch(shrink_mfma_kernel<RMV, LAY>, wgrid, wblock, 0, s, x, pools, ranks, roff, pool_rows,  \
           pstride, M, d_in, n_adapters, seg, ksplit, kc)
#define LORA_SHRINK_LAUNCH(RMV)                                                                  \
    if (layout == kPadRM) LORA_SHRINK_ONE(RMV, kPadRM);                                          \
    else if (layout == kVarW) LORA_SHRINK_ONE(RMV, kVarW);                                       \
    else LORA_SHRINK_ONE(RMV, kFlat);
    switch (r_max) {
        case 8: LORA_SHRINK_LAUNCH(8) break;
        case 16: LORA_SHRINK_LAUNCH(16) break;
        case 32: LORA_SHRINK_LAUNCH(32) break;
        case 64: LORA_SHRINK_LAUNCH(64) break;
        default: return hipErrorInvalidValue;
    }
#undef LORA_SHRINK_LAUNCH
#undef LORA_SHRINK_ONE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shrink(const uint16_t *x, const uint16_t *A, const int32_t *ranks,
                         const int32_t *roff, int pool_rows, int pstride, int M, int d_in,
                         int r_max, int n_adapters, Seg seg, float *partial, int kc, int ksplit,
                         hipStream_t s) {
    ShrinkPools pools{};
    pools.A[0] = A;
    pools.partial[0] = partial;
    pools.n = 1;
    return launch_shrink_pools(x, pools, ranks, roff, pool_rows, pstride, M, d_in, r_max,
                               n_adapters, seg, kc, ksplit, s);
}

hipError_t launch_shrink_multi(const uint16_t *x, int n_proj, const uint16_t *const *A,
                               float *const *partial, const int32_t *ranks, int pstride, int M,
                               int d_in, int r_max, int n_adapters, Seg seg, int kc, int ksplit,
                               hipStream_t s) {
    if (n_proj < 1 || n_proj > kMaxProj) return hipErrorInvalidValue;
    ShrinkPools pools{};
    for (int p = 0; p < n_proj; ++p) {
        pools.A[p] = A[p];
        pools.partial[p] = partial[p];
    }
    pools.n = n_proj;
    return launch_shrink_pools(x, pools, ranks, nullptr, 0, pstride, M, d_in, r_max, n_adapters,
                               seg, kc, ksplit, s);
}

hipError_t launch_shrink_finalize(const float *partial, int M, int r_max, int ksplit, Seg seg,
                                  float *t, int t_stride, hipStream_t s) {
    if (t_stride < 1 || t_stride > r_max) return hipErrorInvalidValue;
    const long threads = (long)M * (r_max / 4);
    const int grid = (int)((threads + 255) / 256);
    launch(shrink_finalize_kernel, dim3(grid), dim3(256), 0, s, partial, M, r_max, ksplit, seg, t,
           t_stride);
    return hipGetLastError();
}

}  // namespace lora

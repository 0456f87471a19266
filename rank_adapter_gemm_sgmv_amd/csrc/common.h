// common.h -- device helpers and launch interfaces shared by the gfx950 kernels of
// liblora_mi355x.so.  Internal: the public interface is include/lora.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora.h"

namespace lora {

constexpr int kTileRows = LORA_TILE_ROWS;

// Segment buffers as seen by the kernels.
struct Seg {
    int32_t *perm;
    int32_t *offsets;
    int32_t *seg_adapter;
    int32_t *tiles;
    int32_t *meta;
};

inline Seg to_seg(const lora_segments_t &s) {
    return Seg{s.perm, s.offsets, s.seg_adapter, s.tiles, s.meta};
}

// ---- bfloat16 <-> float32 --------------------------------------------------------------
// bf16 is the high half of a float32 word: widening is a shift, exact.
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Round to nearest even; a NaN stays a (quiet) NaN.  Branch-free (a select).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t quiet_nan = (u >> 16) | 0x40u;
    return (f != f) ? quiet_nan : rounded;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// 8 bf16 (one 16-byte vector) -> 8 floats
__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
// A store that writes through the L2 to memory (sc0 sc1), for data only a later kernel reads:
// the end-of-kernel write-back then finds no dirty lines of it.  A vector store; p is global.
__device__ __forceinline__ void st_wt(float *p, float v) {
    asm volatile("global_store_dword %0, %1, off sc0 sc1" ::"v"(p), "v"(v) : "memory");
}

// ---- where an adapter's rank rows are ----------------------------------------------------
// A padded pool (roff == nullptr) holds adapter a at rank rows a * stride .. a * stride +
// stride - 1, stride being the caller's r_max (rows beyond the adapter's rank are zero):
// A_a = A[a] is [d_in][stride], B_a = B[a] is [stride][d_out].  A rank-compact pool holds an
// adapter of rank r in w = round_up(r, 8) rank rows roff[a] .. roff[a] + w - 1 of its
// pool_rows rank rows (rank rows r .. w - 1 zero): A_a is the [d_in][w] block at element
// roff[a] * d_in of A, B_a the [w][d_out] block at row roff[a] of B; so every k row of A_a
// starts 16-byte aligned.  r is the adapter's rank, already clamped to [0, width]; in a
// compact pool an adapter whose rows leave the pool gets r = 0 (it adds nothing; the checked
// mode of the ABI reports such a table), so no access leaves the pool.  Returns the first
// rank row (0 when r becomes 0).
__device__ __forceinline__ int adapter_row0(const int32_t *roff, int pool_rows, int a, int stride,
                                            int &r) {
    if (roff == nullptr) return a * stride;
    const int o = roff[a];
    if (o < 0 || o > pool_rows - ((r + 7) & ~7)) r = 0;
    return r > 0 ? o : 0;
}

// Kernel rank bucket of a pool whose widest adapter has r_max rank rows: t, the shrink's
// partial sums and every other internal buffer use the bucket as their row width.
// Projections one lora_linear_multi launch takes, and entry i of a per-projection pointer
// array held in kernel arguments, by selects (a runtime index into the argument array would
// copy it to scratch memory).
constexpr int kMaxProj = 4;
template <class T>
__device__ __forceinline__ T pick_proj(int i, T const (&v)[kMaxProj]) {
    static_assert(kMaxProj == 4, "selects below");
    return i == 0 ? v[0] : i == 1 ? v[1] : i == 2 ? v[2] : v[3];
}

constexpr int rank_bucket(int r_max) { return r_max <= 8 ? 8 : r_max <= 16 ? 16 : r_max <= 32 ? 32 : 64; }
// Width of an adapter's slot in the small-batch GEMM's adapter tiles for rank bucket rb (the
// bf16 base; t there has this row width).  Rank-8 pools take 16-wide slots: an 8-wide slot
// gave each load of an adapter tile 16 bytes of 16 adapters, half a cache line each, twice
// the lines per byte of the wider slots (64 x 4096 x 4096 with 28 rank-8 adapters: 20.5 us per
// step against 18.3 at rank 16); in a 16-wide slot the second group re-reads the first.
constexpr int fused_tile_rank(int rb) { return rb < 16 ? 16 : rb; }

// ---- kernel launches -------------------------------------------------------------------
// Every kernel of the library is launched through launch().  Normally it is a plain launch;
// while a KernelTimer is installed for the calling host thread (lora_linear_profiled), the
// launch carries a start and a stop event that the GPU stamps from the kernel's own dispatch
// packet, so the elapsed time is the kernel's duration with no extra packet in the stream.
struct KernelTimer {
    static constexpr int kMax = 24;
    hipEvent_t start[kMax] = {};
    hipEvent_t stop[kMax] = {};
    int n = 0;
};
extern thread_local KernelTimer *g_timer;

template <typename... Args, typename F>
inline void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
    KernelTimer *t = g_timer;
    if (t != nullptr && t->n < KernelTimer::kMax) {
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, t->start[t->n], t->stop[t->n], 0, args...);
        ++t->n;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
    }
}

// ---- launchers (one kernel each) -------------------------------------------------------

hipError_t launch_build_segments(const int32_t *ids, int M, int n_adapters, Seg seg,
                                 hipStream_t s);

// Split-K shrink: partial[ks][m][j] for rows of every tile; ks = 0..ksplit-1, chunks of
// kc columns of x.  Followed by launch_shrink_finalize to sum the partials into t.
// r_max: the kernel rank bucket (8, 16, 32 or 64; the partial sums' row width); pstride: the
// padded pool's rank-row stride per adapter (the caller's r_max, <= the bucket; not read for
// a compact pool).
hipError_t launch_shrink(const uint16_t *x, const uint16_t *A, const int32_t *ranks,
                         const int32_t *roff, int pool_rows, int pstride, int M, int d_in,
                         int r_max, int n_adapters, Seg seg, float *partial, int kc, int ksplit,
                         hipStream_t s);
// The same over n_proj <= kMaxProj pools that share x, the tables and the segments
// (lora_linear_multi) in one launch: pool p reads A[p] and writes partial[p].
hipError_t launch_shrink_multi(const uint16_t *x, int n_proj, const uint16_t *const *A,
                               float *const *partial, const int32_t *ranks, int pstride, int M,
                               int d_in, int r_max, int n_adapters, Seg seg, int kc, int ksplit,
                               hipStream_t s);
// t[m][0 : t_stride) from the partial sums (t_stride <= r_max, the bucket).
hipError_t launch_shrink_finalize(const float *partial, int M, int r_max, int ksplit, Seg seg,
                                  float *t, int t_stride, hipStream_t s);

// t rows are t_stride floats apart (t_stride >= the widest rank).
hipError_t launch_expand(const float *t, int t_stride, const uint16_t *B, const float *scale,
                         const int32_t *ranks, const int32_t *roff, int pool_rows, int pstride,
                         int M, int d_out, int r_max, int n_adapters, Seg seg, void *y, bool y_f32,
                         hipStream_t s);

// LoRA epilogue arguments of the prefill GEMM (rows are taken in segment order).
struct LoraEpilogue {
    const float *tpart;    // [n_chunks][M][r_max]: the shrink's k-chunk sums of t
    int n_chunks;
    const uint16_t *B;     // [n][r_max][d_out]
    const float *scale;    // [n]
    const int32_t *ids;    // [M]
    int r_max;
    int n_adapters;
    const int32_t *ranks;  // [n], read only for a rank-compact pool
    const int32_t *roff;   // [n] first rank row of each adapter (rank-compact pool), or nullptr
    int pool_rows;
    int pstride;           // padded pool: rank rows per adapter (<= r_max, the bucket)
};

// y = x W (+ LoRA epilogue when lora != nullptr).  `prefill` selects the 256x256 tiling
// and segment-ordered rows; otherwise a decode tiling, which may split K: then the partial
// sums go to ws_partial and *ksplit_out != 1: > 1 split-K slices (launch_splitk_reduce must
// follow), or -1 stream-K partial tiles (launch_sk_reduce_lora must follow).
hipError_t launch_gemm(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y,
                       bool y_f32, bool prefill, Seg seg, const LoraEpilogue *lora,
                       float *ws_partial, size_t ws_partial_floats, int *ksplit_out,
                       hipStream_t s);
// Large-batch MFMA GEMM (csrc/gemm_big.hip): with lora != nullptr, rows in segment order and
// the LoRA delta of each adapter run added before the only store (prefill); otherwise plain
// y = x W in natural row order.
hipError_t launch_gemm_big(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y,
                           bool y_f32, Seg seg, const LoraEpilogue *lora, hipStream_t s);

// Stream-K decode GEMM (csrc/gemm_big.hip) for batches of 257-1024 rows whose 256 x 256
// tiles are too few to fill the chip: L lanes of equal K length, n_tm workgroups per lane.
// Several projections of one layer that read the same x (lora_linear_multi) share one
// launch: their column panels are laid end to end, projection after projection (n_proj
// projections of n_tn1 panels each, n_tn = n_proj * n_tn1).
struct SkPlan {
    bool use;
    int n_tm, n_tn, L;
    int n_proj, n_tn1;
};
SkPlan sk_plan(int M, int K, int N, int n_proj = 1);
size_t sk_partial_floats(const SkPlan &p);
// Per-projection operands of the stream-K launches (entries past p.n_proj unused).
struct SkProj {
    const uint16_t *W[kMaxProj];   // [K][N]
    const uint16_t *B[kMaxProj];   // adapter pool B of each projection
    const float *tpart[kMaxProj];  // its shrink's chunk sums [n_chunks][M][r_max]
    void *y[kMaxProj];             // [M][N]
};
hipError_t launch_gemm_sk(const uint16_t *x, const SkProj &pj, int M, int K, int N,
                          const SkPlan &p, float *partial, hipStream_t s);
// y = (the stream-K partial tiles added in lane order) + scale_a t B_a on rows with an
// adapter, rows in segment order; t summed from the shrink's n_chunks chunk sums; rounds
// once into y (each projection's own B, t and y).
hipError_t launch_sk_reduce_lora(const float *partial, int M, int K, int N, const SkPlan &p,
                                 Seg seg, const SkProj &pj, int n_chunks, const float *scale,
                                 const int32_t *ids, const int32_t *ranks, const int32_t *roff,
                                 int pool_rows, int pstride, int r_max, int n_adapters,
                                 bool y_f32, hipStream_t s);

// Adds the split-K decode GEMM's ksplit > 1 partial slices into y, in order.
hipError_t launch_splitk_reduce(const float *partial, int M, int N, int ksplit, void *y,
                                bool y_f32, hipStream_t s);

// LoRA operands of the small-batch decode GEMM and reduction (csrc/decode_gemm.hip).
struct DecodeLora {
    const float *tpart;    // [n_chunks][M][r_max]: the segment-path shrink's chunk sums of t
                           // (calls without adapter tiles)
    int n_chunks;
    const uint16_t *B;     // [n][r_max][d_out]
    const float *scale;    // [n]
    const int32_t *ids;    // [M]
    const int32_t *ranks;  // [n] true ranks, or nullptr (= pstride)
    int r_max;             // the kernel rank bucket (with adapter tiles: the slot width,
                           // fused_tile_rank of the bucket for the bf16 base)
    int n_adapters;
    const int32_t *roff;   // [n] first rank row of each adapter (rank-compact pool), or nullptr
    int pool_rows;
    int pstride;           // padded pool: rank rows per adapter (<= r_max)
};

// The segment build the medium-batch decode GEMM launch runs in one extra workgroup beside
// the GEMM (the GEMM itself does not read segments; the shrink launched after it does).
struct SegBuild {
    const int32_t *ids;  // [M]
    int n_adapters;
    Seg seg;
};

// Decode batches up to this many rows take the fused path (x W and x A_i as tiles of one
// split-K launch) when d_in % 32 == 0: beyond it the adapter tiles (up to one slot per row)
// cost more than the segment-path shrink.
constexpr int kDecodeMaxRows = 128;
// The split-K decode GEMM + LoRA reduction serve batches up to this many rows (beyond
// kDecodeMaxRows with the segment-path shrink writing the chunk sums).
constexpr int kDecodeGemmMaxRows = 256;
bool decode_gemm_supported(int M, int K, int N);  // M <= kDecodeGemmMaxRows
bool decode_fused_supported(int M, int K, int N);  // and M <= kDecodeMaxRows
// Split partial floats of the decode GEMM at these sizes: the most any of its plans (with or
// without adapter tiles) writes.
size_t decode_gemm_partial_floats(int M, int K, int N, int r_max, int n_adapters);
// Split-K partial tiles of x W for a decode batch; with `adapters` (M <= kDecodeMaxRows)
// the same launch also streams the batch's adapters' A as extra tiles (the LoRA shrink).
// Tiles of bm (32 or 64) rows x 128 columns, the n_tn column tiles of W then the adapter
// tiles; K cut into ks splits (the last may be shorter); partial tiles laid out
// [split][tm + tn * n_tm][bm][128] (fp32), what launch_decode_reduce adds.  build
// (nullable): also build the segments of these ids, in one more workgroup.
hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, const uint16_t *A, int M,
                              int K, int N, const DecodeLora &lo, bool adapters, float *partial,
                              const SegBuild *build, hipStream_t s);

// x W_eff for a decode batch whose base weight is fp8 E4M3 codes W8[N][K] with per-column
// scales w_scale[N] (csrc/decode_gemm.hip): the scaled partial tiles of the decode plan without
// adapter tiles, laid out [split][tm + tn * n_tm][bm][128] (fp32) as launch_decode_gemm's.
// As decode_gemm_supported, and N % 8 == 0.  build (nullable): also build the segments of
// these ids in one more workgroup.
hipError_t launch_decode_gemm_fp8(const uint16_t *x, const uint8_t *W8, const float *w_scale,
                                  int M, int K, int N, float *partial, const SegBuild *build,
                                  hipStream_t s);

// The same fp8 GEMM with the shrink x A_a as adapter tiles of the same launch (a batch of at
// most kDecodeMaxRows rows, a pool padded at a rank bucket: lo.r_max 8, 16, 32 or 64): the
// partial tiles of dec_plan with adapter tiles, what launch_decode_reduce (adapters = true)
// adds.
hipError_t launch_decode_gemm_fp8_lora(const uint16_t *x, const uint8_t *W8, const float *w_scale,
                                       const uint16_t *A, int M, int K, int N,
                                       const DecodeLora &lo, float *partial, hipStream_t s);

// y = (split partials added in order) + scale_a * t B_a, t from the adapter tiles' splits
// (`adapters`) or from the segment-path shrink's chunk sums; rounds once into y.  With the
// chunk sums and `seg` (the segments of these ids, nullable) the rows of one adapter share
// each load of B_a; the result is the same.
hipError_t launch_decode_reduce(const float *partial, int M, int K, int N, void *y, bool y_f32,
                                const DecodeLora &lo, bool adapters, const Seg *seg,
                                hipStream_t s);

// Workspace floats the decode GEMM needs for split-K partials at these sizes.
size_t gemm_partial_floats(int M, int K, int N);

// Split-K plan of the shrink for d_in.
void shrink_plan(int d_in, int r_max, int *kc, int *ksplit);

// ---- MoE-LoRA (csrc/moe.hip) ---------------------------------------------------------------
// Plan: tiles of 128 columns (n_tn of W[e], n_lt adapter tiles of 128 / rm adapters), K cut
// into ks splits of k_per_split; pairs in blocks of bm rows; partial rows np floats apart.
struct MoePlan {
    int rm, bm, n_tn, n_lt, ks, k_per_split, np;
};
MoePlan moe_plan(int M, int top_k, int E, int K, int N, int r_max, int n_adapters);
size_t moe_partial_floats(const MoePlan &p, int P);  // [ks][P][np]
size_t moe_tpart_floats(const MoePlan &p, int P);    // [ks][P][rm]

struct MoeGemmArgs {
    const uint16_t *x;         // [M][K]
    const uint16_t *W;         // [E][K][N]
    const uint16_t *A;         // [n_adapters][E][K][r_stride]
    const int32_t *topk_ids;   // [P] = [M][top_k]
    const int32_t *ids;        // [M]
    int P, top_k, E, K, N, r_stride, n_adapters;
    int n_tn, n_lt, k_per_split, np;  // set from the plan by launch_moe_gemm
    float *partial;            // [ks][P][np]
    float *tpart;              // [ks][P][rm]
};
struct MoeReduceArgs {
    const float *partial, *tpart;
    const uint16_t *B;         // [n_adapters][E][r_stride][N]
    const float *scale;        // [n_adapters]
    const int32_t *ranks;      // [n_adapters] or nullptr (= r_stride)
    const int32_t *topk_ids;   // [P]
    const int32_t *ids;        // [M]
    const float *topk_w;       // [P] or nullptr (= 1)
    int P, top_k, E, N, r_stride, n_adapters;
    int ks, np;                // set from the plan by launch_moe_reduce
    void *y;                   // [P][N]
};
hipError_t launch_moe_gemm(const MoePlan &p, const MoeGemmArgs &a, hipStream_t s);
hipError_t launch_moe_reduce(const MoePlan &p, const MoeReduceArgs &a, bool y_f32, hipStream_t s);

// Records e as the error lora_last_hip_error() reports; LORA_ERR_HIP unless e is hipSuccess.
lora_status_t hip_error_status(hipError_t e);

// lora_linear on the workspace ws (validation, checked mode, launches).
lora_status_t linear_on_workspace(const void *x, const void *W, const void *A, const void *B,
                                  const float *scale, const int32_t *ranks, const int32_t *ids,
                                  int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, const lora_segments_t *segs, void *y,
                                  lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                  size_t ws_bytes, void *stream);

}  // namespace lora

// api.cpp -- the C ABI of liblora_mi355x.so (include/lora.h): host-side validation,
// workspace layout and the launch sequence of each call.  No call allocates device memory or
// keeps state; only the checked mode and the measurement aids synchronise.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "common.h"

using namespace lora;

thread_local KernelTimer *lora::g_timer = nullptr;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxDim = 1 << 20;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool rank_ok(int32_t r_max) { return r_max >= 1 && r_max <= 64; }

bool dim_ok(int32_t d) { return d > 0 && d <= kMaxDim && d % 8 == 0; }

lora_status_t check_common(int32_t M, int32_t r_max, int32_t n_adapters) {
    if (M < 0 || M > LORA_MAX_ROWS) return LORA_ERR_SHAPE;
    if (n_adapters < 1 || n_adapters > LORA_MAX_ADAPTERS) return LORA_ERR_SHAPE;
    if (!rank_ok(r_max)) return LORA_ERR_RANK;
    return LORA_OK;
}

lora_status_t check_seg(const lora_segments_t &s) {
    if (!s.perm || !s.offsets || !s.seg_adapter || !s.tiles || !s.meta) return LORA_ERR_NULL;
    if (!aligned(s.perm, 4) || !aligned(s.offsets, 4) || !aligned(s.seg_adapter, 4) ||
        !aligned(s.tiles, 8) || !aligned(s.meta, 4))
        return LORA_ERR_ALIGN;
    return LORA_OK;
}

size_t segments_bytes(int32_t M, int32_t n) {
    const int32_t segs = M < n ? M : n;
    return round_up((size_t)M * 4) + round_up((size_t)(n + 1) * 4) +
           round_up((size_t)(segs > 1 ? segs : 1) * 4) +
           round_up((size_t)2 * lora_max_tiles(M, n) * 4) + round_up(4 * 4);
}

lora_segments_t carve_segments(char *&p, int32_t M, int32_t n) {
    lora_segments_t s;
    const int32_t segs = M < n ? M : n;
    s.perm = reinterpret_cast<int32_t *>(p); p += round_up((size_t)M * 4);
    s.offsets = reinterpret_cast<int32_t *>(p); p += round_up((size_t)(n + 1) * 4);
    s.seg_adapter = reinterpret_cast<int32_t *>(p); p += round_up((size_t)(segs > 1 ? segs : 1) * 4);
    s.tiles = reinterpret_cast<int32_t *>(p); p += round_up((size_t)2 * lora_max_tiles(M, n) * 4);
    s.meta = reinterpret_cast<int32_t *>(p); p += round_up(4 * 4);
    return s;
}

// Internal buffers (t, partial sums) are laid out at the kernel rank bucket of r_max.
size_t shrink_partial_bytes(int32_t M, int32_t d_in, int32_t r_max) {
    const int rb = rank_bucket(r_max);
    int kc, ksplit;
    shrink_plan(d_in, rb, &kc, &ksplit);
    return round_up((size_t)ksplit * M * rb * sizeof(float));
}

size_t t_bytes(int32_t M, int32_t r_max) {
    return round_up((size_t)M * rank_bucket(r_max) * sizeof(float));
}

size_t gemm_bytes(int32_t M, int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters) {
    const size_t a = gemm_partial_floats(M, d_in, d_out),
                 b = decode_gemm_partial_floats(M, d_in, d_out, rank_bucket(r_max), n_adapters);
    return round_up((a > b ? a : b) * sizeof(float));
}


thread_local hipError_t g_last_hip_error = hipSuccess;

lora_status_t hip_status(hipError_t e) {
    g_last_hip_error = e;
    return e == hipSuccess ? LORA_OK : LORA_ERR_HIP;
}

// Launch errors are read with hipGetLastError after each launch; clear anything pending
// from before this call so it is not reported as ours.
void clear_stale_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

int32_t lora_max_tiles(int32_t M, int32_t n_adapters) {
    if (M <= 0 || n_adapters <= 0) return 0;
    const int32_t segs = M < n_adapters ? M : n_adapters;
    return segs + M / LORA_TILE_ROWS;
}

size_t lora_workspace_bytes(int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                            int32_t n_adapters) {
    if (check_common(M, r_max, n_adapters) != LORA_OK || !dim_ok(d_in) || !dim_ok(d_out)) return 0;
    if (M == 0) return 0;
    return segments_bytes(M, n_adapters) + t_bytes(M, r_max) + shrink_partial_bytes(M, d_in, r_max) +
           gemm_bytes(M, d_in, d_out, r_max, n_adapters);
}

lora_status_t lora_build_segments(const int32_t *ids, int32_t M, int32_t n_adapters,
                                  lora_segments_t seg, void *stream) {
    if (M < 0 || M > LORA_MAX_ROWS || n_adapters < 1 || n_adapters > LORA_MAX_ADAPTERS)
        return LORA_ERR_SHAPE;
    if (M == 0) return LORA_OK;
    if (!ids) return LORA_ERR_NULL;
    lora_status_t st = check_seg(seg);
    if (st != LORA_OK) return st;
    if (!aligned(ids, 4)) return LORA_ERR_ALIGN;
    clear_stale_error();
    return hip_status(launch_build_segments(ids, M, n_adapters, to_seg(seg), (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Extra arguments of a rank-compact pool: the table of first rank rows and the pool's
// rank-row count (at least one row, at most what the padded pool would hold).
lora_status_t check_compact(const int32_t *ranks, const int32_t *rank_offsets, int32_t pool_rows,
                            int32_t r_max, int32_t n_adapters) {
    if (!ranks || !rank_offsets) return LORA_ERR_NULL;
    if (!aligned(rank_offsets, 4)) return LORA_ERR_ALIGN;
    if (pool_rows < 1 || (int64_t)pool_rows > (int64_t)n_adapters * ((r_max + 7) & ~7))
        return LORA_ERR_SHAPE;
    return LORA_OK;
}

// lora_shrink / lora_shrink_compact (roff != nullptr): validated here, then the segment-path
// shrink and the ordered sum of its chunks into t[M][r_max].
lora_status_t shrink_call(const void *x, const void *A, const int32_t *ranks, const int32_t *roff,
                          int32_t pool_rows, int32_t M, int32_t d_in, int32_t r_max,
                          int32_t n_adapters, lora_segments_t seg, float *t, void *ws,
                          size_t ws_bytes, void *stream) {
    lora_status_t st = check_common(M, r_max, n_adapters);
    if (st != LORA_OK) return st;
    if (!dim_ok(d_in)) return LORA_ERR_SHAPE;
    if (M == 0) return LORA_OK;
    if (!x || !A || !t || !ws) return LORA_ERR_NULL;
    if ((st = check_seg(seg)) != LORA_OK) return st;
    if (!aligned(x, 16) || !aligned(A, 16) || !aligned(t, 16) || !aligned(ws, kAlign) ||
        (ranks && !aligned(ranks, 4)))
        return LORA_ERR_ALIGN;
    if (ws_bytes < shrink_partial_bytes(M, d_in, r_max)) return LORA_ERR_WORKSPACE;
    const int rb = rank_bucket(r_max);
    int kc, ksplit;
    shrink_plan(d_in, rb, &kc, &ksplit);
    clear_stale_error();
    hipStream_t s = (hipStream_t)stream;
    float *partial = static_cast<float *>(ws);
    const Seg sg = to_seg(seg);
    hipError_t e = launch_shrink(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(A),
                                 ranks, roff, pool_rows, r_max, M, d_in, rb, n_adapters, sg, partial,
                                 kc, ksplit, s);
    if (e == hipSuccess) e = launch_shrink_finalize(partial, M, rb, ksplit, sg, t, r_max, s);
    return hip_status(e);
}

lora_status_t expand_call(const float *t, const void *B, const float *scale, const int32_t *ranks,
                          const int32_t *roff, int32_t pool_rows, int32_t M, int32_t d_out,
                          int32_t r_max, int32_t n_adapters, lora_segments_t seg, void *y,
                          lora_dtype_t y_dtype, void *stream) {
    lora_status_t st = check_common(M, r_max, n_adapters);
    if (st != LORA_OK) return st;
    if (!dim_ok(d_out)) return LORA_ERR_SHAPE;
    if (y_dtype != LORA_BF16 && y_dtype != LORA_F32) return LORA_ERR_DTYPE;
    if (M == 0) return LORA_OK;
    if (!t || !B || !scale || !y) return LORA_ERR_NULL;
    if ((st = check_seg(seg)) != LORA_OK) return st;
    if (!aligned(t, 4) || !aligned(B, 16) || !aligned(y, 16) || !aligned(scale, 4) ||
        (ranks && !aligned(ranks, 4)))
        return LORA_ERR_ALIGN;
    clear_stale_error();
    return hip_status(launch_expand(t, r_max, static_cast<const uint16_t *>(B), scale, ranks, roff,
                                    pool_rows, r_max, M, d_out, rank_bucket(r_max), n_adapters,
                                    to_seg(seg), y, y_dtype == LORA_F32, (hipStream_t)stream));
}

}  // namespace

extern "C" {

lora_status_t lora_shrink(const void *x, const void *A, const int32_t *ranks, int32_t M,
                          int32_t d_in, int32_t r_max, int32_t n_adapters, lora_segments_t seg,
                          float *t, void *ws, size_t ws_bytes, void *stream) {
    return shrink_call(x, A, ranks, nullptr, 0, M, d_in, r_max, n_adapters, seg, t, ws, ws_bytes,
                       stream);
}

lora_status_t lora_shrink_compact(const void *x, const void *A, const int32_t *ranks,
                                  const int32_t *rank_offsets, int32_t pool_rows, int32_t M,
                                  int32_t d_in, int32_t r_max, int32_t n_adapters,
                                  lora_segments_t seg, float *t, void *ws, size_t ws_bytes,
                                  void *stream) {
    lora_status_t st = check_common(M, r_max, n_adapters);
    if (st == LORA_OK) st = check_compact(ranks, rank_offsets, pool_rows, r_max, n_adapters);
    if (st != LORA_OK) return st;
    return shrink_call(x, A, ranks, rank_offsets, pool_rows, M, d_in, r_max, n_adapters, seg, t, ws,
                       ws_bytes, stream);
}

lora_status_t lora_expand(const float *t, const void *B, const float *scale, const int32_t *ranks,
                          int32_t M, int32_t d_out, int32_t r_max, int32_t n_adapters,
                          lora_segments_t seg, void *y, lora_dtype_t y_dtype, void *stream) {
    return expand_call(t, B, scale, ranks, nullptr, 0, M, d_out, r_max, n_adapters, seg, y, y_dtype,
                       stream);
}

lora_status_t lora_expand_compact(const float *t, const void *B, const float *scale,
                                  const int32_t *ranks, const int32_t *rank_offsets,
                                  int32_t pool_rows, int32_t M, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, lora_segments_t seg, void *y,
                                  lora_dtype_t y_dtype, void *stream) {
    lora_status_t st = check_common(M, r_max, n_adapters);
    if (st == LORA_OK) st = check_compact(ranks, rank_offsets, pool_rows, r_max, n_adapters);
    if (st != LORA_OK) return st;
    return expand_call(t, B, scale, ranks, rank_offsets, pool_rows, M, d_out, r_max, n_adapters, seg,
                       y, y_dtype, stream);
}

}  // extern "C"

namespace {

// Names of the kernels a call launches, in launch order (lora_linear_profiled); their
// durations come from the KernelTimer events of each launch.  A null Marker records nothing.
struct Marker {
    static constexpr int kMax = KernelTimer::kMax;
    const char *names[kMax] = {};
    int n = 0;
    void mark(const char *name) {
        if (n < kMax) names[n++] = name;
    }
};

void mark(Marker *mk, const char *name) {
    if (mk) mk->mark(name);
}

lora_status_t check_linear(const void *x, const void *W, const void *A, const void *B,
                           const float *scale, const int32_t *ranks, const int32_t *ids, int32_t M,
                           int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
                           const lora_segments_t *segs, void *y, lora_dtype_t y_dtype,
                           lora_mode_t mode, void *ws, size_t ws_bytes) {
    lora_status_t st = check_common(M, r_max, n_adapters);
    if (st != LORA_OK) return st;
    if (!dim_ok(d_in) || !dim_ok(d_out)) return LORA_ERR_SHAPE;
    if (y_dtype != LORA_BF16 && y_dtype != LORA_F32) return LORA_ERR_DTYPE;
    const int bm = mode & ~LORA_MODE_CHECKED;
    if (bm != LORA_MODE_AUTO && bm != LORA_MODE_DECODE && bm != LORA_MODE_PREFILL)
        return LORA_ERR_MODE;
    if (M == 0) return LORA_OK;
    if (!x || !W || !A || !B || !scale || !ids || !y || !ws) return LORA_ERR_NULL;
    if (segs && (st = check_seg(*segs)) != LORA_OK) return st;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(A, 16) || !aligned(B, 16) ||
        !aligned(y, 16) || !aligned(ws, kAlign) || !aligned(scale, 4) || !aligned(ids, 4) ||
        (ranks && !aligned(ranks, 4)))
        return LORA_ERR_ALIGN;
    if (ws_bytes < lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters)) return LORA_ERR_WORKSPACE;
    return LORA_OK;
}

// LORA_MODE_CHECKED: wait for the stream (the tables may be written by work queued on it),
// copy ids, ranks and rank_offsets to host memory and check them: every id in [-1, n),
// every rank in [1, r_max], and in a compact pool every adapter's round_up(rank, 8) rows
// inside the pool.
// Returns LORA_ERR_BAD_ID, LORA_ERR_RANK or LORA_ERR_POOL for the first violation found.
lora_status_t check_tables(const int32_t *ids, int32_t M, const int32_t *ranks,
                           const int32_t *roff, int32_t pool_rows, int32_t r_max,
                           int32_t n_adapters, hipStream_t s) {
    hipError_t e = hipStreamSynchronize(s);
    std::vector<int32_t> h_ids(M), h_ranks(ranks ? n_adapters : 0), h_off(roff ? n_adapters : 0);
    if (e == hipSuccess) e = hipMemcpy(h_ids.data(), ids, (size_t)M * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess && ranks)
        e = hipMemcpy(h_ranks.data(), ranks, (size_t)n_adapters * 4, hipMemcpyDeviceToHost);
    if (e == hipSuccess && roff)
        e = hipMemcpy(h_off.data(), roff, (size_t)n_adapters * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    for (int32_t m = 0; m < M; ++m)
        if (h_ids[m] < -1 || h_ids[m] >= n_adapters) return LORA_ERR_BAD_ID;
    for (int32_t a = 0; a < (int32_t)h_ranks.size(); ++a)
        if (h_ranks[a] < 1 || h_ranks[a] > r_max) return LORA_ERR_RANK;
    for (int32_t a = 0; a < (int32_t)h_off.size(); ++a)
        if (h_off[a] < 0 || (int64_t)h_off[a] + ((h_ranks[a] + 7) & ~7) > pool_rows)
            return LORA_ERR_POOL;
    return LORA_OK;
}

// The launch sequence of lora_linear (arguments already validated, M > 0).
//   decode, M <= 128 and d_in % 32 == 0: one split-K GEMM over W and the batch's adapters'
//            A laid side by side (the shrink as extra column tiles), then the ordered
//            reduction that adds scale_a t B_a (no segment-building launch: adapters are
//            numbered by id or grouped in LDS; segs is not needed)
//   decode, 128 < M <= 256 and d_in % 32 == 0: the split-K GEMM with build_segments in one
//            extra workgroup, shrink (chunk sums), the ordered reduction with the expand
//   decode, 256 < M <= 1024, d_in % 128 == 0 and few 256 x 256 tiles: build_segments,
//            shrink (chunk sums), the stream-K GEMM, one pass adding its partial tiles, t
//            and the expand
//   decode otherwise: build_segments, shrink, shrink_finalize, gemm [, splitk_reduce], expand
//   prefill: build_segments, shrink, gemm with the LoRA epilogue (which adds t from the
//            shrink's chunk sums)
// A rank-compact pool (roff != nullptr, lora_linear_compact) takes the same sequences; a padded
// pool whose r_max is not a rank bucket (8, 16, 32, 64) too, except that its decode batches of
// at most 128 rows take the second one (the first lays adapters side by side at row stride
// r_max = the bucket).
hipError_t run_linear(const void *x, const void *W, const void *A, const void *B,
                      const float *scale, const int32_t *ranks, const int32_t *roff,
                      int32_t pool_rows, const int32_t *ids, int32_t M, int32_t d_in,
                      int32_t d_out, int32_t r_max, int32_t n_adapters,
                      const lora_segments_t *segs, void *y, lora_dtype_t y_dtype, lora_mode_t mode,
                      void *ws, hipStream_t s, Marker *mk) {
    const bool prefill = mode == LORA_MODE_PREFILL || (mode == LORA_MODE_AUTO && M >= LORA_PREFILL_MIN_ROWS);
    char *p = static_cast<char *>(ws);
    lora_segments_t own = carve_segments(p, M, n_adapters);
    float *t = reinterpret_cast<float *>(p); p += t_bytes(M, r_max);
    float *spart = reinterpret_cast<float *>(p); p += shrink_partial_bytes(M, d_in, r_max);
    float *gpart = reinterpret_cast<float *>(p);
    const size_t gpart_floats = gemm_partial_floats(M, d_in, d_out);

    const Seg sg = to_seg(segs ? *segs : own);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const uint16_t *Wb = static_cast<const uint16_t *>(W);
    const uint16_t *Bb = static_cast<const uint16_t *>(B);
    const bool yf = y_dtype == LORA_F32;
    hipError_t e;
    // kernels work at the rank bucket rb (t and partial sums rb wide); a padded pool's rank
    // rows per adapter are the caller's r_max (pstride)
    const int rb = rank_bucket(r_max), pstride = r_max;
    int kc, ksplit;
    shrink_plan(d_in, rb, &kc, &ksplit);
    // (the fused path lays adapters side by side in slots fused_tile_rank(rb) columns wide,
    // each adapter's rows read at its own width: a padded pool's stride when that is a
    // multiple of 8 (16-byte loads), or a rank-compact adapter's round8(rank))
    if (!prefill && (roff != nullptr || r_max % 8 == 0) && decode_fused_supported(M, d_in, d_out)) {
        // small decode batch: x W and the shrink x A_i as tiles of one split-K GEMM, then one
        // reduction adds the splits and the expand
        const DecodeLora lo{nullptr, 0, Bb, scale, ids, ranks,
                            fused_tile_rank(rb), n_adapters, roff, pool_rows, pstride};
        if ((e = launch_decode_gemm(xb, Wb, static_cast<const uint16_t *>(A), M, d_in, d_out, lo,
                                    true, gpart, nullptr, s)) != hipSuccess)
            return e;
        mark(mk, "decode_gemm_lora");
        if ((e = launch_decode_reduce(gpart, M, d_in, d_out, y, yf, lo, true, nullptr, s)) != hipSuccess) return e;
        mark(mk, "decode_reduce_lora");
        return hipSuccess;
    }
    if (!prefill && decode_gemm_supported(M, d_in, d_out)) {
        // medium decode batch: the split-K GEMM, with the segment build in one extra
        // workgroup of the same launch (unless the caller passed segments); then the
        // segment-path shrink, whose per-chunk partial sums have the layout the decode
        // reduction reads; the reduction with the expand
        const DecodeLora lo{spart, ksplit, Bb, scale, ids, ranks, rb, n_adapters, roff,
                            pool_rows, pstride};
        const SegBuild bld{ids, n_adapters, sg};
        if ((e = launch_decode_gemm(xb, Wb, nullptr, M, d_in, d_out, lo, false, gpart,
                                    segs ? nullptr : &bld, s)) != hipSuccess)
            return e;
        mark(mk, "decode_gemm");
        if ((e = launch_shrink(xb, static_cast<const uint16_t *>(A), ranks, roff, pool_rows, pstride, M,
                               d_in, rb, n_adapters, sg, spart, kc, ksplit, s)) != hipSuccess)
            return e;
        mark(mk, "shrink");
        if ((e = launch_decode_reduce(gpart, M, d_in, d_out, y, yf, lo, false, &sg, s)) != hipSuccess) return e;
        mark(mk, "decode_reduce_lora");
        return hipSuccess;
    }
    if (!segs) {
        if ((e = launch_build_segments(ids, M, n_adapters, sg, s)) != hipSuccess) return e;
        mark(mk, "build_segments");
    }
    if ((e = launch_shrink(xb, static_cast<const uint16_t *>(A), ranks, roff, pool_rows, pstride, M, d_in,
                           rb, n_adapters, sg, spart, kc, ksplit, s)) != hipSuccess)
        return e;
    mark(mk, "shrink");
    // the stream-K reduction and the prefill GEMM's epilogue add the shrink's chunk sums
    // themselves; the expand reads t
    const bool stream_k = !prefill && sk_plan(M, d_in, d_out).use;
    if (!stream_k && !prefill) {
        if ((e = launch_shrink_finalize(spart, M, rb, ksplit, sg, t, rb, s)) != hipSuccess)
            return e;
        mark(mk, "shrink_finalize");
    }
    int gsplit = 1;
    if (prefill) {
        LoraEpilogue ep{spart, ksplit, Bb, scale, ids, rb, n_adapters, ranks, roff, pool_rows, pstride};
        if ((e = launch_gemm(xb, Wb, M, d_in, d_out, y, yf, true, sg, &ep, nullptr, 0, &gsplit, s)) != hipSuccess)
            return e;
        mark(mk, "gemm_prefill_lora");
        return hipSuccess;
    }
    if ((e = launch_gemm(xb, Wb, M, d_in, d_out, y, yf, false, sg, nullptr, gpart, gpart_floats,
                         &gsplit, s)) != hipSuccess)
        return e;
    mark(mk, "gemm_decode");
    if (gsplit < 0) {
        // stream-K partial tiles: one pass adds them, t from the chunk sums, and the expand,
        // rows in segment order
        SkProj pj{};
        pj.B[0] = Bb;
        pj.tpart[0] = spart;
        pj.y[0] = y;
        if ((e = launch_sk_reduce_lora(gpart, M, d_in, d_out, sk_plan(M, d_in, d_out), sg, pj,
                                       ksplit, scale, ids, ranks, roff, pool_rows, pstride, rb,
                                       n_adapters, yf, s)) != hipSuccess)
            return e;
        mark(mk, "decode_reduce_lora");
        return hipSuccess;
    }
    if (gsplit > 1) {
        if ((e = launch_splitk_reduce(gpart, M, d_out, gsplit, y, yf, s)) != hipSuccess) return e;
        mark(mk, "splitk_reduce");
    }
    if ((e = launch_expand(t, rb, Bb, scale, ranks, roff, pool_rows, pstride, M, d_out, rb, n_adapters,
                           sg, y, yf, s)) != hipSuccess)
        return e;
    mark(mk, "expand");
    return hipSuccess;
}

}  // namespace

lora_status_t lora::hip_error_status(hipError_t e) { return hip_status(e); }

namespace {

// lora_linear_fp8w: the quantized-base decode sequence (arguments already validated, M > 0).
// Batches of at most 128 rows with r_max a rank bucket: the fp8 GEMM with the shrink as
// adapter tiles of the same launch, then the decode reduction (two launches, no segments).
// Otherwise: the fp8 decode GEMM (with the segment build in one extra workgroup unless
// segments are given), the segment-path shrink (chunk sums), and the decode reduction that
// adds the GEMM's scaled split partials and the expand.
hipError_t run_fp8w(const void *x, const void *W8, const float *w_scale, const void *A,
                    const void *B, const float *scale, const int32_t *ranks, const int32_t *ids,
                    int32_t M, int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
                    const lora_segments_t *segs, void *y, lora_dtype_t y_dtype, void *ws,
                    hipStream_t s, Marker *mk) {
    char *p = static_cast<char *>(ws);
    lora_segments_t own = carve_segments(p, M, n_adapters);
    float *t = reinterpret_cast<float *>(p); p += t_bytes(M, r_max);
    float *spart = reinterpret_cast<float *>(p); p += shrink_partial_bytes(M, d_in, r_max);
    float *gpart = reinterpret_cast<float *>(p);
    const Seg sg = to_seg(segs ? *segs : own);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const int rb = rank_bucket(r_max);
    hipError_t e;
    if (r_max == rb && decode_fused_supported(M, d_in, d_out)) {
        // small batch, pool padded at a rank bucket: the shrink as adapter tiles of the fp8
        // GEMM's launch, then the reduction
        const DecodeLora lo{nullptr, 0, static_cast<const uint16_t *>(B),
                            scale, ids, ranks, rb, n_adapters, nullptr, 0, r_max};
        if ((e = launch_decode_gemm_fp8_lora(xb, static_cast<const uint8_t *>(W8), w_scale,
                                             static_cast<const uint16_t *>(A), M, d_in, d_out, lo,
                                             gpart, s)) != hipSuccess)
            return e;
        mark(mk, "decode_gemm_fp8_lora");
        if ((e = launch_decode_reduce(gpart, M, d_in, d_out, y, y_dtype == LORA_F32, lo, true,
                                      nullptr, s)) != hipSuccess)
            return e;
        mark(mk, "decode_reduce_lora");
        return hipSuccess;
    }
    int kc, ksplit;
    shrink_plan(d_in, rb, &kc, &ksplit);
    const DecodeLora lo{spart, ksplit, static_cast<const uint16_t *>(B), scale, ids, ranks,
                        rb, n_adapters, nullptr, 0, r_max};
    const SegBuild bld{ids, n_adapters, sg};
    e = launch_decode_gemm_fp8(xb, static_cast<const uint8_t *>(W8), w_scale, M, d_in, d_out, gpart,
                               segs ? nullptr : &bld, s);
    if (e != hipSuccess) return e;
    mark(mk, "decode_gemm_fp8");
    if ((e = launch_shrink(xb, static_cast<const uint16_t *>(A), ranks, nullptr, 0, r_max, M, d_in,
                           rb, n_adapters, sg, spart, kc, ksplit, s)) != hipSuccess)
        return e;
    mark(mk, "shrink");
    if ((e = launch_decode_reduce(gpart, M, d_in, d_out, y, y_dtype == LORA_F32, lo, false, &sg, s)) !=
        hipSuccess)
        return e;
    mark(mk, "decode_reduce_lora");
    return hipSuccess;
}

lora_status_t check_fp8w(const void *x, const void *W8, const float *w_scale, const void *A,
                         const void *B, const float *scale, const int32_t *ranks,
                         const int32_t *ids, int32_t M, int32_t d_in, int32_t d_out,
                         int32_t r_max, int32_t n_adapters, const lora_segments_t *segs, void *y,
                         lora_dtype_t y_dtype, lora_mode_t mode, void *ws, size_t ws_bytes) {
    lora_status_t st = check_common(M, r_max, n_adapters);
    if (st != LORA_OK) return st;
    if (!dim_ok(d_in) || !dim_ok(d_out) || d_in % 32 != 0 || d_in < 128 ||
        M > kDecodeGemmMaxRows)
        return LORA_ERR_SHAPE;
    if (y_dtype != LORA_BF16 && y_dtype != LORA_F32) return LORA_ERR_DTYPE;
    const int bm = mode & ~LORA_MODE_CHECKED;
    if (bm != LORA_MODE_AUTO && bm != LORA_MODE_DECODE) return LORA_ERR_MODE;
    if (M == 0) return LORA_OK;
    if (!x || !W8 || !w_scale || !A || !B || !scale || !ids || !y || !ws) return LORA_ERR_NULL;
    if (segs && (st = check_seg(*segs)) != LORA_OK) return st;
    if (!aligned(x, 16) || !aligned(W8, 16) || !aligned(A, 16) || !aligned(B, 16) ||
        !aligned(y, 16) || !aligned(ws, kAlign) || !aligned(scale, 4) || !aligned(w_scale, 4) ||
        !aligned(ids, 4) || (ranks && !aligned(ranks, 4)))
        return LORA_ERR_ALIGN;
    if (ws_bytes < lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters)) return LORA_ERR_WORKSPACE;
    return LORA_OK;
}

}  // namespace

// lora_linear's body on a given workspace: shared with the entry point that brings its own
// device-resident scratch (csrc/noalloc.hip).
lora_status_t lora::linear_on_workspace(const void *x, const void *W, const void *A,
                                        const void *B, const float *scale, const int32_t *ranks,
                                        const int32_t *ids, int32_t M, int32_t d_in,
                                        int32_t d_out, int32_t r_max, int32_t n_adapters,
                                        const lora_segments_t *segs, void *y,
                                        lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                        size_t ws_bytes, void *stream) {
    lora_status_t st = check_linear(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max, n_adapters,
                                    segs, y, y_dtype, mode, ws, ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    clear_stale_error();
    if ((mode & LORA_MODE_CHECKED) &&
        (st = check_tables(ids, M, ranks, nullptr, 0, r_max, n_adapters, (hipStream_t)stream)) != LORA_OK)
        return st;
    return hip_status(run_linear(x, W, A, B, scale, ranks, nullptr, 0, ids, M, d_in, d_out, r_max,
                                 n_adapters, segs, y, y_dtype,
                                 (lora_mode_t)(mode & ~LORA_MODE_CHECKED), ws, (hipStream_t)stream,
                                 nullptr));
}

extern "C" {

lora_status_t lora_linear(const void *x, const void *W, const void *A, const void *B,
                          const float *scale, const int32_t *ranks, const int32_t *ids, int32_t M,
                          int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
                          const lora_segments_t *segs, void *y, lora_dtype_t y_dtype,
                          lora_mode_t mode, void *ws, size_t ws_bytes, void *stream) {
    return linear_on_workspace(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max, n_adapters, segs,
                               y, y_dtype, mode, ws, ws_bytes, stream);
}

lora_status_t lora_linear_compact(const void *x, const void *W, const void *A, const void *B,
                                  const float *scale, const int32_t *ranks,
                                  const int32_t *rank_offsets, int32_t pool_rows,
                                  const int32_t *ids, int32_t M, int32_t d_in, int32_t d_out,
                                  int32_t r_max, int32_t n_adapters, const lora_segments_t *segs,
                                  void *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                  size_t ws_bytes, void *stream) {
    lora_status_t st = check_linear(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max, n_adapters,
                                    segs, y, y_dtype, mode, ws, ws_bytes);
    if (st == LORA_OK) st = check_compact(ranks, rank_offsets, pool_rows, r_max, n_adapters);
    if (st != LORA_OK || M == 0) return st;
    clear_stale_error();
    if ((mode & LORA_MODE_CHECKED) &&
        (st = check_tables(ids, M, ranks, rank_offsets, pool_rows, r_max, n_adapters,
                           (hipStream_t)stream)) != LORA_OK)
        return st;
    return hip_status(run_linear(x, W, A, B, scale, ranks, rank_offsets, pool_rows, ids, M, d_in,
                                 d_out, r_max, n_adapters, segs, y, y_dtype,
                                 (lora_mode_t)(mode & ~LORA_MODE_CHECKED), ws, (hipStream_t)stream,
                                 nullptr));
}

lora_status_t lora_linear_fp8w(const void *x, const void *W8, const float *w_scale, const void *A,
                               const void *B, const float *scale, const int32_t *ranks,
                               const int32_t *ids, int32_t M, int32_t d_in, int32_t d_out,
                               int32_t r_max, int32_t n_adapters, const lora_segments_t *segs,
                               void *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                               size_t ws_bytes, void *stream) {
    lora_status_t st = check_fp8w(x, W8, w_scale, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                  n_adapters, segs, y, y_dtype, mode, ws, ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    clear_stale_error();
    if ((mode & LORA_MODE_CHECKED) &&
        (st = check_tables(ids, M, ranks, nullptr, 0, r_max, n_adapters, (hipStream_t)stream)) != LORA_OK)
        return st;
    return hip_status(run_fp8w(x, W8, w_scale, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                               n_adapters, segs, y, y_dtype, ws, (hipStream_t)stream, nullptr));
}

}  // extern "C"

namespace {

// lora_linear_multi: the most projections one merged stream-K launch takes (the largest g <=
// n_proj whose g x n_tn panels still leave the data-parallel tiling short of the chip), or 0
// when the batch does not take the stream-K path at all.
static_assert(kMaxProj == LORA_MAX_PROJ, "projection arrays");

int multi_group(int32_t M, int32_t d_in, int32_t d_out, int32_t n_proj) {
    if (!sk_plan(M, d_in, d_out).use) return 0;
    int g = n_proj;
    while (g > 1 && !sk_plan(M, d_in, d_out, g).use) --g;
    return g;
}

// Workspace of the merged stream-K sequence: segments, one shrink chunk-sum area per
// projection, the partial tiles of one group of g projections.
size_t multi_sk_bytes(int32_t M, int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
                      int32_t n_proj) {
    const int g = multi_group(M, d_in, d_out, n_proj);
    if (g < 2) return 0;
    return segments_bytes(M, n_adapters) + (size_t)n_proj * shrink_partial_bytes(M, d_in, r_max) +
           round_up(sk_partial_floats(sk_plan(M, d_in, d_out, g)) * sizeof(float));
}

// The launch sequence of lora_linear_multi (arguments already validated, M > 0).  Batches
// that take lora_linear's stream-K sequence (decode, 257-1024 rows) build the segments once,
// run every projection's shrink in one launch, then one stream-K GEMM and one reduction per
// group of up to g
// projections, whose column panels are laid end to end on one K line (longer lanes: fewer
// partial tiles per panel).  Every other batch runs lora_linear's sequence per projection.
hipError_t run_linear_multi(const void *x, int32_t n_proj, const void *const *W,
                            const void *const *A, const void *const *B, const float *scale,
                            const int32_t *ranks, const int32_t *ids, int32_t M, int32_t d_in,
                            int32_t d_out, int32_t r_max, int32_t n_adapters,
                            const lora_segments_t *segs, void *const *y, lora_dtype_t y_dtype,
                            lora_mode_t mode, void *ws, hipStream_t s, Marker *mk) {
    const bool prefill = mode == LORA_MODE_PREFILL || (mode == LORA_MODE_AUTO && M >= LORA_PREFILL_MIN_ROWS);
    const int g = prefill ? 0 : multi_group(M, d_in, d_out, n_proj);
    hipError_t e;
    if (g < 2) {
        for (int i = 0; i < n_proj; ++i)
            if ((e = run_linear(x, W[i], A[i], B[i], scale, ranks, nullptr, 0, ids, M, d_in, d_out,
                                r_max, n_adapters, segs, y[i], y_dtype, mode, ws, s, mk)) != hipSuccess)
                return e;
        return hipSuccess;
    }
    char *p = static_cast<char *>(ws);
    lora_segments_t own = carve_segments(p, M, n_adapters);
    float *spart[kMaxProj] = {};
    for (int i = 0; i < n_proj; ++i) {
        spart[i] = reinterpret_cast<float *>(p);
        p += shrink_partial_bytes(M, d_in, r_max);
    }
    float *gpart = reinterpret_cast<float *>(p);
    const Seg sg = to_seg(segs ? *segs : own);
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const int rb = rank_bucket(r_max), pstride = r_max;
    int kc, ksplit;
    shrink_plan(d_in, rb, &kc, &ksplit);
    if (!segs) {
        if ((e = launch_build_segments(ids, M, n_adapters, sg, s)) != hipSuccess) return e;
        mark(mk, "build_segments");
    }
    // every projection's shrink in one launch
    const uint16_t *Ab[kMaxProj] = {};
    for (int i = 0; i < n_proj; ++i) Ab[i] = static_cast<const uint16_t *>(A[i]);
    if ((e = launch_shrink_multi(xb, n_proj, Ab, spart, ranks, pstride, M, d_in, rb, n_adapters, sg,
                                 kc, ksplit, s)) != hipSuccess)
        return e;
    mark(mk, "shrink");
    for (int i0 = 0; i0 < n_proj; i0 += g) {
        const int gn = n_proj - i0 < g ? n_proj - i0 : g;
        const SkPlan sp = sk_plan(M, d_in, d_out, gn);
        if (!sp.use) return hipErrorInvalidValue;
        SkProj pj{};
        for (int j = 0; j < gn; ++j) {
            pj.W[j] = static_cast<const uint16_t *>(W[i0 + j]);
            pj.B[j] = static_cast<const uint16_t *>(B[i0 + j]);
            pj.tpart[j] = spart[i0 + j];
            pj.y[j] = y[i0 + j];
        }
        if ((e = launch_gemm_sk(xb, pj, M, d_in, d_out, sp, gpart, s)) != hipSuccess) return e;
        mark(mk, "gemm_decode");
        if ((e = launch_sk_reduce_lora(gpart, M, d_in, d_out, sp, sg, pj, ksplit, scale, ids, ranks,
                                       nullptr, 0, pstride, rb, n_adapters, y_dtype == LORA_F32,
                                       s)) != hipSuccess)
            return e;
        mark(mk, "decode_reduce_lora");
    }
    return hipSuccess;
}

lora_status_t check_multi(const void *x, int32_t n_proj, const void *const *W,
                          const void *const *A, const void *const *B, const float *scale,
                          const int32_t *ranks, const int32_t *ids, int32_t M, int32_t d_in,
                          int32_t d_out, int32_t r_max, int32_t n_adapters,
                          const lora_segments_t *segs, void *const *y, lora_dtype_t y_dtype,
                          lora_mode_t mode, void *ws, size_t ws_bytes) {
    if (n_proj < 1 || n_proj > LORA_MAX_PROJ) return LORA_ERR_SHAPE;
    if (!W || !A || !B || !y) return LORA_ERR_NULL;
    for (int i = 0; i < n_proj; ++i) {
        const lora_status_t st = check_linear(x, W[i], A[i], B[i], scale, ranks, ids, M, d_in, d_out,
                                              r_max, n_adapters, segs, y[i], y_dtype, mode, ws,
                                              ws_bytes);
        if (st != LORA_OK) return st;
    }
    if (ws_bytes < lora_workspace_bytes_multi(M, d_in, d_out, r_max, n_adapters, n_proj))
        return LORA_ERR_WORKSPACE;
    return LORA_OK;
}

}  // namespace

extern "C" {

size_t lora_workspace_bytes_multi(int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, int32_t n_proj) {
    if (n_proj < 1 || n_proj > LORA_MAX_PROJ) return 0;
    const size_t one = lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters);
    if (one == 0) return 0;
    const size_t merged = multi_sk_bytes(M, d_in, d_out, r_max, n_adapters, n_proj);
    return merged > one ? merged : one;
}

lora_status_t lora_linear_multi(const void *x, int32_t n_proj, const void *const *W,
                                const void *const *A, const void *const *B, const float *scale,
                                const int32_t *ranks, const int32_t *ids, int32_t M, int32_t d_in,
                                int32_t d_out, int32_t r_max, int32_t n_adapters,
                                const lora_segments_t *segs, void *const *y, lora_dtype_t y_dtype,
                                lora_mode_t mode, void *ws, size_t ws_bytes, void *stream) {
    lora_status_t st = check_multi(x, n_proj, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                   n_adapters, segs, y, y_dtype, mode, ws, ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    clear_stale_error();
    if ((mode & LORA_MODE_CHECKED) &&
        (st = check_tables(ids, M, ranks, nullptr, 0, r_max, n_adapters, (hipStream_t)stream)) != LORA_OK)
        return st;
    return hip_status(run_linear_multi(x, n_proj, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                       n_adapters, segs, y, y_dtype,
                                       (lora_mode_t)(mode & ~LORA_MODE_CHECKED), ws,
                                       (hipStream_t)stream, nullptr));
}

}  // extern "C"

namespace {

// lora_linear / lora_linear_compact with each launch timed by start / stop events taken
// from its own dispatch packet (arguments already validated, M > 0).
// `run(marker)` enqueues a call's launches; each is timed by start / stop events taken from its
// own dispatch packet.  Waits for the last one and reports the durations in launch order.
template <class F>
lora_status_t time_launches(F run, float *kernel_ms, const char **kernel_names, int32_t max_kernels,
                            int32_t *n_kernels) {
    clear_stale_error();
    KernelTimer timer;
    hipError_t e = hipSuccess;
    int made = 0;
    for (; made < KernelTimer::kMax && e == hipSuccess; ++made) {
        e = hipEventCreate(&timer.start[made]);
        if (e == hipSuccess) e = hipEventCreate(&timer.stop[made]);
    }
    Marker mk;
    if (e == hipSuccess) {
        g_timer = &timer;
        e = run(&mk);
        g_timer = nullptr;
    }
    if (e == hipSuccess && timer.n > 0) e = hipEventSynchronize(timer.stop[timer.n - 1]);
    const int n = timer.n < mk.n ? timer.n : mk.n;
    for (int i = 0; e == hipSuccess && i < n; ++i) {
        float ms = 0.0f;
        e = hipEventElapsedTime(&ms, timer.start[i], timer.stop[i]);
        if (i < max_kernels) {
            kernel_ms[i] = ms;
            kernel_names[i] = mk.names[i];
        }
    }
    if (e == hipSuccess) *n_kernels = n < max_kernels ? n : max_kernels;
    for (int i = 0; i < KernelTimer::kMax; ++i) {
        if (timer.start[i]) (void)hipEventDestroy(timer.start[i]);
        if (timer.stop[i]) (void)hipEventDestroy(timer.stop[i]);
    }
    return hip_status(e);
}

lora_status_t run_profiled(const void *x, const void *W, const void *A, const void *B,
                           const float *scale, const int32_t *ranks, const int32_t *roff,
                           int32_t pool_rows, const int32_t *ids, int32_t M, int32_t d_in,
                           int32_t d_out, int32_t r_max, int32_t n_adapters,
                           const lora_segments_t *segs, void *y, lora_dtype_t y_dtype,
                           lora_mode_t mode, void *ws, void *stream, float *kernel_ms,
                           const char **kernel_names, int32_t max_kernels, int32_t *n_kernels) {
    return time_launches(
        [&](Marker *mk) {
            return run_linear(x, W, A, B, scale, ranks, roff, pool_rows, ids, M, d_in, d_out, r_max,
                              n_adapters, segs, y, y_dtype, (lora_mode_t)(mode & ~LORA_MODE_CHECKED),
                              ws, (hipStream_t)stream, mk);
        },
        kernel_ms, kernel_names, max_kernels, n_kernels);
}

}  // namespace

extern "C" {

lora_status_t lora_linear_profiled(const void *x, const void *W, const void *A, const void *B,
                                   const float *scale, const int32_t *ranks, const int32_t *ids,
                                   int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                   int32_t n_adapters, const lora_segments_t *segs, void *y,
                                   lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                   size_t ws_bytes, void *stream, float *kernel_ms,
                                   const char **kernel_names, int32_t max_kernels,
                                   int32_t *n_kernels) {
    if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0) return LORA_ERR_NULL;
    *n_kernels = 0;
    lora_status_t st = check_linear(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max, n_adapters,
                                    segs, y, y_dtype, mode, ws, ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    return run_profiled(x, W, A, B, scale, ranks, nullptr, 0, ids, M, d_in, d_out, r_max,
                        n_adapters, segs, y, y_dtype, mode, ws, stream, kernel_ms, kernel_names,
                        max_kernels, n_kernels);
}

lora_status_t lora_linear_multi_profiled(
    const void *x, int32_t n_proj, const void *const *W, const void *const *A,
    const void *const *B, const float *scale, const int32_t *ranks, const int32_t *ids, int32_t M,
    int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters, const lora_segments_t *segs,
    void *const *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws, size_t ws_bytes, void *stream,
    float *kernel_ms, const char **kernel_names, int32_t max_kernels, int32_t *n_kernels) {
    if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0) return LORA_ERR_NULL;
    *n_kernels = 0;
    lora_status_t st = check_multi(x, n_proj, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                   n_adapters, segs, y, y_dtype, mode, ws, ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    return time_launches(
        [&](Marker *mk) {
            return run_linear_multi(x, n_proj, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                    n_adapters, segs, y, y_dtype,
                                    (lora_mode_t)(mode & ~LORA_MODE_CHECKED), ws,
                                    (hipStream_t)stream, mk);
        },
        kernel_ms, kernel_names, max_kernels, n_kernels);
}

lora_status_t lora_linear_compact_profiled(
    const void *x, const void *W, const void *A, const void *B, const float *scale,
    const int32_t *ranks, const int32_t *rank_offsets, int32_t pool_rows, const int32_t *ids,
    int32_t M, int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
    const lora_segments_t *segs, void *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
    size_t ws_bytes, void *stream, float *kernel_ms, const char **kernel_names,
    int32_t max_kernels, int32_t *n_kernels) {
    if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0) return LORA_ERR_NULL;
    *n_kernels = 0;
    lora_status_t st = check_linear(x, W, A, B, scale, ranks, ids, M, d_in, d_out, r_max, n_adapters,
                                    segs, y, y_dtype, mode, ws, ws_bytes);
    if (st == LORA_OK) st = check_compact(ranks, rank_offsets, pool_rows, r_max, n_adapters);
    if (st != LORA_OK || M == 0) return st;
    return run_profiled(x, W, A, B, scale, ranks, rank_offsets, pool_rows, ids, M, d_in, d_out,
                        r_max, n_adapters, segs, y, y_dtype, mode, ws, stream, kernel_ms,
                        kernel_names, max_kernels, n_kernels);
}

lora_status_t lora_linear_fp8w_profiled(const void *x, const void *W8, const float *w_scale,
                                        const void *A, const void *B, const float *scale,
                                        const int32_t *ranks, const int32_t *ids, int32_t M,
                                        int32_t d_in, int32_t d_out, int32_t r_max,
                                        int32_t n_adapters, const lora_segments_t *segs, void *y,
                                        lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                        size_t ws_bytes, void *stream, float *kernel_ms,
                                        const char **kernel_names, int32_t max_kernels,
                                        int32_t *n_kernels) {
    if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0) return LORA_ERR_NULL;
    *n_kernels = 0;
    lora_status_t st = check_fp8w(x, W8, w_scale, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                                  n_adapters, segs, y, y_dtype, mode, ws, ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    return time_launches(
        [&](Marker *mk) {
            return run_fp8w(x, W8, w_scale, A, B, scale, ranks, ids, M, d_in, d_out, r_max,
                            n_adapters, segs, y, y_dtype, ws, (hipStream_t)stream, mk);
        },
        kernel_ms, kernel_names, max_kernels, n_kernels);
}

}  // extern "C"

namespace {

// ---- MoE-LoRA ----------------------------------------------------------------------------

lora_status_t check_moe_sizes(int32_t M, int32_t top_k, int32_t n_experts, int32_t d_in,
                              int32_t d_out, int32_t r_max, int32_t n_adapters) {
    if (M < 0 || top_k < 1 || top_k > 64 || n_experts < 1 || n_experts > 4096 ||
        (int64_t)M * top_k > LORA_MOE_MAX_PAIRS || n_adapters < 1 ||
        n_adapters > LORA_MAX_ADAPTERS)
        return LORA_ERR_SHAPE;
    if (!dim_ok(d_in) || !dim_ok(d_out) || d_in % 32 != 0 || d_in < 128) return LORA_ERR_SHAPE;
    if (r_max < 8 || r_max > 64 || r_max % 8 != 0) return LORA_ERR_RANK;
    return LORA_OK;
}

size_t moe_ws_bytes(int32_t M, int32_t top_k, int32_t n_experts, int32_t d_in, int32_t d_out,
                    int32_t r_max, int32_t n_adapters) {
    const MoePlan p = moe_plan(M, top_k, n_experts, d_in, d_out, r_max, n_adapters);
    const int P = M * top_k;
    return round_up(moe_partial_floats(p, P) * 4) + round_up(moe_tpart_floats(p, P) * 4);
}

lora_status_t check_moe(const void *x, const void *W, const void *A, const void *B,
                        const float *scale, const int32_t *ranks, const int32_t *ids,
                        const int32_t *topk_ids, const float *topk_w, int32_t M, int32_t top_k,
                        int32_t n_experts, int32_t d_in, int32_t d_out, int32_t r_max,
                        int32_t n_adapters, void *y, lora_dtype_t y_dtype, lora_mode_t mode,
                        void *ws, size_t ws_bytes) {
    lora_status_t st = check_moe_sizes(M, top_k, n_experts, d_in, d_out, r_max, n_adapters);
    if (st != LORA_OK) return st;
    if (y_dtype != LORA_BF16 && y_dtype != LORA_F32) return LORA_ERR_DTYPE;
    const int bm = mode & ~LORA_MODE_CHECKED;
    if (bm != LORA_MODE_AUTO && bm != LORA_MODE_DECODE) return LORA_ERR_MODE;
    if (M == 0) return LORA_OK;
    if (!x || !W || !A || !B || !scale || !ids || !topk_ids || !y || !ws) return LORA_ERR_NULL;
    if (!aligned(x, 16) || !aligned(W, 16) || !aligned(A, 16) || !aligned(B, 16) ||
        !aligned(y, 16) || !aligned(ws, kAlign) || !aligned(scale, 4) || !aligned(ids, 4) ||
        !aligned(topk_ids, 4) || (topk_w && !aligned(topk_w, 4)) || (ranks && !aligned(ranks, 4)))
        return LORA_ERR_ALIGN;
    if (ws_bytes < moe_ws_bytes(M, top_k, n_experts, d_in, d_out, r_max, n_adapters))
        return LORA_ERR_WORKSPACE;
    return LORA_OK;
}

// Checked mode of lora_moe_linear: ids and ranks as lora_linear's, and every topk_ids entry
// in [-1, n_experts).
lora_status_t check_moe_tables(const int32_t *ids, const int32_t *ranks, const int32_t *topk_ids,
                               int32_t M, int32_t top_k, int32_t n_experts, int32_t r_max,
                               int32_t n_adapters, hipStream_t s) {
    lora_status_t st = check_tables(ids, M, ranks, nullptr, 0, r_max, n_adapters, s);
    if (st != LORA_OK) return st;
    std::vector<int32_t> h((size_t)M * top_k);
    hipError_t e = hipMemcpy(h.data(), topk_ids, h.size() * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e);
    for (int32_t v : h)
        if (v < -1 || v >= n_experts) return LORA_ERR_BAD_ID;
    return LORA_OK;
}

// The launch sequence of lora_moe_linear (arguments validated, M > 0): the expert-routed
// split-K GEMM with the adapters' A as extra column tiles, then the reduction with the expand
// and the routing weight.
hipError_t run_moe(const void *x, const void *W, const void *A, const void *B, const float *scale,
                   const int32_t *ranks, const int32_t *ids, const int32_t *topk_ids,
                   const float *topk_w, int32_t M, int32_t top_k, int32_t n_experts, int32_t d_in,
                   int32_t d_out, int32_t r_max, int32_t n_adapters, void *y,
                   lora_dtype_t y_dtype, void *ws, hipStream_t s, Marker *mk) {
    const MoePlan p = moe_plan(M, top_k, n_experts, d_in, d_out, r_max, n_adapters);
    const int P = M * top_k;
    char *c = static_cast<char *>(ws);
    float *partial = reinterpret_cast<float *>(c);
    c += round_up(moe_partial_floats(p, P) * 4);
    float *tpart = reinterpret_cast<float *>(c);
    MoeGemmArgs g{};
    g.x = static_cast<const uint16_t *>(x);
    g.W = static_cast<const uint16_t *>(W);
    g.A = static_cast<const uint16_t *>(A);
    g.topk_ids = topk_ids;
    g.ids = ids;
    g.P = P; g.top_k = top_k; g.E = n_experts; g.K = d_in; g.N = d_out;
    g.r_stride = r_max; g.n_adapters = n_adapters;
    g.partial = partial;
    g.tpart = tpart;
    hipError_t e = launch_moe_gemm(p, g, s);
    if (e != hipSuccess) return e;
    mark(mk, "moe_gemm");
    MoeReduceArgs r{};
    r.partial = partial; r.tpart = tpart;
    r.B = static_cast<const uint16_t *>(B);
    r.scale = scale; r.ranks = ranks; r.topk_ids = topk_ids; r.ids = ids; r.topk_w = topk_w;
    r.P = P; r.top_k = top_k; r.E = n_experts; r.N = d_out; r.r_stride = r_max;
    r.n_adapters = n_adapters;
    r.y = y;
    if ((e = launch_moe_reduce(p, r, y_dtype == LORA_F32, s)) != hipSuccess) return e;
    mark(mk, "moe_reduce");
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t lora_moe_workspace_bytes(int32_t M, int32_t top_k, int32_t n_experts, int32_t d_in,
                                int32_t d_out, int32_t r_max, int32_t n_adapters) {
    if (check_moe_sizes(M, top_k, n_experts, d_in, d_out, r_max, n_adapters) != LORA_OK || M == 0)
        return 0;
    return moe_ws_bytes(M, top_k, n_experts, d_in, d_out, r_max, n_adapters);
}

lora_status_t lora_moe_linear(const void *x, const void *W, const void *A, const void *B,
                              const float *scale, const int32_t *ranks, const int32_t *ids,
                              const int32_t *topk_ids, const float *topk_w, int32_t M,
                              int32_t top_k, int32_t n_experts, int32_t d_in, int32_t d_out,
                              int32_t r_max, int32_t n_adapters, void *y, lora_dtype_t y_dtype,
                              lora_mode_t mode, void *ws, size_t ws_bytes, void *stream) {
    lora_status_t st = check_moe(x, W, A, B, scale, ranks, ids, topk_ids, topk_w, M, top_k,
                                 n_experts, d_in, d_out, r_max, n_adapters, y, y_dtype, mode, ws,
                                 ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    clear_stale_error();
    if ((mode & LORA_MODE_CHECKED) &&
        (st = check_moe_tables(ids, ranks, topk_ids, M, top_k, n_experts, r_max, n_adapters,
                               (hipStream_t)stream)) != LORA_OK)
        return st;
    return hip_status(run_moe(x, W, A, B, scale, ranks, ids, topk_ids, topk_w, M, top_k, n_experts,
                              d_in, d_out, r_max, n_adapters, y, y_dtype, ws, (hipStream_t)stream,
                              nullptr));
}

lora_status_t lora_moe_linear_profiled(const void *x, const void *W, const void *A, const void *B,
                                       const float *scale, const int32_t *ranks,
                                       const int32_t *ids, const int32_t *topk_ids,
                                       const float *topk_w, int32_t M, int32_t top_k,
                                       int32_t n_experts, int32_t d_in, int32_t d_out,
                                       int32_t r_max, int32_t n_adapters, void *y,
                                       lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                       size_t ws_bytes, void *stream, float *kernel_ms,
                                       const char **kernel_names, int32_t max_kernels,
                                       int32_t *n_kernels) {
    if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0) return LORA_ERR_NULL;
    *n_kernels = 0;
    lora_status_t st = check_moe(x, W, A, B, scale, ranks, ids, topk_ids, topk_w, M, top_k,
                                 n_experts, d_in, d_out, r_max, n_adapters, y, y_dtype, mode, ws,
                                 ws_bytes);
    if (st != LORA_OK || M == 0) return st;
    return time_launches(
        [&](Marker *mk) {
            return run_moe(x, W, A, B, scale, ranks, ids, topk_ids, topk_w, M, top_k, n_experts,
                           d_in, d_out, r_max, n_adapters, y, y_dtype, ws, (hipStream_t)stream, mk);
        },
        kernel_ms, kernel_names, max_kernels, n_kernels);
}

const char *lora_status_string(lora_status_t status) {
    switch (status) {
        case LORA_OK: return "LORA_OK";
        case LORA_ERR_NULL: return "LORA_ERR_NULL: a required pointer is NULL";
        case LORA_ERR_SHAPE: return "LORA_ERR_SHAPE: M, d_in, d_out, n_adapters (or top_k, n_experts) out of range";
        case LORA_ERR_RANK: return "LORA_ERR_RANK: r_max outside [1, 64], or (checked mode) a rank outside [1, r_max]";
        case LORA_ERR_ALIGN: return "LORA_ERR_ALIGN: a pointer is not aligned as required";
        case LORA_ERR_WORKSPACE:
            return "LORA_ERR_WORKSPACE: workspace smaller than lora_workspace_bytes() (lora_linear_noalloc: "
                   "the call needs more than LORA_NOALLOC_SCRATCH_BYTES of scratch)";
        case LORA_ERR_DTYPE: return "LORA_ERR_DTYPE: unknown output dtype";
        case LORA_ERR_HIP: return "LORA_ERR_HIP: a kernel launch failed";
        case LORA_ERR_BAD_ID: return "LORA_ERR_BAD_ID: (checked mode) adapter id or expert id out of range";
        case LORA_ERR_MODE: return "LORA_ERR_MODE: unknown mode";
        case LORA_ERR_POOL: return "LORA_ERR_POOL: (checked mode) an adapter's rank rows leave the compact pool";
    }
    return "unknown lora_status_t";
}

const char *lora_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

}  // extern "C"

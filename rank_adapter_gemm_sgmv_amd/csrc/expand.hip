// expand.hip -- y[m, :] += scale_i * (t[m, :] B_i) for every row of a mixed batch.
//
// Source: the adapter "expand" step of "Multi-LoRA Serving: Sharing One GPU Across Adapters"
// (cloudai.pt), "MoE Models Raise the Bar"; the scale alpha / r of the layer equation in
// "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Why can't you just merge
// LoRA weights into the base model?".  Memory-bound on B_i (same page, "How does one batch
// run 30 different adapters at once?").
//
// Work item = (tile, column chunk), one wave each.  The wave holds B_i[0:rank, chunk] in
// registers -- CPL consecutive columns per lane (8 for r_max <= 16, else 4), one load per
// rank row, rows at or beyond the adapter's rank are neither read nor multiplied -- and
// streams the tile's rows past it, four at a time: for each row the lane's CPL columns of y
// and one element of t[m, :] (lane j holds t[m, j], broadcast with readlane) are loaded
// together for the whole batch, and each B_i row is unpacked once per batch.  So each B_i
// slice is read once per tile.  The sum over j runs in ascending order in fp32; then
// y = y + scale * sum is rounded once into y's dtype.  Base-only rows are never touched.
#include "common.h"

namespace lora {

namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMaxGrid = 1 << 20;
constexpr int RB = 4;  // rows whose loads are in flight together

template <int RM>
struct ExpandLanes {
    static constexpr int CPL = RM <= 16 ? 8 : 4;  // columns per lane
    static constexpr int COLS = 64 * CPL;         // columns per work item
    static constexpr int BW = CPL / 2;            // 32-bit words of B per rank row and lane
};

template <int CPL>
struct Vec;
template <>
struct Vec<8> {
    uint4 v;
};
template <>
struct Vec<4> {
    uint2 v;
};

template <int CPL>
__device__ __forceinline__ Vec<CPL> ldv(const uint16_t *p) {
    Vec<CPL> r;
    if constexpr (CPL == 8) r.v = *reinterpret_cast<const uint4 *>(p);
    else r.v = *reinterpret_cast<const uint2 *>(p);
    return r;
}

template <int CPL>
__device__ __forceinline__ void unpackv(const Vec<CPL> &b, float (&f)[CPL]) {
    if constexpr (CPL == 8) {
        unpack8(b.v, f);
    } else {
        f[0] = bf16_lo(b.v.x); f[1] = bf16_hi(b.v.x);
        f[2] = bf16_lo(b.v.y); f[3] = bf16_hi(b.v.y);
    }
}

// y row slice: bf16 (CPL * 2 bytes) or f32 (CPL * 4 bytes)
template <int CPL, bool YF32>
struct YSlice {
    float f[CPL];
};

template <int CPL, bool YF32>
__device__ __forceinline__ void load_y(YSlice<CPL, YF32> &ys, const void *y, size_t off) {
    if constexpr (YF32) {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(y) + off);
#pragma unroll
        for (int q = 0; q < CPL / 4; ++q) {
            const float4 v = p[q];
            ys.f[4 * q] = v.x; ys.f[4 * q + 1] = v.y; ys.f[4 * q + 2] = v.z; ys.f[4 * q + 3] = v.w;
        }
    } else {
        const Vec<CPL> v = ldv<CPL>(reinterpret_cast<const uint16_t *>(y) + off);
        unpackv<CPL>(v, ys.f);
    }
}

template <int CPL, bool YF32>
__device__ __forceinline__ void store_y(void *y, size_t off, const float (&f)[CPL]) {
    if constexpr (YF32) {
        float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + off);
#pragma unroll
        for (int q = 0; q < CPL / 4; ++q) p[q] = make_float4(f[4 * q], f[4 * q + 1], f[4 * q + 2], f[4 * q + 3]);
    } else {
        uint16_t *p = reinterpret_cast<uint16_t *>(y) + off;
        if constexpr (CPL == 8) {
            st16(p, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                               pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])));
        } else {
            *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
        }
    }
}

// t rows are t_stride floats apart; a padded pool (roff == nullptr) holds pstride <= RM rank
// rows per adapter.
template <int RM, bool YF32>
__global__ __launch_bounds__(64 * kWavesPerBlock) void expand_kernel(
    const float *__restrict__ t, int t_stride, const uint16_t *__restrict__ B,
    const float *__restrict__ scale, const int32_t *__restrict__ ranks,
    const int32_t *__restrict__ roff, int pool_rows, int pstride, int M, int d_out, int n_cc,
    int n_adapters, Seg seg, void *__restrict__ y) {
    using L = ExpandLanes<RM>;
    constexpr int CPL = L::CPL;
    const int lane = threadIdx.x & 63;
    const int total = seg.meta[3] * n_cc;
    const int nw = gridDim.x * kWavesPerBlock;
    for (int w = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); w < total; w += nw) {
        const int tile = w / n_cc, cc = w % n_cc;
        const int p0 = seg.tiles[2 * tile], a = seg.tiles[2 * tile + 1];
        if (a < 0 || a >= n_adapters) continue;  // only in segments a caller built: adds nothing
        const int p1 = min(p0 + kTileRows, seg.offsets[a + 1]);
        const int width = roff ? RM : pstride;
        int r = ranks ? min(max(ranks[a], 0), width) : width;
        const int row0 = adapter_row0(roff, pool_rows, a, pstride, r);
        const float s = scale[a];
        const int c = cc * L::COLS + lane * CPL;
        const bool colok = c < d_out;  // d_out % 8 == 0: a lane's columns are all in or all out
        const int cl = colok ? c : 0;

        // B_a[0:r, c .. c+CPL): one load per rank row, all issued together.  Rows at or
        // beyond the rank load row r - 1 again (the same cache lines: no extra HBM bytes)
        // and are multiplied by zero below.
        Vec<CPL> bj[RM];
        const uint16_t *Bp = B + (size_t)row0 * d_out + cl;
        const int rl = r > 0 ? r - 1 : 0;
#pragma unroll
        for (int j = 0; j < RM; ++j) bj[j] = ldv<CPL>(Bp + (size_t)min(j, rl) * d_out);

        // rows of the tile in batches of RB: the lane's y slice of each row and t[m, lane]
        // (lane j < r_max holds t[m, j]; read back with readlane) are loaded together
        for (int pb = p0; pb < p1; pb += RB) {
            int mb[RB];
            YSlice<CPL, YF32> yb[RB];
            float tv[RB];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                mb[i] = seg.perm[min(pb + i, M - 1)];
                load_y<CPL, YF32>(yb[i], y, (size_t)mb[i] * d_out + cl);
                tv[i] = t[(size_t)mb[i] * t_stride + (lane < r ? lane : 0)];
            }
            float acc[RB][CPL];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int e = 0; e < CPL; ++e) acc[i][e] = 0.0f;
            // keep B packed across the row loop: unpacking it once outside would hold
            // RM x CPL floats live and serialise its loads
#pragma unroll
            for (int j = 0; j < RM; ++j) {
                if constexpr (CPL == 8) {
                    asm volatile("" : "+v"(bj[j].v.x), "+v"(bj[j].v.y), "+v"(bj[j].v.z), "+v"(bj[j].v.w));
                } else {
                    asm volatile("" : "+v"(bj[j].v.x), "+v"(bj[j].v.y));
                }
            }
            // rank row j outer: B_a[j] is unpacked once per batch and used by all its rows
#pragma unroll
            for (int j = 0; j < RM; ++j) {
                if (j < r) {  // uniform: the wave's adapter
                    float b[CPL];
                    unpackv<CPL>(bj[j], b);
#pragma unroll
                    for (int i = 0; i < RB; ++i) {
                        const float tj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tv[i]), j));
#pragma unroll
                        for (int e = 0; e < CPL; ++e) acc[i][e] = fmaf(tj, b[e], acc[i][e]);
                    }
                }
            }
            if (colok) {
#pragma unroll
                for (int i = 0; i < RB; ++i) {
                    if (pb + i < p1) {
                        float out[CPL];
#pragma unroll
                        for (int e = 0; e < CPL; ++e) out[e] = fmaf(s, acc[i][e], yb[i].f[e]);
                        store_y<CPL, YF32>(y, (size_t)mb[i] * d_out + c, out);
                    }
                }
            }
        }
    }
}

template <int RM>
hipError_t launch_rm(const float *t, int t_stride, const uint16_t *B, const float *scale,
                     const int32_t *ranks, const int32_t *roff, int pool_rows, int pstride, int M,
                     int d_out, int n_adapters, Seg seg, void *y, bool y_f32, hipStream_t s) {
    using L = ExpandLanes<RM>;
    const int n_cc = (d_out + L::COLS - 1) / L::COLS;
    const long items = (long)lora_max_tiles(M, n_adapters) * n_cc;
    const long blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    const dim3 grid((unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid));
    const dim3 block(64 * kWavesPerBlock);
    if (y_f32)
        launch((expand_kernel<RM, true>), grid, block, 0, s, t, t_stride, B, scale, ranks, roff,
               pool_rows, pstride, M, d_out, n_cc, n_adapters, seg, y);
    else
        launch((expand_kernel<RM, false>), grid, block, 0, s, t, t_stride, B, scale, ranks, roff,
               pool_rows, pstride, M, d_out, n_cc, n_adapters, seg, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand(const float *t, int t_stride, const uint16_t *B, const float *scale,
                         const int32_t *ranks, const int32_t *roff, int pool_rows, int pstride,
                         int M, int d_out, int r_max, int n_adapters, Seg seg, void *y, bool y_f32,
                         hipStream_t s) {
    if ((roff == nullptr && (pstride < 1 || pstride > r_max)) || t_stride < 1) return hipErrorInvalidValue;
    switch (r_max) {
        case 8: return launch_rm<8>(t, t_stride, B, scale, ranks, roff, pool_rows, pstride, M, d_out, n_adapters, seg, y, y_f32, s);
        case 16: return launch_rm<16>(t, t_stride, B, scale, ranks, roff, pool_rows, pstride, M, d_out, n_adapters, seg, y, y_f32, s);
        case 32: return launch_rm<32>(t, t_stride, B, scale, ranks, roff, pool_rows, pstride, M, d_out, n_adapters, seg, y, y_f32, s);
        case 64: return launch_rm<64>(t, t_stride, B, scale, ranks, roff, pool_rows, pstride, M, d_out, n_adapters, seg, y, y_f32, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lora

// expand.hip -- y[m, :] += scale_i * (t[m, :] B_i) for every row of a mixed batch.
//
// Source: the adapter "expand" step of "Multi-LoRA Serving: Sharing One GPU Across Adapters"
// (cloudai.pt), "MoE Models Raise the Bar"; the scale alpha / r of the layer equation in
// "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Why can't you just merge
// LoRA weights into the base model?".  Memory-bound on B_i (same page, "How does one batch
// run 30 different adapters at once?").
//
// Work item = (tile, 512-column chunk), one wave64 each, 8 consecutive columns per lane, so
// every load of B_i[j, c:c+8] and of y is a 16-byte vector and a wave touches 1 KiB
// contiguous per B row.  For r_max <= 16 the wave keeps its B_i[0:r, c:c+8] slice in
// registers and sweeps the tile's rows over it, so B_i comes from HBM once per tile; for
// larger r_max the rows re-read it from L1/L2.  t[m, :] is uniform across the wave and is
// read through the scalar cache.  The sum over j runs in ascending order in fp32; then
// y = y + scale * sum is rounded once into y's dtype.  Base-only rows are never touched.
#include "common.h"

namespace lora {

namespace {

constexpr int kCols = 512;  // columns per work item: 64 lanes x 8
constexpr int kMaxGrid = 1 << 20;

template <bool YF32>
__device__ __forceinline__ void add_into_y(void *y, size_t off, const float acc[8], float s) {
    if constexpr (YF32) {
        float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + off);
        float4 a = p[0], b = p[1];
        a.x = fmaf(s, acc[0], a.x); a.y = fmaf(s, acc[1], a.y);
        a.z = fmaf(s, acc[2], a.z); a.w = fmaf(s, acc[3], a.w);
        b.x = fmaf(s, acc[4], b.x); b.y = fmaf(s, acc[5], b.y);
        b.z = fmaf(s, acc[6], b.z); b.w = fmaf(s, acc[7], b.w);
        p[0] = a;
        p[1] = b;
    } else {
        uint16_t *p = reinterpret_cast<uint16_t *>(y) + off;
        const uint4 v = ld16(p);
        float f[8];
        unpack8(v, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = fmaf(s, acc[e], f[e]);
        st16(p, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                           pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])));
    }
}

template <int RM, bool YF32>
__global__ __launch_bounds__(64) void expand_kernel(const float *__restrict__ t,
                                                    const uint16_t *__restrict__ B,
                                                    const float *__restrict__ scale,
                                                    const int32_t *__restrict__ ranks, int d_out,
                                                    int n_cc, Seg seg, void *__restrict__ y) {
    const int lane = threadIdx.x;
    const int total = seg.meta[3] * n_cc;
    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        const int tile = w / n_cc, cc = w % n_cc;
        const int p0 = seg.tiles[2 * tile], a = seg.tiles[2 * tile + 1];
        const int p1 = min(p0 + kTileRows, seg.offsets[a + 1]);
        const int r = ranks ? min(max(ranks[a], 0), RM) : RM;
        const float s = scale[a];
        const int c = cc * kCols + lane * 8;
        if (c >= d_out) continue;  // no barriers in this kernel: idle lanes may leave
        const uint16_t *Bp = B + (size_t)a * RM * d_out + c;

        if constexpr (RM <= 16) {
            uint4 bj[RM];
#pragma unroll
            for (int j = 0; j < RM; ++j)
                bj[j] = (j < r) ? ld16(Bp + (size_t)j * d_out) : make_uint4(0, 0, 0, 0);
            for (int p = p0; p < p1; ++p) {
                const int m = seg.perm[p];
                const float *tm = t + (size_t)m * RM;
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
                for (int j = 0; j < RM; ++j) {
                    if (j < r) {
                        float b[8];
                        unpack8(bj[j], b);
                        const float tj = tm[j];
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] = fmaf(tj, b[e], acc[e]);
                    }
                }
                add_into_y<YF32>(y, (size_t)m * d_out + c, acc, s);
            }
        } else {
            for (int p = p0; p < p1; ++p) {
                const int m = seg.perm[p];
                const float *tm = t + (size_t)m * RM;
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
                for (int j0 = 0; j0 < r; j0 += 16) {
                    uint4 bj[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        bj[u] = (j0 + u < r) ? ld16(Bp + (size_t)(j0 + u) * d_out) : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 16; ++u) {
                        if (j0 + u < r) {
                            float b[8];
                            unpack8(bj[u], b);
                            const float tj = tm[j0 + u];
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc[e] = fmaf(tj, b[e], acc[e]);
                        }
                    }
                }
                add_into_y<YF32>(y, (size_t)m * d_out + c, acc, s);
            }
        }
    }
}

template <int RM>
hipError_t launch_rm(const float *t, const uint16_t *B, const float *scale, const int32_t *ranks,
                     int d_out, int n_cc, int grid, Seg seg, void *y, bool y_f32, hipStream_t s) {
    if (y_f32)
        launch((expand_kernel<RM, true>), dim3(grid), dim3(64), 0, s, t, B, scale, ranks, d_out, n_cc, seg, y);
    else
        launch((expand_kernel<RM, false>), dim3(grid), dim3(64), 0, s, t, B, scale, ranks, d_out, n_cc, seg, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand(const float *t, const uint16_t *B, const float *scale,
                         const int32_t *ranks, int M, int d_out, int r_max, int n_adapters,
                         Seg seg, void *y, bool y_f32, hipStream_t s) {
    const int n_cc = (d_out + kCols - 1) / kCols;
    const long items = (long)lora_max_tiles(M, n_adapters) * n_cc;
    const int grid = (int)(items < kMaxGrid ? items : kMaxGrid);
    switch (r_max) {
        case 8: return launch_rm<8>(t, B, scale, ranks, d_out, n_cc, grid, seg, y, y_f32, s);
        case 16: return launch_rm<16>(t, B, scale, ranks, d_out, n_cc, grid, seg, y, y_f32, s);
        case 32: return launch_rm<32>(t, B, scale, ranks, d_out, n_cc, grid, seg, y, y_f32, s);
        case 64: return launch_rm<64>(t, B, scale, ranks, d_out, n_cc, grid, seg, y, y_f32, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lora

// shrink.hip -- t = x A_i per row, for all adapters of a mixed batch in one launch.
//
// Source: the adapter "shrink" step of "Multi-LoRA Serving: Sharing One GPU Across
// Adapters" (cloudai.pt), section "MoE Models Raise the Bar", which also names split-K for
// these skinny products; the [B, 4096] x [4096, r] product of "Multi-LoRA Serving: Why 100
// Adapters Fit on One GPU" (dev.to), "How does one batch run 30 different adapters at
// once?", memory-bound on the adapter weights.
//
// Work item = (tile, k-chunk): a tile is up to LORA_TILE_ROWS rows of one adapter a (from
// the segment builder), a k-chunk is kKC consecutive rows of A_a.  Because A_a[k0:k0+kKC, :]
// is one contiguous block of the padded pool, the workgroup streams it with 16-byte loads
// (only the column groups below the adapter's rank are fetched), together with its rows of
// x, into LDS, and every A_a byte is read from HBM once per segment (tiles of one adapter
// share the chunk through L2: their block ids differ by a multiple of the k-split, hence by
// a multiple of 8, so they are dispatched to the same XCD).
//
// Inside the workgroup, thread = (row q, column group g of 8 rank columns, k-slice ks):
// it accumulates 8 fp32 sums over its contiguous k-slice from LDS, then the k-slices of one
// (q, g) -- adjacent lanes -- are added by an xor butterfly.  The partial sums of each
// k-chunk go to partial[chunk][row][j]; lora_shrink sums them in chunk order
// (shrink_finalize_kernel), so the result does not depend on scheduling.
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 256;
constexpr int kKC = 256;  // k rows of A per work item

template <int RM>
__global__ __launch_bounds__(kThreads) void shrink_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ A,
                                                          const int32_t *__restrict__ ranks,
                                                          int M, int d_in, Seg seg,
                                                          float *__restrict__ partial,
                                                          int ksplit) {
    constexpr int JG = RM / 8;        // 16-byte column groups per row of A_a
    constexpr int KSUB = 16 / JG;     // threads splitting the k-chunk of one (row, group)
    constexpr int KCS = kKC / KSUB;   // k rows per thread
    constexpr int XC = kKC / 8;       // 16-byte chunks per staged row of x
    static_assert(kTileRows * JG * KSUB == kThreads, "thread layout");

    // A chunk: row k at LDS row k + k / KCS (one pad row per k-slice keeps the 16 lanes
    // of one read instruction on distinct banks); x rows padded by one 16-byte chunk.
    __shared__ uint4 As[(kKC + KSUB) * JG];
    __shared__ uint4 Xs[kTileRows][XC + 1];

    const int tid = threadIdx.x;
    const int ksub = tid % KSUB;
    const int g = (tid / KSUB) % JG;
    const int q = tid / (KSUB * JG);

    const int total = seg.meta[3] * ksplit;
    for (int w = blockIdx.x; w < total; w += gridDim.x) {
        const int tile = w / ksplit, kcx = w % ksplit;
        const int p0 = seg.tiles[2 * tile], a = seg.tiles[2 * tile + 1];
        const int rows = min(p0 + kTileRows, seg.offsets[a + 1]) - p0;
        const int r = ranks ? min(max(ranks[a], 0), RM) : RM;
        const int k0 = kcx * kKC;
        const int kn = min(kKC, d_in - k0);

        const uint16_t *Ab = A + ((size_t)a * d_in + k0) * RM;
        for (int pc = tid; pc < kKC * JG; pc += kThreads) {
            const int k = pc / JG, gg = pc % JG;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k < kn && gg * 8 < r) v = ld16(Ab + (size_t)k * RM + gg * 8);
            As[(k + k / KCS) * JG + gg] = v;
        }
        for (int pc = tid; pc < kTileRows * XC; pc += kThreads) {
            const int qq = pc / XC, c = pc % XC;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qq < rows && c * 8 < kn) {
                const int m = seg.perm[p0 + qq];
                v = ld16(x + (size_t)m * d_in + k0 + c * 8);
            }
            Xs[qq][c] = v;
        }
        __syncthreads();

        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        if (q < rows && g * 8 < r) {
            const uint4 *arow = &As[(ksub * KCS + ksub) * JG + g];
            const uint4 *xrow = &Xs[q][ksub * (KCS / 8)];
#pragma unroll 2
            for (int kk = 0; kk < KCS; kk += 8) {
                float xv[8];
                unpack8(xrow[kk / 8], xv);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    float av[8];
                    unpack8(arow[(kk + u) * JG], av);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[j] = fmaf(xv[u], av[j], acc[j]);
                }
            }
        }
#pragma unroll
        for (int off = 1; off < KSUB; off <<= 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += __shfl_xor(acc[j], off, 64);
        }
        if (ksub == 0 && q < rows) {
            const int m = seg.perm[p0 + q];
            float *dst = partial + ((size_t)kcx * M + m) * RM + g * 8;
            *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
        __syncthreads();  // LDS is refilled by the next work item
    }
}

// t[m, :] = sum over chunks (ascending) of partial[chunk][m][:] for LoRA rows; 0 for
// base-only rows.  One thread per 4 columns of one position of perm.
__global__ __launch_bounds__(256) void shrink_finalize_kernel(const float *__restrict__ partial,
                                                              int M, int RM, int ksplit, Seg seg,
                                                              float *__restrict__ t) {
    const int per_row = RM / 4;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)M * per_row) return;
    const int p = (int)(idx / per_row), j = (int)(idx % per_row) * 4;
    const int m = seg.perm[p];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p < seg.meta[1]) {
        for (int c = 0; c < ksplit; ++c) {
            const float4 v = *reinterpret_cast<const float4 *>(partial + ((size_t)c * M + m) * RM + j);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
    }
    *reinterpret_cast<float4 *>(t + (size_t)m * RM + j) = acc;
}

constexpr int kMaxGrid = 1 << 20;

}  // namespace

void shrink_plan(int d_in, int *kc, int *ksplit) {
    *kc = kKC;
    *ksplit = (d_in + kKC - 1) / kKC;
}

hipError_t launch_shrink(const uint16_t *x, const uint16_t *A, const int32_t *ranks, int M,
                         int d_in, int r_max, int n_adapters, Seg seg, float *partial, int kc,
                         int ksplit, hipStream_t s) {
    (void)kc;
    const long items = (long)lora_max_tiles(M, n_adapters) * ksplit;
    const int grid = (int)(items < kMaxGrid ? items : kMaxGrid);
    switch (r_max) {
        case 8:
            launch(shrink_kernel<8>, dim3(grid), dim3(kThreads), 0, s, x, A, ranks, M, d_in, seg, partial, ksplit);
            break;
        case 16:
            launch(shrink_kernel<16>, dim3(grid), dim3(kThreads), 0, s, x, A, ranks, M, d_in, seg, partial, ksplit);
            break;
        case 32:
            launch(shrink_kernel<32>, dim3(grid), dim3(kThreads), 0, s, x, A, ranks, M, d_in, seg, partial, ksplit);
            break;
        case 64:
            launch(shrink_kernel<64>, dim3(grid), dim3(kThreads), 0, s, x, A, ranks, M, d_in, seg, partial, ksplit);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_shrink_finalize(const float *partial, int M, int r_max, int ksplit, Seg seg,
                                  float *t, hipStream_t s) {
    const long threads = (long)M * (r_max / 4);
    const int grid = (int)((threads + 255) / 256);
    launch(shrink_finalize_kernel, dim3(grid), dim3(256), 0, s, partial, M, r_max,
                       ksplit, seg, t);
    return hipGetLastError();
}

}  // namespace lora

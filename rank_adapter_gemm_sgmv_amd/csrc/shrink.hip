// shrink.hip -- t = x A_i per row, for all adapters of a mixed batch in one launch.
//
// Source: the adapter "shrink" step of "Multi-LoRA Serving: Sharing One GPU Across
// Adapters" (cloudai.pt), section "MoE Models Raise the Bar", which also names split-K for
// these skinny products; the [B, 4096] x [4096, r] product of "Multi-LoRA Serving: Why 100
// Adapters Fit on One GPU" (dev.to), "How does one batch run 30 different adapters at
// once?", memory-bound on the adapter weights.
//
// Work item = (tile, k-chunk): a tile is up to LORA_TILE_ROWS rows of one adapter a (from
// the segment builder), a k-chunk is KC consecutive rows of A_a (one contiguous block of the
// padded pool; only the 8-column groups below the adapter's rank are fetched).  Each A_a
// byte is read from HBM once per tile.  Two kernels, chosen by r_max:
//
//  * r_max <= 16, shrink_lds_kernel: a 256-thread workgroup stages the A chunk (8 KB at
//    most) and the tile's x rows in LDS; thread = (row q, column group g, k-slice ks)
//    accumulates 8 fp32 sums over its k-slice, then the k-slices of one (q, g) -- adjacent
//    lanes -- are added by an xor butterfly.  Tiles of one adapter share the chunk through
//    L2: their block ids differ by a multiple of the k-split, hence of 8, so they land on
//    the same XCD.
//  * r_max >= 32, shrink_reg_kernel: the chunk would be 16-32 KB of LDS per workgroup, so a
//    wave instead holds A_a[chunk, 0:rank] in registers -- lane = (k-slice, 8 rank columns)
//    -- and streams the tile's rows of x past it, four rows' loads in flight at a time,
//    each A element unpacked once per batch of rows; then the same xor butterfly.
//
// The partial sums of each k-chunk go to partial[chunk][row][0:r_max] (zero beyond the
// rank); shrink_finalize_kernel adds the chunks in ascending order, so the result does not
// depend on scheduling.
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 256;      // shrink_lds_kernel
constexpr int kKC = 256;           // k rows of A per work item in shrink_lds_kernel
constexpr int kWavesPerBlock = 4;  // shrink_reg_kernel
constexpr int kMaxGrid = 1 << 20;

template <int RM>
__global__ __launch_bounds__(kThreads) void shrink_lds_kernel(const uint16_t *__restrict__ x,
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

template <int RM>
struct ShrinkLanes {
    static constexpr int KC = RM == 64 ? 128 : 256;  // k per chunk
    static constexpr int JG = RM / 8;                // 8-column groups
    static constexpr int KSUB = 64 / JG;             // k-slices across a wave
    static constexpr int SL = KC / KSUB;             // k per lane: 16 for r_max 32 and 64
    static constexpr int XV = SL >= 8 ? SL / 8 : 1;  // 16-byte x loads per row
    static constexpr int RB = 4;                     // rows whose x loads are in flight together
};

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int q) {
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

template <int RM>
__global__ __launch_bounds__(64 * kWavesPerBlock) void shrink_reg_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ A, const int32_t *__restrict__ ranks,
    int M, int d_in, Seg seg, float *__restrict__ partial, int n_chunks) {
    using L = ShrinkLanes<RM>;
    const int lane = threadIdx.x & 63;
    const int ks = lane % L::KSUB, g = lane / L::KSUB;
    const int total = seg.meta[3] * n_chunks;
    const int nw = gridDim.x * kWavesPerBlock;
    for (int w = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6); w < total; w += nw) {
        const int tile = w / n_chunks, c = w % n_chunks;
        const int p0 = seg.tiles[2 * tile], a = seg.tiles[2 * tile + 1];
        const int p1 = min(p0 + kTileRows, seg.offsets[a + 1]);
        const int r = ranks ? min(max(ranks[a], 0), RM) : RM;
        const int k0 = c * L::KC + ks * L::SL;
        const bool colok = g * 8 < r;

        // A_a[k0 .. k0+SL][8g .. 8g+7]: only column groups below the rank are read
        uint4 araw[L::SL];
        const uint16_t *Ap = A + ((size_t)a * d_in + k0) * RM + g * 8;
#pragma unroll
        for (int kk = 0; kk < L::SL; ++kk)
            araw[kk] = (colok && k0 + kk < d_in) ? ld16(Ap + (size_t)kk * RM) : make_uint4(0, 0, 0, 0);

        // x[row][k0 ..] of the row at perm position p (clamped in bounds)
        auto load_x = [&](int p, uint4 (&xv)[L::XV]) {
            const int m = seg.perm[min(p, M - 1)];
            const uint16_t *xr = x + (size_t)m * d_in;
            if constexpr (L::SL >= 8) {
#pragma unroll
                for (int v = 0; v < L::XV; ++v) xv[v] = ld16(xr + min(k0 + 8 * v, d_in - 8));
            } else {
                const uint2 h = *reinterpret_cast<const uint2 *>(xr + min(k0, d_in - 4));
                xv[0] = make_uint4(h.x, h.y, 0, 0);
            }
        };
        // rows in batches of RB: all of a batch's x loads are in flight together; each A
        // element is unpacked once per batch and used by every row of it
        for (int pb = p0; pb < p1; pb += L::RB) {
            uint4 xb[L::RB][L::XV];
#pragma unroll
            for (int i = 0; i < L::RB; ++i) load_x(pb + i, xb[i]);
            float acc[L::RB][8];
#pragma unroll
            for (int i = 0; i < L::RB; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
#pragma unroll
            for (int kk = 0; kk < L::SL; ++kk) {
                if (k0 + kk < d_in) {
                    float av[8];
                    unpack8(araw[kk], av);
#pragma unroll
                    for (int i = 0; i < L::RB; ++i) {
                        const uint32_t w = word_of(xb[i][kk / 8], (kk % 8) / 2);
                        const float xf = (kk & 1) ? bf16_hi(w) : bf16_lo(w);
#pragma unroll
                        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(xf, av[j], acc[i][j]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < L::RB; ++i) {
#pragma unroll
                for (int off = 1; off < L::KSUB; off <<= 1) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[i][j] += __shfl_xor(acc[i][j], off, 64);
                }
            }
            if (ks == 0) {
#pragma unroll
                for (int i = 0; i < L::RB; ++i) {
                    if (pb + i < p1) {
                        const int m = seg.perm[pb + i];
                        float *dst = partial + ((size_t)c * M + m) * RM + g * 8;
                        *reinterpret_cast<float4 *>(dst) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
                        *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
                    }
                }
            }
        }
    }
}

// t[m, :] = sum over chunks (ascending) of partial[chunk][m][:] for LoRA rows; 0 for
// base-only rows.  One thread per 4 columns of one position of perm; eight chunk loads are
// in flight at a time and added in chunk order.
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
    *reinterpret_cast<float4 *>(t + (size_t)m * RM + j) = acc;
}

}  // namespace

void shrink_plan(int d_in, int r_max, int *kc, int *ksplit) {
    *kc = r_max == 64 ? 128 : kKC;
    *ksplit = (d_in + *kc - 1) / *kc;
}

hipError_t launch_shrink(const uint16_t *x, const uint16_t *A, const int32_t *ranks, int M,
                         int d_in, int r_max, int n_adapters, Seg seg, float *partial, int kc,
                         int ksplit, hipStream_t s) {
    (void)kc;
    const long items = (long)lora_max_tiles(M, n_adapters) * ksplit;
    const dim3 lgrid((unsigned)(items < kMaxGrid ? items : kMaxGrid));
    const long rblocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    const dim3 rgrid((unsigned)(rblocks < kMaxGrid ? rblocks : kMaxGrid));
    const dim3 rblock(64 * kWavesPerBlock);
    switch (r_max) {
        case 8: launch(shrink_lds_kernel<8>, lgrid, dim3(kThreads), 0, s, x, A, ranks, M, d_in, seg, partial, ksplit); break;
        case 16: launch(shrink_lds_kernel<16>, lgrid, dim3(kThreads), 0, s, x, A, ranks, M, d_in, seg, partial, ksplit); break;
        case 32: launch(shrink_reg_kernel<32>, rgrid, rblock, 0, s, x, A, ranks, M, d_in, seg, partial, ksplit); break;
        case 64: launch(shrink_reg_kernel<64>, rgrid, rblock, 0, s, x, A, ranks, M, d_in, seg, partial, ksplit); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_shrink_finalize(const float *partial, int M, int r_max, int ksplit, Seg seg,
                                  float *t, hipStream_t s) {
    const long threads = (long)M * (r_max / 4);
    const int grid = (int)((threads + 255) / 256);
    launch(shrink_finalize_kernel, dim3(grid), dim3(256), 0, s, partial, M, r_max, ksplit, seg, t);
    return hipGetLastError();
}

}  // namespace lora

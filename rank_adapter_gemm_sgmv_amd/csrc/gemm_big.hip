// gemm_big.hip -- the shared term y = x W on bf16 MFMA for large batches (prefill and the
// wide decode batches), with the LoRA delta of each adapter run fused into the epilogue.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Why can't you
// just merge LoRA weights into the base model?" (x W is one big GEMM across the whole batch)
// and "How does one batch run 30 different adapters at once?" (prefill is compute-bound; the
// delta is small next to x W).
//
// gfx950 design
//  * Tile BM x BN (256 x 256, 256 x 128 or 128 x 128).  256 x 256 tiles use eight waves in a
//    2 x 4 grid (each owns 128 x 64 of the output: 128 accumulator registers, so two waves
//    share a SIMD and one issues MFMAs while the other waits on LDS or the barrier); the
//    smaller tiles use four waves in a 2 x 2 grid.  Accumulators are 32 x 32
//    v_mfma_f32_32x32x16_bf16 blocks.
//  * K is consumed 32 at a time through a 4-stage LDS ring filled by direct global->LDS
//    loads (global_load_lds_dwordx4): no staging registers, three stages in flight while one
//    is multiplied.  Each stage slot is its own __shared__ array, named statically and
//    reached through __restrict__ parameters, so the compiler can tell the in-flight loads
//    from the slot being read and only the explicit s_waitcnt below orders them.
//  * x tile: [BM rows][32 k] (64-byte rows).  A operand = one ds_read_b128 per lane
//    (8 consecutive k of one row).  The 16-byte chunk c of row r is stored at c ^ ((r/4) % 4),
//    so the 32 rows a wave reads at once spread over all LDS banks.
//  * W tile: [32 k][BN n], exactly as W is laid out in HBM (n contiguous), so its loads are
//    plain row copies.  The B operand needs 8 consecutive k of one column per lane; gfx950's
//    transposing LDS read (ds_read_b64_tr_b16) delivers 4 of them per instruction: inside a
//    group of 16 lanes, lane i names 8 bytes (4 columns) of row i/4, and lane j receives
//    column j of the 4 x 16 block.  Chunk c of row r is stored at c ^ (4 (r % 4)), so the
//    four rows of one read hit distinct banks.
//  * Prefill rows are taken in segment order (positions of perm), so a tile holds a few long
//    runs of one adapter.  After the K loop, every run adds s_a * t[rows, :] B_a[:, cols]
//    as extra 32-deep MFMA steps (the K-extension [x | s t] [W ; B_a]) before the only store.
//  * Tiles are handed to XCDs in compact blocks (workgroup b runs on XCD b % 8), so the
//    x and W panels a tile group shares are read once into that XCD's L2.
#include <type_traits>

#include "common.h"

namespace lora {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kBK = 32;     // k per stage

// Tile BM x BN computed by WM x WN waves, each owning (BM / WM) x (BN / WN).
template <int BM_, int BN_, int WM_ = 2, int WN_ = 2>
struct Big {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN, NT = 64 * NW;  // waves, threads
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // per-wave tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int XSLOT = BM * kBK * 2 / 16;  // uint4 per x slot
    static constexpr int WSLOT = kBK * BN * 2 / 16;  // uint4 per W slot
    static constexpr int XINS = XSLOT / 64 / NW;     // DMA instructions per wave per stage
    static constexpr int WINS = WSLOT / 64 / NW;
    static constexpr int PER = XINS + WINS;
    static constexpr int WROWS = 1024 / (BN * 2);     // W rows per DMA instruction
    static constexpr int WCH = BN / 8;                // 16-byte chunks per W row
    static_assert(BN == 128 || BN == 256, "W swizzle needs at least 16 chunks per row");
    static_assert(BM == 128 || BM == 256, "x tile");
    static_assert(XINS >= 1 && WINS >= 1, "per-wave DMA split");
    static_assert(XINS * 64 * NW == XSLOT && WINS * 64 * NW == WSLOT, "whole DMA instructions");
    static_assert(NW == 4 || NW == 8, "four or eight waves (staging slots)");
    static_assert(TM >= 1 && TN >= 1, "per-wave tile of whole 32 x 32 blocks");
};

// s_waitcnt with only vmcnt = n (n < 64); expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that orders LDS accesses in the compiler but adds no vmcnt wait.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads have returned
    asm volatile("s_barrier" ::: "memory");
}

// ---- operand fragments of one 32-deep step ------------------------------------------------
// a[kk][i]: rows wm0 + 32 i + lane % 32, k = 16 kk + 8 (lane / 32) .. +7 (one ds_read_b128);
// b[kk][j]: column wn0 + 32 j + lane % 32, the same 8 k (two ds_read_b64_tr_b16).
template <class C>
struct Frags {
    bf16x8_t a[2][C::TM];
    bf16x8_t b[2][C::TN];
};

template <class C>
__device__ __forceinline__ void read_frags(Frags<C> &f, const uint4 *__restrict__ xs,
                                           const uint4 *__restrict__ ws, int lane, int wm0,
                                           int wn0) {
    const lds_char_t *wsb = (const lds_char_t *)(ws);
    const int g = lane >> 4, li = lane & 15;
    const int rsw = (li >> 2) << 2;  // (row % 4) * 4 for every W row this lane names
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int row = wm0 + 32 * i + (lane & 31);
            const int lc = 2 * kk + (lane >> 5);
            f.a[kk][i] = *reinterpret_cast<const bf16x8_t *>(&xs[row * 4 + (lc ^ ((row >> 2) & 3))]);
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = wn0 + 32 * j + 16 * (g & 1) + 4 * (li & 3);
            const int lc = col >> 3, half = (col >> 2) & 1;
            const int r = 16 * kk + 8 * (g >> 1) + (li >> 2);
            const lds_char_t *p = wsb + r * (C::BN * 2) + ((lc ^ rsw) << 4) + half * 8;
            const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)p);
            const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(p + 4 * C::BN * 2));
            f.b[kk][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
}

template <class C>
__device__ __forceinline__ void mfma_frags(f32x16_t (&acc)[C::TM][C::TN], const Frags<C> &f) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j], acc[i][j], 0, 0, 0);
}

// One 32-deep step straight from LDS (used outside the pipelined loop).
template <class C>
__device__ __forceinline__ void mfma_stage(f32x16_t (&acc)[C::TM][C::TN],
                                           const uint4 *__restrict__ xs,
                                           const uint4 *__restrict__ ws, int lane, int wm0, int wn0) {
    Frags<C> f;
    read_frags<C>(f, xs, ws, lane, wm0, wn0);
    mfma_frags<C>(acc, f);
}

// Interleave the LDS reads of the next step's fragments with this step's MFMAs: groups of
// DS reads, then MFMAs, in order (one scheduling group sequence).
template <class C>
__device__ __forceinline__ void interleave_reads_with_mfma() {
    constexpr int reads = 2 * (C::TM + 2 * C::TN);
    constexpr int mfmas = 2 * C::TM * C::TN;
    constexpr int groups = 8;
    constexpr int rpg = (reads + groups - 1) / groups;
    constexpr int mpg = mfmas / groups;
#pragma unroll
    for (int gi = 0; gi < groups; ++gi) {
        __builtin_amdgcn_sched_group_barrier(0x100, rpg, 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, mpg, 0);  // MFMA
    }
}

// ---- per-lane DMA sources ----------------------------------------------------------------
// x: instruction q covers tile rows 16q .. 16q+15; lane i fills row 16q + i/4, stored chunk
// i % 4, which holds logical chunk (i % 4) ^ ((i / 16) % 4).
// W: instruction q covers tile rows WROWS q ..; lane i fills row WROWS q + i / WCH, stored
// chunk i % WCH, holding logical chunk (i % WCH) ^ (4 (row % 4)).
template <class C>
struct DmaSrc {
    const uint16_t *xp[C::XINS];  // row start + logical chunk offset, k = 0
    const uint16_t *wp[C::WINS];  // (row, logical chunk) at k = 0
};

template <class C>
__device__ __forceinline__ void issue_stage(const DmaSrc<C> &src, uint4 *__restrict__ xslot,
                                            uint4 *__restrict__ wslot,
                                            int wave, int k0, int N) {
#pragma unroll
    for (int j = 0; j < C::XINS; ++j) {
        const int q = wave * C::XINS + j;
        __builtin_amdgcn_global_load_lds((const void *)(src.xp[j] + k0), (lds_void_t *)&xslot[q * 64], 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::WINS; ++j) {
        const int q = wave * C::WINS + j;
        __builtin_amdgcn_global_load_lds((const void *)(src.wp[j] + (size_t)k0 * N), (lds_void_t *)&wslot[q * 64], 16, 0, 0);
    }
}

// The same sources as 32-bit byte offsets from x and W (the prefill instances, when both
// tensors fit in 4 GiB): the direct load's scalar-base form then takes one VGPR per address
// instead of two, which frees the two registers the LoRA epilogue's kernel otherwise kept in
// scratch memory across the K loop (prefill GEMM 118.1 -> 116.5 us).
template <class C>
struct DmaSrc32 {
    const char *xb, *wb;
    uint32_t xo[C::XINS];
    uint32_t wo[C::WINS];
};

template <class C>
__device__ __forceinline__ void issue_stage(const DmaSrc32<C> &src, uint4 *__restrict__ xslot,
                                            uint4 *__restrict__ wslot,
                                            int wave, int k0, int N) {
#pragma unroll
    for (int j = 0; j < C::XINS; ++j) {
        const int q = wave * C::XINS + j;
        __builtin_amdgcn_global_load_lds((const void *)(src.xb + (uint32_t)(src.xo[j] + 2u * (uint32_t)k0)),
                                         (lds_void_t *)&xslot[q * 64], 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::WINS; ++j) {
        const int q = wave * C::WINS + j;
        __builtin_amdgcn_global_load_lds(
            (const void *)(src.wb + (uint32_t)(src.wo[j] + 2u * (uint32_t)k0 * (uint32_t)N)),
            (lds_void_t *)&wslot[q * 64], 16, 0, 0);
    }
}

// Tile order: XCD-major (workgroup b runs on XCD b % 8), then groups of 4 tile rows, column-
// major inside a group, so each XCD works on a compact block of tiles.
__device__ __forceinline__ void tile_of(int b, int n_tm, int n_tn, int &tm, int &tn) {
    const int T = n_tm * n_tn;
    int lin = b;
    if ((T % 8) == 0) lin = (b % 8) * (T / 8) + b / 8;
    constexpr int G = 4;
    const int group = lin / (G * n_tn);
    const int first = group * G;
    const int gsz = min(n_tm - first, G);
    const int in = lin % (G * n_tn);
    tm = first + in % gsz;
    tn = in / gsz;
}

// Register-path fill of slot 0 with K step k0 .. k0+31 (zero beyond K), for the steps the
// DMA ring does not cover.
template <class C, bool SEGROWS>
__device__ __forceinline__ void fill_stage(uint4 *xs, uint4 *ws, const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ W, int M, int K, int N,
                                          int row0, int n0, int k0, const int32_t *perm, int tid) {
    for (int c = tid; c < C::BM * 4; c += C::NT) {
        const int row = c >> 2, lc = c & 3;
        const int rr = row0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        const int k = k0 + lc * 8;
        if (rr < M && k < K) {
            const int m = SEGROWS ? perm[rr] : rr;
            v = ld16(x + (size_t)m * K + k);
        }
        xs[row * 4 + (lc ^ ((row >> 2) & 3))] = v;
    }
    for (int c = tid; c < kBK * C::WCH; c += C::NT) {
        const int r = c / C::WCH, lc = c % C::WCH;
        const int n = n0 + lc * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k0 + r < K && n < N) v = ld16(W + (size_t)(k0 + r) * N + n);
        ws[r * C::WCH + (lc ^ ((r & 3) << 2))] = v;
    }
}

// O32: DMA sources as 32-bit byte offsets (x and W each below 4 GiB).
template <class C, bool SEGROWS, bool LORA, bool YF32, bool O32>
__global__ __launch_bounds__(C::NT) void gemm_big_kernel(const uint16_t *__restrict__ x,
                                                            const uint16_t *__restrict__ W,
                                                            int M, int K, int N,
                                                            void *__restrict__ y, int n_tm,
                                                            int n_tn, Seg seg, LoraEpilogue ep) {
    __shared__ __attribute__((aligned(1024))) uint4 X0[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 X1[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 X2[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 X3[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W0[C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W1[C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W2[C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W3[C::WSLOT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::WTM, wn0 = (wave % C::WN) * C::WTN;
    int tmi, tni;
    tile_of(blockIdx.x, n_tm, n_tn, tmi, tni);
    const int row0 = tmi * C::BM, n0 = tni * C::BN;

    // DMA sources of this lane (rows beyond M and columns beyond N are clamped in bounds;
    // their results are never stored)
    std::conditional_t<O32, DmaSrc32<C>, DmaSrc<C>> src;
    if constexpr (O32) {
        src.xb = reinterpret_cast<const char *>(x);
        src.wb = reinterpret_cast<const char *>(W);
    }
#pragma unroll
    for (int j = 0; j < C::XINS; ++j) {
        const int q = wave * C::XINS + j;
        const int row = 16 * q + (lane >> 2);
        const int lc = (lane & 3) ^ ((lane >> 4) & 3);
        const int rr = min(row0 + row, M - 1);
        const int m = SEGROWS ? seg.perm[rr] : rr;
        if constexpr (O32) src.xo[j] = (uint32_t)(((size_t)m * K + lc * 8) * 2);
        else src.xp[j] = x + (size_t)m * K + lc * 8;
    }
#pragma unroll
    for (int j = 0; j < C::WINS; ++j) {
        const int q = wave * C::WINS + j;
        const int r = C::WROWS * q + lane / C::WCH;
        const int lc = (lane % C::WCH) ^ ((r & 3) << 2);
        const int n = min(n0 + lc * 8, N - 8);
        if constexpr (O32) src.wo[j] = (uint32_t)(((size_t)r * N + n) * 2);
        else src.wp[j] = W + (size_t)r * N + n;
    }

    f32x16_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // K steps 0 .. nmain-1 go through the DMA ring, four per loop trip.  Every trip issues
    // its loads unconditionally (stages past the last real one reload the last real stage
    // into slots that are never multiplied), so the outstanding-load count is the same on
    // every path and the explicit waits are exact.
    const int nfull = K / kBK;
    const int nmain = nfull & ~3;
    if (nmain > 0) {
        // Prologue: stages 0..2 in flight, stage 0's fragments in registers, stage 3 issued.
        // In loop trip s the fragments of stage s are multiplied while those of stage s+1 are
        // read from LDS and stage s+4 is loaded into the slot stage s occupied.
        Frags<C> fa, fb;
        issue_stage<C>(src, X0, W0, wave, 0, N);
        issue_stage<C>(src, X1, W1, wave, min(1, nmain - 1) * kBK, N);
        issue_stage<C>(src, X2, W2, wave, min(2, nmain - 1) * kBK, N);
        wait_vm<2 * C::PER>();
        lds_barrier();
        read_frags<C>(fa, X0, W0, lane, wm0, wn0);
        issue_stage<C>(src, X3, W3, wave, min(3, nmain - 1) * kBK, N);
#define LORA_BIG_STEP(SS, FC, FN, XN, WN, XF, WF)                                 \
        wait_vm<2 * C::PER>();                                                   \
        lds_barrier();                                                           \
        issue_stage<C>(src, XF, WF, wave, min((SS) + 4, nmain - 1) * kBK, N);    \
        read_frags<C>(FN, XN, WN, lane, wm0, wn0);                               \
        mfma_frags<C>(acc, FC);                                                  \
        interleave_reads_with_mfma<C>();
        for (int s = 0; s < nmain; s += 4) {
            LORA_BIG_STEP(s, fa, fb, X1, W1, X0, W0)
            LORA_BIG_STEP(s + 1, fb, fa, X2, W2, X1, W1)
            LORA_BIG_STEP(s + 2, fa, fb, X3, W3, X2, W2)
            LORA_BIG_STEP(s + 3, fb, fa, X0, W0, X3, W3)
        }
#undef LORA_BIG_STEP
        wait_vm<0>();
    }
    // remaining steps (K not a multiple of 128), the last one possibly partial: through
    // registers into slot 0, zero beyond K
    for (int k0 = nmain * kBK; k0 < K; k0 += kBK) {
        lds_barrier();
        fill_stage<C, SEGROWS>(X0, W0, x, W, M, K, N, row0, n0, k0, seg.perm, tid);
        __syncthreads();
        mfma_stage<C>(acc, X0, W0, lane, wm0, wn0);
    }

    if constexpr (LORA) {
        // Runs of one adapter among this tile's rows (positions of perm): for each run, 16
        // rank columns at a time, stage T = scale_a * t[rows, :] (zero outside the run) in
        // slot 0's x layout as a pair of bf16 values per element -- k slots 0..15 the value
        // rounded to bf16, slots 16..31 the remainder (exact in fp32) rounded to bf16 -- and
        // B_a's same 16 rank rows twice in its W layout (zero beyond the rank), then one more
        // MFMA step.  The pair carries scale * t to about 16 significant bits, so the delta is
        // not rounded to bf16 precision before it is added.
        const int n_lora = seg.meta[1];
        const int RM = ep.r_max;
        constexpr int kHalf = kBK / 2;
        int p = row0;
        const int p_end = min(row0 + C::BM, n_lora);
        while (p < p_end) {
            const int a = ep.ids[seg.perm[p]];
            if (a < 0 || a >= ep.n_adapters) break;  // segments not built for these ids
            const int q_end = min(seg.offsets[a + 1], p_end);
            if (q_end <= p) break;
            const float s = ep.scale[a];
            // B_a's rank rows: all of a padded pool's stride (zero past the rank), the
            // rank's in a compact one
            int ra = ep.roff ? min(max(ep.ranks[a], 0), RM) : ep.pstride;
            const int brow0 = adapter_row0(ep.roff, ep.pool_rows, a, ep.pstride, ra);
            for (int rc = 0; rc < RM; rc += kHalf) {
                lds_barrier();
                for (int c = tid; c < C::BM * 4; c += C::NT) {
                    const int row = c >> 2, lc = c & 3;
                    const int pos = row0 + row;
                    const int j = rc + (lc & 1) * 8;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (pos >= p && pos < q_end && j < RM) {
                        // t[m, j .. j+7]: the shrink's chunk sums added in chunk order, four
                        // chunks' loads in flight at a time
                        const float *tp = ep.tpart + (size_t)seg.perm[pos] * RM + j;
                        const size_t cs = (size_t)M * RM;
                        float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                        for (int c0 = 0; c0 < ep.n_chunks; c0 += 4) {
                            float4 v[4][2];
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const bool in = c0 + c < ep.n_chunks;
                                const float *q = tp + (size_t)(in ? c0 + c : 0) * cs;
                                v[c][0] = in ? *reinterpret_cast<const float4 *>(q) : make_float4(0.f, 0.f, 0.f, 0.f);
                                v[c][1] = in ? *reinterpret_cast<const float4 *>(q + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
                            }
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                if (c0 + c < ep.n_chunks) {
                                    t[0] += v[c][0].x; t[1] += v[c][0].y; t[2] += v[c][0].z; t[3] += v[c][0].w;
                                    t[4] += v[c][1].x; t[5] += v[c][1].y; t[6] += v[c][1].z; t[7] += v[c][1].w;
                                }
                            }
                        }
                        float f[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) f[e] = s * t[e];
                        if (lc >= 2) {  // the remainder after rounding to bf16
#pragma unroll
                            for (int e = 0; e < 8; ++e) f[e] -= __uint_as_float(f32_to_bf16_rne(f[e]) << 16);
                        }
                        v = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                       pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
                    }
                    X0[row * 4 + (lc ^ ((row >> 2) & 3))] = v;
                }
                for (int c = tid; c < kBK * C::WCH; c += C::NT) {
                    const int r = c / C::WCH, lc = c % C::WCH;
                    const int rank = rc + (r & (kHalf - 1));
                    const int n = n0 + lc * 8;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (rank < ra && n < N) v = ld16(ep.B + ((size_t)brow0 + rank) * N + n);
                    W0[r * C::WCH + (lc ^ ((r & 3) << 2))] = v;
                }
                __syncthreads();
                mfma_stage<C>(acc, X0, W0, lane, wm0, wn0);
            }
            p = q_end;
        }
    }

    // store: accumulator element v of a 32 x 32 block is row (v/4)*8 + (lane/32)*4 + v%4,
    // column lane%32.
    if constexpr (YF32) {
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rr = row0 + wm0 + 32 * i + (v / 4) * 8 + (lane >> 5) * 4 + (v % 4);
                if (rr >= M) continue;
                const int m = SEGROWS ? seg.perm[rr] : rr;
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int col = n0 + wn0 + 32 * j + (lane & 31);
                    if (col < N) reinterpret_cast<float *>(y)[(size_t)m * N + col] = acc[i][j][v];
                }
            }
        }
    } else {
        // bf16 y: each wave stages 32 rows of its tile at a time in its own LDS slot, then
        // writes whole 16-byte pieces of rows (a wave covers several full row segments per
        // store instruction).  LDS accesses of one wave complete in order, so the staging
        // needs no barrier beyond the one that frees the slots.
        lds_barrier();
        // wave w stages in slot w of X0 .. X3, W0 .. W3
        uint4 *const sl = wave == 0 ? X0 : wave == 1 ? X1 : wave == 2 ? X2 : wave == 3 ? X3
                        : wave == 4 ? W0 : wave == 5 ? W1 : wave == 6 ? W2 : W3;
        uint16_t *stg = reinterpret_cast<uint16_t *>(sl);
        constexpr int SROW = C::WTN + 8;  // staged row length (bf16), 16-byte pad
        constexpr int CPR = C::WTN / 8;   // 16-byte pieces per staged row
        static_assert(32 * SROW * 2 <= C::XSLOT * 16 && 32 * SROW * 2 <= C::WSLOT * 16,
                      "staging fits one slot");
        uint16_t *yb = reinterpret_cast<uint16_t *>(y);
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = (v / 4) * 8 + (lane >> 5) * 4 + (v % 4);
                    stg[r * SROW + 32 * j + (lane & 31)] = (uint16_t)f32_to_bf16_rne(acc[i][j][v]);
                }
#pragma unroll
            for (int c = lane; c < 32 * CPR; c += 64) {
                const int r = c / CPR, cc = c % CPR;
                const int rr = row0 + wm0 + 32 * i + r;
                const int col = n0 + wn0 + 8 * cc;
                const uint4 val = *reinterpret_cast<const uint4 *>(&stg[r * SROW + 8 * cc]);
                if (rr < M && col < N) {
                    const int m = SEGROWS ? seg.perm[rr] : rr;
                    st16(yb + (size_t)m * N + col, val);
                }
            }
        }
    }
}

// ---- stream-K decode GEMM -----------------------------------------------------------------
// Decode batches of a few hundred rows have too few 256 x 256 output tiles to fill the chip
// (512 x 11008: 86 tiles on 256 CUs), and smaller tiles lose the large tile's MFMA rate.
// Instead the K steps of all column panels, laid end to end panel after panel (projection
// after projection when several that share x run in one launch), are cut into L equal lanes.
// Each lane is run by n_tm workgroups, one per 256-row tile, placed on the same XCD
// (workgroup b runs on XCD b % 8), so the W panel they share is read once into that XCD's L2.
// A lane's range may start inside one panel and end inside the next: for every panel it
// meets, the lane writes its fp32 partial tile to slot (lane + panel) * n_tm + tm. lane +
// panel differs for every (lane, panel) pair that meets, because panels and lanes both
// advance along the one K line. sk_reduce_lora_kernel adds a panel's slots in lane order,
// so the sum does not depend on scheduling.

// Lane run by the workgroups of each rank: lanes sorted by the K offset at which they
// start inside their panel, so the ranks an XCD gets (16 when L = 128) read neighbouring
// K slices of x and share them through that XCD's L2.
struct SkLanes {
    uint8_t lane[256];
};

// First K step (of the panel-major line of `total` steps) of lane l out of L.  Lanes start
// on multiples of 4 steps and K is a multiple of 4 steps (128), so every (lane, panel) piece
// is a whole number of trips of the 4-stage ring.
__device__ __forceinline__ int sk_start(int l, int total, int L) {
    return 4 * (int)(((long)l * (total / 4)) / L);
}

template <class C>
__global__ __launch_bounds__(C::NT) void gemm_sk_kernel(const uint16_t *__restrict__ x,
                                                        SkProj pj, int M, int K, int N,
                                                        float *__restrict__ partial, int n_tm,
                                                        int n_tn, int n_tn1, int L, SkLanes lanes) {
    __shared__ __attribute__((aligned(1024))) uint4 X0[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 X1[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 X2[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 X3[C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W0[C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W1[C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W2[C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 W3[C::WSLOT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::WTM, wn0 = (wave % C::WN) * C::WTN;
    // workgroup b runs on XCD b % 8; its n_tm row tiles of one lane are consecutive there
    const int b = blockIdx.x;
    const int i = b >> 3;
    const int tm = i % n_tm;
    const int ln = lanes.lane[(b & 7) * (L >> 3) + i / n_tm];
    const int KI = K / kBK;
    const int total = n_tn * KI;
    const int s0 = sk_start(ln, total, L), s1 = sk_start(ln + 1, total, L);
    const int row0 = tm * C::BM;

    DmaSrc<C> src;
#pragma unroll
    for (int j = 0; j < C::XINS; ++j) {
        const int q = wave * C::XINS + j;
        const int row = 16 * q + (lane >> 2);
        const int lc = (lane & 3) ^ ((lane >> 4) & 3);
        src.xp[j] = x + (size_t)min(row0 + row, M - 1) * K + lc * 8;
    }

    for (int p = s0 / KI; p * KI < s1; ++p) {
        const int kb = max(s0, p * KI) - p * KI;
        const int n = min(s1, (p + 1) * KI) - p * KI - kb;  // steps of this panel, 4 | n
        // panel p is panel pl of projection pr
        const int pr = p / n_tn1, pl = p - pr * n_tn1;
        const uint16_t *__restrict__ W = pick_proj(pr, pj.W);
        const int n0 = pl * C::BN;
#pragma unroll
        for (int j = 0; j < C::WINS; ++j) {
            const int q = wave * C::WINS + j;
            const int r = C::WROWS * q + lane / C::WCH;
            const int lc = (lane % C::WCH) ^ ((r & 3) << 2);
            src.wp[j] = W + (size_t)r * N + min(n0 + lc * 8, N - 8);
        }
        f32x16_t acc[C::TM][C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // every wave is done reading the previous panel's slots before they are refilled
        lds_barrier();
        // The ring of the large kernel over steps kb .. kb+n-1; loads past the last step
        // reload the last step (in bounds, never multiplied), so every step issues one stage
        // and the waits stay exact.
        const int last = kb + n - 1;
        Frags<C> fa, fb;
        issue_stage<C>(src, X0, W0, wave, kb * kBK, N);
        issue_stage<C>(src, X1, W1, wave, min(kb + 1, last) * kBK, N);
        issue_stage<C>(src, X2, W2, wave, min(kb + 2, last) * kBK, N);
        wait_vm<2 * C::PER>();
        lds_barrier();
        read_frags<C>(fa, X0, W0, lane, wm0, wn0);
        issue_stage<C>(src, X3, W3, wave, min(kb + 3, last) * kBK, N);
#define LORA_SK_STEP(SS, FC, FN, XN, WN, XF, WF)                                  \
        wait_vm<2 * C::PER>();                                                   \
        lds_barrier();                                                           \
        issue_stage<C>(src, XF, WF, wave, min(kb + (SS) + 4, last) * kBK, N);    \
        read_frags<C>(FN, XN, WN, lane, wm0, wn0);                               \
        mfma_frags<C>(acc, FC);                                                  \
        interleave_reads_with_mfma<C>();
        for (int s = 0; s < n; s += 4) {
            LORA_SK_STEP(s, fa, fb, X1, W1, X0, W0)
            LORA_SK_STEP(s + 1, fb, fa, X2, W2, X1, W1)
            LORA_SK_STEP(s + 2, fa, fb, X3, W3, X2, W2)
            LORA_SK_STEP(s + 3, fb, fa, X0, W0, X3, W3)
        }
#undef LORA_SK_STEP
        wait_vm<0>();

        // partial tile, row-major [BM][BN]: accumulator element v of a 32 x 32 block is row
        // (v/4)*8 + (lane/32)*4 + v%4, column lane%32 (each store covers two 128-byte rows)
        float *P = partial + (size_t)((ln + p) * n_tm + tm) * (C::BM * C::BN) +
                   (wm0 + (lane >> 5) * 4) * C::BN + wn0 + (lane & 31);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    P[(32 * i + (v / 4) * 8 + (v % 4)) * C::BN + 32 * j] = acc[i][j][v];
    }
}

// y[m][n .. n+7] = (partial tiles of the lanes that meet column panel n / BN, added in lane
// order) + scale_a * sum_{j < rank_a} t[m][j] B_a[j][n .. n+7] for a = ids[m] >= 0 (rows
// with id -1, or an id out of range, take the first term alone), rounded once into y.
// t comes as the shrink's k-chunk partial sums [n_chunks][M][r_max]: each block adds them for
// its 8 rows in LDS (threads of one (row, 4 ranks) group take every TPP-th chunk, and their
// sums are combined in thread order, so t does not depend on scheduling).
// Rows are taken in segment order (positions of perm), so rows of one adapter are neighbours
// and share B_a's rows through L1 and L2.  A block covers 8 positions x 256 columns (one
// panel), 8 columns per thread; blocks are handed to XCDs in contiguous runs (block b runs
// on XCD b % 8), panel-major, so one XCD reads a panel's partial slots and B columns.
template <class C, bool YF32>
__global__ __launch_bounds__(256) void sk_reduce_lora_kernel(
    const float *__restrict__ partial, int M, int K, int N, int n_tm, int n_tn, int n_tn1, int L,
    Seg seg, SkProj pj, int n_chunks, const float *__restrict__ scale,
    const int32_t *__restrict__ ids, const int32_t *__restrict__ ranks,
    const int32_t *__restrict__ roff, int pool_rows, int pstride, int r_max, int n_adapters) {
    static_assert(C::BN == 256, "one panel per block");
    __shared__ float4 s_part[256];
    __shared__ float s_t[8][64];
    const int G = (M + 7) / 8;  // position groups
    const int nblk = G * n_tn;
    int lin = blockIdx.x;
    if ((nblk & 7) == 0) lin = (lin & 7) * (nblk >> 3) + (lin >> 3);
    const int p = lin / G, g = lin % G;
    // panel p of the stream-K line is panel p - pr * n_tn1 of projection pr
    const int pr = p / n_tn1;
    const float *__restrict__ tpart = pick_proj(pr, pj.tpart);
    const uint16_t *__restrict__ B = pick_proj(pr, pj.B);
    void *__restrict__ y = pick_proj(pr, pj.y);
    const int pl = threadIdx.x >> 5;
    const int pos = g * 8 + pl;
    const int n = (p - pr * n_tn1) * C::BN + (threadIdx.x & 31) * 8;
    const bool live = pos < M && n < N;
    // this thread's partial tiles first, so their loads overlap the t sums below
    int m = 0, a = -1;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) {
        m = seg.perm[pos];
        a = ids[m];
        const int tm = m / C::BM, r = m % C::BM, c = n % C::BN;
        const int KI = K / kBK, total = n_tn * KI;
        const int k0 = p * KI, k1 = k0 + KI;
        // the lane whose range holds the panel's first step
        int l = (int)(((long)k0 * L) / total);
        while (l > 0 && sk_start(l, total, L) > k0) --l;
        while (l + 1 < L && sk_start(l + 1, total, L) <= k0) ++l;
        for (; l < L && sk_start(l, total, L) < k1; ++l) {
            const float *P = partial + ((size_t)((l + p) * n_tm + tm) * C::BM + r) * C::BN + c;
            const float4 u = *reinterpret_cast<const float4 *>(P);
            const float4 v = *reinterpret_cast<const float4 *>(P + 4);
            acc[0] += u.x; acc[1] += u.y; acc[2] += u.z; acc[3] += u.w;
            acc[4] += v.x; acc[5] += v.y; acc[6] += v.z; acc[7] += v.w;
        }
    }
    {
        // t of the block's rows: group q = (row, ranks 4 jq .. 4 jq + 3), TPP threads each
        const int groups = 8 * (r_max / 4), TPP = 256 / groups;
        const int q = threadIdx.x / TPP, h = threadIdx.x % TPP;
        const int rl = q / (r_max / 4), jq = q % (r_max / 4);
        const int ps = g * 8 + rl;
        float4 ts = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ps < M && ps < seg.meta[1]) {  // a LoRA row: its chunk sums were written
            const float *src = tpart + (size_t)seg.perm[ps] * r_max + 4 * jq;
            const size_t cs = (size_t)M * r_max;
            for (int ch = h; ch < n_chunks; ch += TPP) {
                const float4 v = *reinterpret_cast<const float4 *>(src + ch * cs);
                ts.x += v.x; ts.y += v.y; ts.z += v.z; ts.w += v.w;
            }
        }
        s_part[threadIdx.x] = ts;
        __syncthreads();
        if (h == 0) {
            float4 tv = s_part[threadIdx.x];
            for (int i = 1; i < TPP; ++i) {
                const float4 v = s_part[threadIdx.x + i];
                tv.x += v.x; tv.y += v.y; tv.z += v.z; tv.w += v.w;
            }
            s_t[rl][4 * jq] = tv.x; s_t[rl][4 * jq + 1] = tv.y;
            s_t[rl][4 * jq + 2] = tv.z; s_t[rl][4 * jq + 3] = tv.w;
        }
        __syncthreads();
    }
    if (!live) return;
    if (a >= 0 && a < n_adapters) {
        // the adapter's rank rows: all of a padded pool's stride, or fewer when ranks are
        // given (entries of t and B beyond the rank are zero), in groups of 4; rows past the
        // last row of the adapter are not loaded (they may be the next adapter's, or past
        // the pool)
        const int width = roff ? r_max : pstride;
        int rk = ranks ? min(max(ranks[a], 0), width) : width;
        const int row0 = adapter_row0(roff, pool_rows, a, pstride, rk);
        const float sc = scale[a];
        const float *tr = &s_t[pl][0];
        const uint16_t *Bp = B + (size_t)row0 * N + n;
        const uint4 z = make_uint4(0, 0, 0, 0);
        float d[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < rk; j += 4) {
            const float4 tv = make_float4(tr[j], tr[j + 1], tr[j + 2], tr[j + 3]);
            const uint4 b0 = ld16(Bp + (size_t)j * N);
            const uint4 b1 = j + 1 < rk ? ld16(Bp + (size_t)(j + 1) * N) : z;
            const uint4 b2 = j + 2 < rk ? ld16(Bp + (size_t)(j + 2) * N) : z;
            const uint4 b3 = j + 3 < rk ? ld16(Bp + (size_t)(j + 3) * N) : z;
            float f[8];
            unpack8(b0, f);
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] += tv.x * f[q];
            unpack8(b1, f);
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] += tv.y * f[q];
            unpack8(b2, f);
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] += tv.z * f[q];
            unpack8(b3, f);
#pragma unroll
            for (int q = 0; q < 8; ++q) d[q] += tv.w * f[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += sc * d[q];
    }
    if constexpr (YF32) {
        float *yf = reinterpret_cast<float *>(y) + (size_t)m * N + n;
        *reinterpret_cast<float4 *>(yf) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *reinterpret_cast<float4 *>(yf + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        st16(reinterpret_cast<uint16_t *>(y) + (size_t)m * N + n,
             make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                        pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])));
    }
}

using CfgSk = Big<256, 256, 2, 4>;

template <class C, bool SEGROWS, bool LORA>
hipError_t launch_big_cfg(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y,
                          bool y_f32, Seg seg, const LoraEpilogue *lora, hipStream_t s) {
    const int n_tm = (M + C::BM - 1) / C::BM, n_tn = (N + C::BN - 1) / C::BN;
    LoraEpilogue ep{};
    if (lora) ep = *lora;
    const dim3 grid(n_tm * n_tn);
    // the LoRA instances take 32-bit load offsets when x and W each fit in 4 GiB
    const bool o32 = LORA && (size_t)M * K * 2 <= 0xFFFFFFFFull && (size_t)K * N * 2 <= 0xFFFFFFFFull;
    if (o32) {
        if (y_f32)
            launch((gemm_big_kernel<C, SEGROWS, LORA, true, LORA>), grid, dim3(C::NT), 0, s, x, W,
                   M, K, N, y, n_tm, n_tn, seg, ep);
        else
            launch((gemm_big_kernel<C, SEGROWS, LORA, false, LORA>), grid, dim3(C::NT), 0, s, x, W,
                   M, K, N, y, n_tm, n_tn, seg, ep);
    } else {
        if (y_f32)
            launch((gemm_big_kernel<C, SEGROWS, LORA, true, false>), grid, dim3(C::NT), 0, s, x, W,
                   M, K, N, y, n_tm, n_tn, seg, ep);
        else
            launch((gemm_big_kernel<C, SEGROWS, LORA, false, false>), grid, dim3(C::NT), 0, s, x, W,
                   M, K, N, y, n_tm, n_tn, seg, ep);
    }
    return hipGetLastError();
}

}  // namespace

// Large-batch GEMM: prefill (segment-ordered rows, LoRA epilogue) when lora != nullptr,
// else plain y = x W in natural row order.  Needs N >= 8 (N % 8 == 0) and M >= 1.
hipError_t launch_gemm_big(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y,
                           bool y_f32, Seg seg, const LoraEpilogue *lora, hipStream_t s) {
    const long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);
    if (lora) {
        if (t256 >= 192) return launch_big_cfg<Big<256, 256, 2, 4>, true, true>(x, W, M, K, N, y, y_f32, seg, lora, s);
        if ((long)((M + 255) / 256) * ((N + 127) / 128) >= 192)
            return launch_big_cfg<Big<256, 128>, true, true>(x, W, M, K, N, y, y_f32, seg, lora, s);
        return launch_big_cfg<Big<128, 128>, true, true>(x, W, M, K, N, y, y_f32, seg, lora, s);
    }
    if (t256 >= 192) return launch_big_cfg<Big<256, 256, 2, 4>, false, false>(x, W, M, K, N, y, y_f32, seg, nullptr, s);
    if ((long)((M + 255) / 256) * ((N + 127) / 128) >= 192)
        return launch_big_cfg<Big<256, 128>, false, false>(x, W, M, K, N, y, y_f32, seg, nullptr, s);
    return launch_big_cfg<Big<128, 128>, false, false>(x, W, M, K, N, y, y_f32, seg, nullptr, s);
}


SkPlan sk_plan(int M, int K, int N, int n_proj) {
    SkPlan p{};
    if (M <= kDecodeGemmMaxRows || M > 1024 || K % (4 * kBK) != 0 || N % 8 != 0) return p;
    if (n_proj < 1 || n_proj > kMaxProj) return p;
    p.n_tm = (M + CfgSk::BM - 1) / CfgSk::BM;
    p.n_proj = n_proj;
    p.n_tn1 = (N + CfgSk::BN - 1) / CfgSk::BN;
    p.n_tn = n_proj * p.n_tn1;
    if ((long)p.n_tm * p.n_tn >= 192) return p;  // the data-parallel tiling fills the chip
    p.L = (256 / p.n_tm) / 8 * 8;
    if ((long)p.n_tn * (K / kBK) < 8L * p.L) return p;  // at least 8 K steps per lane
    p.use = true;
    return p;
}

size_t sk_partial_floats(const SkPlan &p) {
    return p.use ? (size_t)(p.L + p.n_tn - 1) * p.n_tm * CfgSk::BM * CfgSk::BN : 0;
}

hipError_t launch_gemm_sk(const uint16_t *x, const SkProj &pj, int M, int K, int N,
                          const SkPlan &p, float *partial, hipStream_t s) {
    // lanes in order of (K offset of their first step inside its panel, lane)
    const int KI = K / kBK, total = p.n_tn * KI;
    int off[256];
    SkLanes lanes;
    for (int l = 0; l < p.L; ++l) {
        off[l] = (4 * (int)(((long)l * (total / 4)) / p.L)) % KI;
        int r = l;  // insertion sort, stable
        while (r > 0 && off[lanes.lane[r - 1]] > off[l]) {
            lanes.lane[r] = lanes.lane[r - 1];
            --r;
        }
        lanes.lane[r] = (uint8_t)l;
    }
    launch(gemm_sk_kernel<CfgSk>, dim3(p.L * p.n_tm), dim3(CfgSk::NT), 0, s, x, pj, M, K, N,
           partial, p.n_tm, p.n_tn, p.n_tn1, p.L, lanes);
    return hipGetLastError();
}

hipError_t launch_sk_reduce_lora(const float *partial, int M, int K, int N, const SkPlan &p,
                                 Seg seg, const SkProj &pj, int n_chunks, const float *scale,
                                 const int32_t *ids, const int32_t *ranks, const int32_t *roff,
                                 int pool_rows, int pstride, int r_max, int n_adapters,
                                 bool y_f32, hipStream_t s) {
    if (r_max < 8 || r_max > 64 || (r_max & (r_max - 1)) != 0) return hipErrorInvalidValue;
    if (roff == nullptr && (pstride < 1 || pstride > r_max)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(((M + 7) / 8) * p.n_tn));
    if (y_f32)
        launch(sk_reduce_lora_kernel<CfgSk, true>, grid, dim3(256), 0, s, partial, M, K, N, p.n_tm,
               p.n_tn, p.n_tn1, p.L, seg, pj, n_chunks, scale, ids, ranks, roff, pool_rows, pstride,
               r_max, n_adapters);
    else
        launch(sk_reduce_lora_kernel<CfgSk, false>, grid, dim3(256), 0, s, partial, M, K, N, p.n_tm,
               p.n_tn, p.n_tn1, p.L, seg, pj, n_chunks, scale, ids, ranks, roff, pool_rows, pstride,
               r_max, n_adapters);
    return hipGetLastError();
}

}  // namespace lora

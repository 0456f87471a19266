// decode_tiles.h -- the split-K streaming core shared by the small-batch decode GEMM
// (csrc/decode_gemm.hip) and the expert-routed MoE GEMM (csrc/moe.hip): tile shapes, the
// direct global->LDS loads, the per-wave K loop on v_mfma_f32_32x32x16_bf16 and the
// cross-wave reduction of a partial tile.  Internal.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "How does one
// batch run 30 different adapters at once?" (at decode the cost is reading the weight bytes
// from HBM) and "Multi-LoRA Serving: Sharing One GPU Across Adapters" (cloudai.pt), "MoE
// Models Raise the Bar" (split-K for the skinny products).
#pragma once

#include "common.h"

namespace lora {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kBN = 128;  // columns of a tile
constexpr int kBKW = 16;  // k of a W stage (one step)
constexpr int kBKX = 64;  // k of an x stage (four steps)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Per wave: four W stages of 16 rows x 128 columns (256-byte rows, one direct load covers 4
// whole rows) and two x stages of BM rows x 64 k (128-byte rows, 8 whole rows per load).  A
// 128-column tile reads each x byte for twice the W bytes a 64-column tile did.
template <int BM_>
struct Dec {
    static constexpr int BM = BM_;
    static constexpr int TM = BM / 32, TN = kBN / 32;
    static constexpr int XSLOT = BM * kBKX * 2 / 16;     // uint4 per x stage
    static constexpr int WSLOT = kBKW * kBN * 2 / 16;    // uint4 per W stage
    static constexpr int XINS = XSLOT / 64;              // direct loads per x stage
    static constexpr int WINS = WSLOT / 64;              // direct loads per W stage
    static constexpr int WAVE = 2 * XSLOT + 4 * WSLOT;   // uint4 of LDS per wave
    static constexpr int TILE = BM * kBN;                 // floats per tile
    static_assert(BM == 32 || BM == 64, "decode tile rows");
    static_assert(TILE * 4 <= WAVE * 16, "a wave's partial tile fits its part of the LDS");
};

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// W stage rows are 256 bytes (16 chunks of 16 bytes); chunk c of row r is stored at
// c ^ (2 (r % 4)), so the 4 rows x 32 bytes of one transposing read of 16 lanes fall on
// distinct banks.  x stage rows are 128 bytes; chunk c of row r is stored at c ^ (r % 8).
__device__ __forceinline__ int wsw(int r) { return (r & 3) << 1; }

// acc += x[rows, k .. k+15] W[k .. k+15, tile]: `quarter` picks the x stage's 16 k.
template <class C>
__device__ __forceinline__ void dec_mfma(f32x16_t (&acc)[C::TM][C::TN], const uint4 *__restrict__ xs,
                                         int quarter, const uint4 *__restrict__ ws, int lane) {
    const lds_char_t *wsb = (const lds_char_t *)(ws);
    const int g = lane >> 4, li = lane & 15;
    bf16x8_t af[C::TM], bfr[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int row = 32 * i + (lane & 31);
        const int lc = 2 * quarter + (lane >> 5);
        af[i] = *reinterpret_cast<const bf16x8_t *>(&xs[row * 8 + (lc ^ (row & 7))]);
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        const int col = 32 * j + 16 * (g & 1) + 4 * (li & 3);
        const int lc = col >> 3, half = (col >> 2) & 1;
        const int r = 8 * (g >> 1) + (li >> 2);
        const lds_char_t *p = wsb + r * (kBN * 2) + ((lc ^ wsw(r)) << 4) + half * 8;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)p);
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(p + 4 * kBN * 2));
        bfr[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

template <class C>
struct DecSrc {
    const uint16_t *xp[C::XINS];
    const uint16_t *wp[C::WINS];
};
// The same with a row stride per W load: adapters of a rank-compact pool side by side in one
// tile, each load reading its own adapter's block (rows round8(rank) wide).
template <class C>
struct DecSrcVS {
    const uint16_t *xp[C::XINS];
    const uint16_t *wp[C::WINS];
    uint32_t ws[C::WINS];  // row stride of load q, elements
};
template <class C>
__device__ __forceinline__ size_t dec_wstride(const DecSrc<C> &, int, size_t ldw) { return ldw; }
template <class C>
__device__ __forceinline__ size_t dec_wstride(const DecSrcVS<C> &src, int q, size_t) {
    return src.ws[q];
}

// Direct global -> LDS load of 16 bytes per lane: lane i's bytes land at LDS address
// m0 + 16 i.  Issued from asm so that the compiler adds no wait of its own for it: its
// tracking of these loads cannot always tell the ring's stages apart and then waited for
// every load in flight (vmcnt 0) before reading a stage; the waits here are the explicit
// per-stage ones.  One wait state must separate the write of m0 from the load.
__device__ __forceinline__ void dma16(const void *g, const lds_void_t *l) {
    const uint32_t m = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m)
                 : "memory", "m0");
}

// A W stage of this wave: rows k0 .. k0+15 of the tile (row stride ldw, or the load's own).
template <class C, class S>
__device__ __forceinline__ void dec_issue_w(const S &src, uint4 *__restrict__ wslot, int k0,
                                            size_t ldw) {
#pragma unroll
    for (int q = 0; q < C::WINS; ++q)
        dma16(src.wp[q] + (size_t)k0 * dec_wstride<C>(src, q, ldw), (const lds_void_t *)&wslot[q * 64]);
}
// An x stage of this wave: x[rows][k0 .. k0+63].
template <class C, class S>
__device__ __forceinline__ void dec_issue_x(const S &src, uint4 *__restrict__ xslot, int k0) {
#pragma unroll
    for (int q = 0; q < C::XINS; ++q) dma16(src.xp[q] + k0, (const lds_void_t *)&xslot[q * 64]);
}

// Cross-wave reduction.  Value v of lane l in the wave's MFMA block (i, j) is row
// 32 i + 8 (v / 4) + 4 (l / 32) + v % 4, column 32 j + l % 32: the four values v = 4 q ..
// 4 q + 3 are four consecutive rows of one column.  Each wave stores them as one 16-byte
// vector per lane (16 B x 64 lanes contiguous per (i, j, q)); after a barrier, thread tid
// owns column tid % 128 and the row groups (4 rows) tid / 128 + 2 g, and adds the four
// waves' vectors in wave order.
template <class C>
__device__ __forceinline__ void reduce_waves_put(const f32x16_t (&acc)[C::TM][C::TN], float4 *red_mine,
                                                 int lane) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red_mine[((i * C::TN + j) * 4 + q) * 64 + lane] =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
}
// rows 4 g .. 4 g + 3 of column col, summed over the waves in order
template <class C>
__device__ __forceinline__ float4 reduce_waves_group(const float4 *red, int g, int col) {
    const int i = g >> 3, q = (g >> 1) & 3, h = g & 1, j = col >> 5;
    const int e = ((i * C::TN + j) * 4 + q) * 64 + 32 * h + (col & 31);
    constexpr int WV = C::TILE / 4;  // float4 per wave
    float4 s = red[e];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        const float4 v = red[w * WV + e];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    return s;
}

// Column tiles: n_tn tiles of W, then n_lt adapter tiles.  Adapter "slots" are numbered
// 0 .. T-1: with a pool no larger than the batch, slot = adapter id (T = n_adapters), else
// slot = row (T = M; slot m holds row m's adapter).  Adapter tile lt holds slots lt * APT ..
// lt * APT + APT - 1, each r_max columns wide.
template <int RM>
struct AdapterTiles {
    static_assert(RM == 8 || RM == 16 || RM == 32 || RM == 64, "rank bucket");
    static constexpr int APT = kBN / RM;  // adapters per tile
};

// The K loop of one wave: acc += x[rows, kw0 .. kw0 + 16 nst) W[same k, tile], streamed
// through the wave's own part of the LDS (mine_lds, C::WAVE uint4) by direct loads; the
// stages past the last reload it and are not computed.  Returns with loads of the ring still
// in flight (the caller waits vmcnt(0) before the LDS is reused).
template <class C, class S = DecSrc<C>>
__device__ __forceinline__ void dec_kloop(f32x16_t (&acc)[C::TM][C::TN], const S &src,
                                          uint4 *const mine_lds, int kw0, int nst, int K,
                                          size_t ldw, int lane) {
    uint4 *const X0 = mine_lds, *const X1 = mine_lds + C::XSLOT;
    uint4 *const W0 = mine_lds + 2 * C::XSLOT, *const W1 = W0 + C::WSLOT, *const W2 = W1 + C::WSLOT,
                 *const W3 = W2 + C::WSLOT;
    // W stage s holds k = KW(s) .. +15, x stage u holds k = KX(u) .. +63; stages past the last
    // reload the last one (an empty range loads k = 0), and an x stage that would run past K
    // starts at K - 64 instead, its later quarters then holding the wave's last steps
    const int kxl = nst > 0 ? min(kw0 + ((nst - 1) >> 2) * kBKX, K - kBKX) : 0;
#define KW(S) (nst > 0 ? kw0 + min((S), nst - 1) * kBKW : 0)
#define KX(U) (nst > 0 ? min(kw0 + (U) * kBKX, kxl) : 0)
    // Issue order: x(0), W(0), W(1), W(2); then step s issues x(s / 4 + 1) when s % 4 == 0,
    // then W(s + 3).  When step s starts, what was issued after the stages it needs (W(s),
    // and x(s / 4), which is older) is two W stages when s % 4 is 0 or 3, and two W stages
    // and an x stage when it is 1 or 2.
    dec_issue_x<C>(src, X0, KX(0));
    dec_issue_w<C>(src, W0, KW(0), ldw);
    dec_issue_w<C>(src, W1, KW(1), ldw);
    dec_issue_w<C>(src, W2, KW(2), ldw);
#define DEC_STEP(SS, PAT, XC, XN, WC, WN)                                                     \
    if (PAT == 0 || PAT == 3) wait_vm<2 * C::WINS>();                                         \
    else wait_vm<2 * C::WINS + C::XINS>();                                                    \
    wait_lgkm0();                                                                             \
    if (PAT == 0) dec_issue_x<C>(src, XN, KX((SS) / 4 + 1));                                  \
    dec_issue_w<C>(src, WN, KW((SS) + 3), ldw);                                               \
    if ((SS) < nst) dec_mfma<C>(acc, XC, (kw0 + (SS) * kBKW - KX((SS) / 4)) / kBKW, WC, lane);
    for (int s = 0; s < nst; s += 4) {
        // x stage s / 4 is in X0 when s / 4 is even
        uint4 *const XC = (s & 4) ? X1 : X0, *const XN = (s & 4) ? X0 : X1;
        DEC_STEP(s, 0, XC, XN, W0, W3)
        DEC_STEP(s + 1, 1, XC, XN, W1, W0)
        DEC_STEP(s + 2, 2, XC, XN, W2, W1)
        DEC_STEP(s + 3, 3, XC, XN, W3, W2)
    }
#undef DEC_STEP
#undef KW
#undef KX
}

}  // namespace

}  // namespace lora

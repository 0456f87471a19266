// decode_gemm.hip -- y = x W + (x A_i) B_i * scale_i for small (decode) batches: the shared
// GEMM streamed from HBM in K splits, then one kernel that adds the splits in order together
// with the LoRA expand of every row.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Why can't you
// just merge LoRA weights into the base model?" (the layer; x W is one GEMM over the batch)
// and "How does one batch run 30 different adapters at once?" (at decode every request adds
// one row, and the cost is the weight bytes read from HBM); "Multi-LoRA Serving: Sharing One
// GPU Across Adapters" (cloudai.pt), "MoE Models Raise the Bar" (split-K for skinny products,
// the expand step).
//
// gfx950 design.  With one row per request, x W is bound by reading W once from HBM.
//  * Output tile = BM rows (all of a small batch, padded to 32 or 64) x 128 columns; the K
//    range of each tile is split over `ks` workgroups (tiles x ks fills the 256 CUs once)
//    and, inside a workgroup, over its four waves.  Each wave streams its own K sub-range
//    through its own LDS ring filled by direct global->LDS loads, so the K loop has no
//    workgroup barrier at all: only this wave's s_waitcnt orders its loads and reads.
//  * Per wave: four W stages of 16 x 128 (256-byte rows) and two x stages of BM x 64
//    (128-byte rows), XOR-swizzled, every direct load covering whole rows; the W operand is
//    read with the transposing LDS read (ds_read_b64_tr_b16); v_mfma_f32_32x32x16_bf16.  A
//    tile twice as wide as the MFMA needs reads each x byte for twice the W bytes, and the
//    workgroup's memory traffic (W and x through the same CU) is what bounds it.
//  * The LoRA shrink t = x A_a is the same kind of product: the batch's adapters, laid side
//    by side, are 128 / r_max adapters per extra "adapter tile" whose rows are
//    A_a[k, 0:r_max] (row stride r_max instead of N).  Those tiles run in the same launch,
//    split and streamed exactly like the W tiles, so every touched A_a is read from HBM
//    once, at the same rate as W, with no latency chain of its own.  A tile computes t for
//    every row of the batch against its adapters; the reduction keeps each row's own.
//  * The four waves' partial tiles are added through LDS in wave order (16-byte vectors of
//    four rows) and each workgroup writes its partial tile.
//  * reduce_lora_kernel then writes y[m, :] = (sum of the split partials, in split order)
//    + scale_a * (t[m, :] B_a) with t[m, :] summed over the splits of row m's adapter tile,
//    in split order, in fp32, rounded once into y's dtype; each touched B_a row slice is
//    read once from HBM (rows of one adapter share it through L2).  No atomics: the result
//    does not depend on scheduling.
//  * Batches of 129-256 rows (which come with segments) take reduce_seg_kernel instead: the
//    same sums for items of four rows of one adapter, each B_a chunk loaded once per item.
#include <type_traits>

#include "decode_tiles.h"
#include "segments_block.h"

namespace lora {

namespace {

// Sources of adapter tile lt of a fused call: adapters laid side by side, 128 / RM slots per
// tile.  With a pool no larger than the batch, slot = adapter id; otherwise slot = row: slot m
// holds row m's adapter (rows sharing an adapter read the same A lines, from L2), so the tile
// needs only its rows' ids, and the reduction finds row m's t at slot m.  (Grouping the
// batch's distinct adapters first -- an ids load, then a scan and three barriers in LDS --
// held the adapter tiles 2.8 us before their first load against 0.6 us for W tiles, and with 8
// distinct adapters in 64 rows they ended last: 19.0-19.6 us per step at 64 x 4096 x 4096
// against 17.6 with the adapters numbered by id.)  Returns false -- for the whole workgroup --
// when the tile has nothing to compute.  Every thread must call it (barriers).
template <class C, int RM, class S>
__device__ __forceinline__ bool dec_adapter_src(S &src, const DecodeLora &lo, const uint16_t *A,
                                                int M, int K, int lt, int tid, int lane) {
    constexpr int APT = AdapterTiles<RM>::APT;
    constexpr bool COMPACT = !std::is_same<S, DecSrc<C>>::value;
    const bool by_id = lo.n_adapters <= M;
    const int T = by_id ? lo.n_adapters : M;  // slots
    if (lt * APT >= T) return false;  // no slot in this tile
    if (by_id) {
        // numbered by id, a tile may hold only adapters no row of the batch uses
        bool used = false;
        for (int m = tid; m < M; m += kThreads) {
            const int d = lo.ids[m] - lt * APT;
            used |= d >= 0 && d < APT;
        }
        if (!__syncthreads_or(used)) return false;
    }
#pragma unroll
    for (int q = 0; q < C::WINS; ++q) {
        const int r = 4 * q + (lane >> 4);
        const int col = ((lane & 15) ^ wsw(r)) * 8;
        const int sl = lt * APT + col / RM;
        // slots past the last, and rows without a valid adapter, read adapter 0; their columns
        // are never used
        int a = 0;
        if (by_id) {
            a = sl < T ? sl : 0;
        } else if (sl < T) {
            const int id = lo.ids[sl];
            a = id >= 0 && id < lo.n_adapters ? id : 0;
        }
        if constexpr (!COMPACT) {
            src.wp[q] = A + ((size_t)a * K + r) * RM + col % RM;
        } else {
            // the adapter's own block, w rows wide from its first rank row: a padded pool's
            // stride, or a rank-compact adapter's round8(rank); groups past w read the last
            // group again (same lines, no HBM bytes; those t columns lie past the rank and are
            // never read).  A compact adapter whose rows leave the pool (rank read as 0) reads
            // element 0 at stride 0; it adds nothing.
            int row0, w;
            if (lo.roff != nullptr) {
                int rk = lo.ranks ? min(max(lo.ranks[a], 1), RM) : RM;
                row0 = adapter_row0(lo.roff, lo.pool_rows, a, 0, rk);
                w = rk > 0 ? (rk + 7) & ~7 : 0;
            } else {
                row0 = a * lo.pstride;
                w = lo.pstride;
            }
            if (w > 0) {
                src.wp[q] = A + (size_t)row0 * K + (size_t)r * w + min(col % RM, w - 8);
                src.ws[q] = (uint32_t)w;
            } else {
                src.wp[q] = A;
                src.ws[q] = 0;
            }
        }
    }
    return true;
}

// x rows m0 .. m0 + BM of a tile: lane l fills position l % 8 of row 8 q + l / 8, chunk
// (l % 8) ^ (l / 8); rows past the batch repeat its last.
template <class C, class S>
__device__ __forceinline__ void dec_x_src(S &src, const uint16_t *x, int M, int K, int m0,
                                          int lane) {
#pragma unroll
    for (int q = 0; q < C::XINS; ++q) {
        const int row = 8 * q + (lane >> 3);
        const int lc = (lane & 7) ^ (lane >> 3);
        const int m = min(m0 + row, M - 1);
        src.xp[q] = x + (size_t)m * K + lc * 8;
    }
}

// The reduction that follows a decode GEMM starts with dependent loads of the small tables (a
// row's adapter, then its rank and scale, then B); left to it they come from HBM.  Touched at
// the end of the GEMM's tiles, they are in every XCD's L2 by then.  One asm block issues the
// three loads and waits for every load of the wave (the K loop's included), so no load is in
// flight when the block ends; its results are then handed to an empty asm.
__device__ __forceinline__ void touch_tables(const DecodeLora &lo, int M, int tid) {
    const int mm = min(tid, M - 1), aa = min(tid, lo.n_adapters - 1);
    uint32_t d0, d1, d2;
    asm volatile(
        "global_load_dword %0, %3, off\n\t"
        "global_load_dword %1, %4, off\n\t"
        "global_load_dword %2, %5, off\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(d0), "=&v"(d1), "=&v"(d2)
        : "v"(lo.ids + mm), "v"(lo.scale + aa), "v"(lo.ranks ? lo.ranks + aa : lo.ids + mm)
        : "memory");
    asm volatile("" ::"v"(d0), "v"(d1), "v"(d2));
}

// After a tile's K loop: wait for every load (touching the reduction's tables), add the four
// waves' partial tiles in wave order through LDS and write the workgroup's partial tile to
// `mine`.  WT: written through the L2 (the small-batch launches, whose end-of-kernel
// write-back of the partial tiles was a visible part of a launch of ~13 us: 12.8-13.0 ->
// 12.3-12.5 us at 64 x 4096 x 4096; the 256-row GEMM, whose stores overlap a longer W
// stream, measured 0.5 us slower with them, so it keeps plain stores).  Every thread must call
// it (barriers).
template <class C, bool WT>
__device__ __forceinline__ void dec_tile_out(const f32x16_t (&acc)[C::TM][C::TN], uint4 *lds,
                                             const DecodeLora &lo, int M, float *mine, int tid,
                                             int lane, int wave) {
    touch_tables(lo, M, tid);
    __syncthreads();  // every wave is done with its stages

    float4 *const red = reinterpret_cast<float4 *>(lds);
    reduce_waves_put<C>(acc, red + wave * (C::TILE / 4), lane);
    __syncthreads();
    const int col = tid & 127;
#pragma unroll
    for (int q = 0; q < C::BM / 8; ++q) {
        const int g = (tid >> 7) + 2 * q;  // rows 4 g .. 4 g + 3
        const float4 s = reduce_waves_group<C>(red, g, col);
        float *o = mine + (4 * g) * kBN + col;
        if constexpr (WT) {
            st_wt(o, s.x); st_wt(o + kBN, s.y); st_wt(o + 2 * kBN, s.z); st_wt(o + 3 * kBN, s.w);
        } else {
            o[0] = s.x; o[kBN] = s.y; o[2 * kBN] = s.z; o[3 * kBN] = s.w;
        }
    }
}

// Workgroup (tile, split), four waves.  Each wave streams its quarter of split `split` of K
// (rows [split k_per_split, +k_per_split)) for one 128-column tile -- of W, or of the
// adapters' A laid side by side -- and the workgroup writes its partial tile;
// reduce_lora_kernel adds the splits in order.
// BUILD: one more workgroup (the last) builds the segments instead (see SegBuild).
template <class C, int RM, bool BUILD, bool CPT>
__global__ __launch_bounds__(kThreads) void decode_gemm_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, const uint16_t *__restrict__ A,
    int M, int K, int N, int n_tm, int n_tn, int n_lt, int k_per_split, float *__restrict__ partial,
    DecodeLora lo, int n_gemm_blocks, SegBuild build) {
    // wave w's part: x stages 0, 1 then W stages 0 .. 3; after the K loop, its partial tile
    __shared__ __attribute__((aligned(1024))) uint4 lds[kWaves * C::WAVE];

    if (BUILD && (int)blockIdx.x >= n_gemm_blocks) {
        // the extra workgroup: the segment build, in this kernel's LDS (the launch is a grid of
        // one workgroup per CU or fewer, so it runs beside the GEMM on a CU of its own)
        static_assert(kWaves * C::WAVE * 16 >= (LORA_MAX_ADAPTERS + 1) * 4 + 64 * 4,
                      "the builder's tables fit the GEMM's LDS");
        int32_t *cnt = reinterpret_cast<int32_t *>(lds);
        int32_t(*wave_tot)[kWaves] =
            reinterpret_cast<int32_t(*)[kWaves]>(cnt + ((build.n_adapters + 1 + 15) & ~15));
        build_segments_block<kThreads>(build.ids, M, build.n_adapters, build.seg, cnt, wave_tot,
                                       &wave_tot[3][0]);
        return;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_cols = n_tn + n_lt;
    const int n_tiles = n_tm * n_cols;
    // block -> (split, column tile, row tile).  With two row tiles, row tile fastest over
    // consecutive blocks of one XCD (workgroup b runs on XCD b % 8), so both read a W column
    // panel through that XCD's L2
    int lin = blockIdx.x;
    if (n_tm > 1 && (n_gemm_blocks & 7) == 0) lin = (blockIdx.x & 7) * (n_gemm_blocks >> 3) + (blockIdx.x >> 3);
    const int tile = lin % n_tiles, split = lin / n_tiles;
    const int tm = tile % n_tm, tn = tile / n_tm;
    const int m0 = tm * C::BM;

    // per-lane sources of the tile: W, or the adapters of this adapter tile.  Direct load q of
    // a W stage: lane l fills position l % 16 of row 4 q + l / 16, i.e. chunk
    // (l % 16) ^ wsw(row) of the row's 16.  CPT: the adapters come from a rank-compact pool,
    // each load with its adapter's row stride.
    std::conditional_t<CPT, DecSrcVS<C>, DecSrc<C>> src;
    size_t ldw = (size_t)N;
    if (tn < n_tn) {
        const int n0 = tn * kBN;
#pragma unroll
        for (int q = 0; q < C::WINS; ++q) {
            const int r = 4 * q + (lane >> 4);
            const int lc = (lane & 15) ^ wsw(r);
            src.wp[q] = W + (size_t)r * N + min(n0 + lc * 8, N - 8);
            if constexpr (CPT) src.ws[q] = (uint32_t)N;
        }
    } else {
        const int lt = tn - n_tn;
        if (!dec_adapter_src<C, RM>(src, lo, A, M, K, lt, tid, lane)) return;  // whole workgroup
        ldw = RM;
    }
    dec_x_src<C>(src, x, M, K, m0, lane);

    f32x16_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int ks0 = split * k_per_split;
    const int ks1 = min(K, ks0 + k_per_split);
    const int per_wave = k_per_split / kWaves;  // multiple of 16
    const int kw0 = min(ks1, ks0 + wave * per_wave);
    const int kw1 = min(ks1, kw0 + per_wave);
    const int nst = (kw1 - kw0) / kBKW;
    dec_kloop<C>(acc, src, lds + wave * C::WAVE, kw0, nst, K, ldw, lane);
    float *const mine = partial + ((size_t)split * n_tiles + tile) * C::TILE;
    if (n_lt > 0)  // a small-batch launch (adapter tiles)
        dec_tile_out<C, true>(acc, lds, lo, M, mine, tid, lane, wave);
    else
        dec_tile_out<C, false>(acc, lds, lo, M, mine, tid, lane, wave);
}

// ---- the same split-K GEMM with an fp8 base weight -----------------------------------------
// W8 holds E4M3 codes (OCP 8-bit floating point) laid out W8[N][K] -- each output column's K
// codes contiguous -- with one fp32 scale per column: W_eff[k, n] = w_scale[n] dec(W8[n, k]).
// Tiles and splits are decode_gemm_kernel's (dec_plan without adapter tiles), so the decode
// reduction adds these partial tiles unchanged; the partial tile is multiplied by the columns'
// scales before it is stored.
//
// At decode sizes both GEMMs are bound by the memory requests the CU can issue -- the cache
// lines each load instruction touches -- not by HBM: W8[N][K] gives a column's codes as a
// contiguous run, so a 16-byte piece per column touched one line per lane and kept the
// texture unit waiting on L1 (TA_ADDR_STALLED_BY_TC_CYCLES 4.5x the bf16 kernel's).  Here:
//  * the four waves split the 128 columns (32 each) and each load of W8 covers 8 columns x
//    128 codes (whole 128-byte lines); x is loaded once per workgroup and shared;
//  * a stage is 128 k: x[BM rows][128 k] (loaded by all waves) and each wave's W8[32 cols]
//    [128 k]; three stages in a ring, two ahead, one barrier per stage (a fourth slot,
//    three ahead, measured no faster);
//  * W stage of a wave: column c, 16-k chunk kc at LDS slot 8 c + (kc ^ ((c >> 1) & 7)), so an
//    MFMA's B operand (8 codes of 32 columns, ds_read_b64) has 2-way bank conflicts at most;
//    x stage: row r, 8-k chunk lc at slot 16 r + (lc ^ (r % 16));
//  * codes become bf16 with v_cvt_scalef32_pk_bf16_fp8 (scale 1: exact, every E4M3 value is a
//    bf16 value) for v_mfma_f32_32x32x16_bf16, with two accumulator sets (even and odd steps)
//    and no branch inside a stage, so the LDS reads of all eight steps can be issued ahead
//    of the MFMAs (with a branch per step and one set: 16.3 us at 64 x 4096 x 4096, now
//    11.6 us); each wave writes its columns of the partial tile straight from its
//    accumulators.
constexpr int kF8K = 128;  // k per fp8 stage

template <int BM_>
struct DecF8 {
    static constexpr int BM = BM_;
    static constexpr int TM = BM / 32;
    static constexpr int XSLOT = BM * kF8K * 2 / 16;      // uint4 per x stage
    static constexpr int WSLOT_W = 32 * kF8K / 16;         // uint4 per W stage of one wave
    static constexpr int XI = XSLOT / kWaves / 64;         // x loads per wave per stage
    static constexpr int WI = WSLOT_W / 64;                // W loads per wave per stage (4)
    static constexpr int SLOT = XSLOT + kWaves * WSLOT_W;  // uint4 per ring slot
    static constexpr int TILE = BM * kBN;
    static constexpr int BUILD16 = ((LORA_MAX_ADAPTERS + 1 + 15) / 16 * 64 + 64 * 4 + 15) / 16;
    static constexpr int LDS16 = 3 * SLOT > BUILD16 ? 3 * SLOT : BUILD16;  // uint4 of LDS
    static_assert(XI >= 1 && XSLOT % (kWaves * 64) == 0, "whole x loads per wave");
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;

// 8 codes (two dwords) -> 8 bf16
__device__ __forceinline__ bf16x8_t dec_fp8x8(uint32_t lo, uint32_t hi) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Workgroup (tile, split) of fp8 W tile tn: rows m0 .. m0 + BM of x, columns n0 .. n0 + 127
// (wave w: 32 w ..), k in the split; writes partial tile `tile` of split `split` (n_tiles
// tiles per split), through the L2 with WT (small batches, as dec_tile_out).  Every thread
// must call it (barriers).
template <class C, bool WT>
__device__ __forceinline__ void f8_tile(uint4 *lds, const uint16_t *__restrict__ x,
                                        const uint8_t *__restrict__ W8,
                                        const float *__restrict__ w_scale, int M, int K, int N,
                                        int n_tiles, int tile, int split, int tm, int tn,
                                        int k_per_split, float *__restrict__ partial, int lane,
                                        int wave) {
    const int m0 = tm * C::BM, n0 = tn * kBN;
    const int ks0 = split * k_per_split;
    const int ks1 = min(K, ks0 + k_per_split);
    const int nst = (ks1 - ks0) / kBKW;        // 16-k steps (K % 32 == 0)
    const int nsg = (nst + 7) >> 3;             // 128-k stages
    const int klast = ks0 + (nst - 1) * kBKW;   // first k of the last step

    // W8 load q of a stage, lane l: column c = 8 q + l / 8 of the wave's 32 (columns past N
    // read the last one, never used), chunk (l % 8) ^ ((c >> 1) & 7), to slot 64 q + l = 8 c +
    // (l % 8)
    const uint8_t *wp[C::WI];
    int wkc[C::WI];
#pragma unroll
    for (int q = 0; q < C::WI; ++q) {
        const int c = 8 * q + (lane >> 3);
        wp[q] = W8 + (size_t)min(n0 + 32 * wave + c, N - 1) * K;
        wkc[q] = (lane & 7) ^ ((c >> 1) & 7);
    }
    // x load q of a stage, lane l (this wave's part): row r = 4 (XI wave + q) + l / 16, chunk
    // (l % 16) ^ (r % 16), to slot 16 r + (l % 16) (rows past the batch repeat its last)
    const uint16_t *xp[C::XI];
    int xlc[C::XI];
#pragma unroll
    for (int q = 0; q < C::XI; ++q) {
        const int r = 4 * (C::XI * wave + q) + (lane >> 4);
        xp[q] = x + (size_t)min(m0 + r, M - 1) * K;
        xlc[q] = (lane & 15) ^ (r & 15);
    }

    auto issue = [&](int u, uint4 *slot) {
        // stage u: codes and x from k0 = ks0 + 128 u; chunks past the split's last step
        // repeat it (W) or stop at K (x) -- their steps are not computed
        const int k0 = ks0 + kF8K * min(u, nsg - 1);
        uint4 *xs = slot, *ws = slot + C::XSLOT + wave * C::WSLOT_W;
#pragma unroll
        for (int q = 0; q < C::XI; ++q)
            dma16(xp[q] + min(k0 + 8 * xlc[q], K - 8), (const lds_void_t *)&xs[(C::XI * wave + q) * 64]);
#pragma unroll
        for (int q = 0; q < C::WI; ++q)
            dma16(wp[q] + min(k0 + 16 * wkc[q], klast), (const lds_void_t *)&ws[q * 64]);
    };

    // two accumulator sets (even and odd steps) so that twice as many MFMA chains are
    // independent; added at the end
    f32x16_t acc[C::TM][2];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][0][v] = acc[i][1][v] = 0.0f;

    uint4 *const S0 = lds, *const S1 = lds + C::SLOT, *const S2 = lds + 2 * C::SLOT;
    issue(0, S0);
    issue(1, S1);
    const int c = lane & 31, g = lane >> 5;
    for (int u = 0; u < nsg; ++u) {
        uint4 *const SC = (u % 3 == 0) ? S0 : (u % 3 == 1) ? S1 : S2;
        uint4 *const SN = (u % 3 == 0) ? S2 : (u % 3 == 1) ? S0 : S1;  // slot of stage u + 2
        wait_vm<C::XI + C::WI>();  // this wave's loads of stage u are in (stage u + 1's pending)
        __syncthreads();           // every wave's loads of stage u are in; stage u - 1 is done
        issue(u + 2, SN);
        const uint4 *xs = SC;
        const lds_char_t *ws = (const lds_char_t *)(SC + C::XSLOT + wave * C::WSLOT_W);
        // steps past the split's last carry zero codes (a select, not a branch, so the
        // compiler may issue every step's LDS reads ahead of the MFMAs)
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const u32x2_t v = *(const lds_u32x2_t *)(ws + (8 * c + (st ^ ((c >> 1) & 7))) * 16 + 8 * g);
            const bool ok = 8 * u + st < nst;
            const bf16x8_t b = dec_fp8x8(ok ? v[0] : 0u, ok ? v[1] : 0u);
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const int r = 32 * i + c;
                const bf16x8_t a = *reinterpret_cast<const bf16x8_t *>(&xs[16 * r + ((2 * st + g) ^ (r & 15))]);
                acc[i][st & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i][st & 1], 0, 0, 0);
            }
        }
    }
    wait_vm<0>();  // the ring's last (unused) loads land before the workgroup ends

    // the wave's 32 columns of the scaled partial tile: element v of block i is row
    // 32 i + (v / 4) * 8 + g * 4 + v % 4, column c
    const int col = n0 + 32 * wave + c;
    const float sc = w_scale[min(col, N - 1)];
    float *P = partial + ((size_t)split * n_tiles + tile) * C::TILE + 32 * wave + c;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float *const o = &P[(size_t)(32 * i + (v / 4) * 8 + g * 4 + v % 4) * kBN];
            const float val = sc * (acc[i][0][v] + acc[i][1][v]);
            if constexpr (WT) st_wt(o, val);
            else *o = val;
        }
}

// Workgroup (tile, split) of the fp8 GEMM.  BUILD: one more workgroup (the last) builds the
// segments instead.
template <class C, bool BUILD>
__global__ __launch_bounds__(kThreads) void decode_gemm_fp8_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ W8, const float *__restrict__ w_scale,
    int M, int K, int N, int n_tm, int n_tn, int k_per_split, float *__restrict__ partial,
    int n_gemm_blocks, SegBuild build) {
    __shared__ __attribute__((aligned(1024))) uint4 lds[C::LDS16];

    if (BUILD && (int)blockIdx.x >= n_gemm_blocks) {
        int32_t *cnt = reinterpret_cast<int32_t *>(lds);
        int32_t(*wave_tot)[kWaves] =
            reinterpret_cast<int32_t(*)[kWaves]>(cnt + ((build.n_adapters + 1 + 15) & ~15));
        build_segments_block<kThreads>(build.ids, M, build.n_adapters, build.seg, cnt, wave_tot,
                                       &wave_tot[3][0]);
        return;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_tiles = n_tm * n_tn;
    int lin = blockIdx.x;
    if (n_tm > 1 && (n_gemm_blocks & 7) == 0) lin = (blockIdx.x & 7) * (n_gemm_blocks >> 3) + (blockIdx.x >> 3);
    const int tile = lin % n_tiles, split = lin / n_tiles;
    if (M <= kDecodeMaxRows)
        f8_tile<C, true>(lds, x, W8, w_scale, M, K, N, n_tiles, tile, split, tile % n_tm,
                         tile / n_tm, k_per_split, partial, lane, wave);
    else
        f8_tile<C, false>(lds, x, W8, w_scale, M, K, N, n_tiles, tile, split, tile % n_tm,
                          tile / n_tm, k_per_split, partial, lane, wave);
}

// The fp8 GEMM with the shrink as adapter tiles, for batches of at most kDecodeMaxRows rows
// and pools padded at a rank bucket: column tiles 0 .. n_tn - 1 are fp8 W tiles (f8_tile),
// the next n_lt are adapter tiles streamed by the bf16 decode GEMM's core (decode_tiles.h),
// all with one split plan (dec_plan with the adapter tiles) and one partial layout, so the
// decode reduction adds W's scaled splits and sums t from the adapter tiles exactly as after
// decode_gemm_kernel.  Both kinds of workgroup share one LDS array sized for the larger.
template <class CF, class CB, int RM>
__global__ __launch_bounds__(kThreads) void decode_gemm_fp8_lora_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ W8, const float *__restrict__ w_scale,
    const uint16_t *__restrict__ A, int M, int K, int N, int n_tm, int n_tn, int n_lt,
    int k_per_split, float *__restrict__ partial, DecodeLora lo, int n_gemm_blocks) {
    static_assert(CF::BM == CB::BM && CF::TILE == CB::TILE, "one tile shape");
    constexpr int L16 = CF::LDS16 > kWaves * CB::WAVE ? CF::LDS16 : kWaves * CB::WAVE;
    __shared__ __attribute__((aligned(1024))) uint4 lds[L16];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_tiles = n_tm * (n_tn + n_lt);
    int lin = blockIdx.x;
    if (n_tm > 1 && (n_gemm_blocks & 7) == 0) lin = (blockIdx.x & 7) * (n_gemm_blocks >> 3) + (blockIdx.x >> 3);
    const int tile = lin % n_tiles, split = lin / n_tiles;
    const int tm = tile % n_tm, tn = tile / n_tm;
    if (tn < n_tn) {
        f8_tile<CF, true>(lds, x, W8, w_scale, M, K, N, n_tiles, tile, split, tm, tn,
                          k_per_split, partial, lane, wave);
        return;
    }
    const int lt = tn - n_tn;
    DecSrc<CB> src;
    if (!dec_adapter_src<CB, RM>(src, lo, A, M, K, lt, tid, lane)) return;  // whole workgroup
    dec_x_src<CB>(src, x, M, K, tm * CB::BM, lane);
    f32x16_t acc[CB::TM][CB::TN];
#pragma unroll
    for (int i = 0; i < CB::TM; ++i)
#pragma unroll
        for (int j = 0; j < CB::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const int ks0 = split * k_per_split;
    const int ks1 = min(K, ks0 + k_per_split);
    const int per_wave = k_per_split / kWaves;  // multiple of 16
    const int kw0 = min(ks1, ks0 + wave * per_wave);
    const int kw1 = min(ks1, kw0 + per_wave);
    dec_kloop<CB>(acc, src, lds + wave * CB::WAVE, kw0, (kw1 - kw0) / kBKW, K, RM, lane);
    dec_tile_out<CB, true>(acc, lds, lo, M, partial + ((size_t)split * n_tiles + tile) * CB::TILE, tid,
                     lane, wave);
}

// y[m, n .. n+3] = (sum over splits, in order, of the partial tiles)
//                  + scale_a * sum_j t[m, j] B_a[j, n .. n+3]   (a = ids[m], when valid)
// with t[m, j] the sum, in order, of n_t parts tsrc[c * t_stride + ...]: the splits of row
// m's adapter tile (n_lt > 0), or the segment-path shrink's chunk sums tpart[c][m][j]
// (n_lt == 0).  Block (column chunk of 1024, row m), 256 threads x 4 columns.  The partial
// and B loads are issued before t is summed, so their latency overlaps it.
// MS: the most splits the launch can have (4 or 16; registers for the split partials).
// PADRM: the pool is padded at stride RM (no roff, pstride == RM); the row addressing then
// uses the compile-time stride (a runtime stride measured 2 us slower at 256 rows, r_max 64).
template <int BM, int RM, bool YF32, int MS, bool PADRM>
__global__ __launch_bounds__(256) void reduce_lora_kernel(const float *__restrict__ partial,
                                                          int M, int N, int n_tm, int n_tn,
                                                          int n_lt, int n_splits, DecodeLora lo,
                                                          void *__restrict__ y) {
    constexpr int kMaxSplits = MS;
    constexpr int APT = AdapterTiles<RM>::APT;
    __shared__ float s_t[RM];
    constexpr int kTpartMax = 4096;  // n_t x RM floats staged in LDS
    const int m = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    const bool col_ok = n < N;
    const int nc = col_ok ? n : 0;
    const int id = lo.ids[m];
    const bool has = id >= 0 && id < lo.n_adapters;
    const int a = has ? id : 0;
    const int n_tiles = n_tm * (n_tn + n_lt);
    const size_t stride = (size_t)n_tiles * BM * kBN;  // one split of the partial tiles

    // split partials of (m, nc .. nc+3)
    const int tile = (m / BM) + (nc / kBN) * n_tm;
    const float *pp = partial + (size_t)tile * BM * kBN + (m % BM) * kBN + (nc % kBN);
    float4 pv[kMaxSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp)
        if (sp < n_splits) pv[sp] = *reinterpret_cast<const float4 *>(pp + sp * stride);
    // B_a[j, nc .. nc+3] for the adapter's rank rows, issued together (the rank is uniform
    // in the block, so rows at or beyond it are not added, and above r_max 16 not loaded)
    const int width = PADRM || lo.roff ? RM : lo.pstride;
    int r = !has ? 0 : lo.ranks ? min(max(lo.ranks[a], 1), width) : width;
    const int row0 = PADRM ? a * RM : adapter_row0(lo.roff, lo.pool_rows, a, lo.pstride, r);
    // the first BCH rank rows of B are loaded here; above r_max 16 the rest follow in chunks
    // of 16 rows after t is summed (all 64 at once would take 128 registers)
    constexpr int BCH = RM <= 16 ? RM : 16;
    uint2 bv[BCH];
    const uint16_t *bp = lo.B + (size_t)row0 * N + nc;
    // in a padded pool at r_max <= 16 every row is loaded (the padding rows exist), so the
    // loads need not wait for the rank; a compact pool's rows past the rank are the next
    // adapter's, and so are a padded pool's past its stride when that is below the bucket
    if (RM <= 16 && PADRM) {
#pragma unroll
        for (int j = 0; j < BCH; ++j) bv[j] = *reinterpret_cast<const uint2 *>(bp + (size_t)j * N);
    } else {
#pragma unroll
        for (int j = 0; j < BCH; ++j)
            bv[j] = j < r ? *reinterpret_cast<const uint2 *>(bp + (size_t)j * N) : make_uint2(0, 0);
    }
    // where the parts of t[m, :] are
    const float *tsrc;
    size_t t_stride;
    int n_t;
    if (n_lt > 0) {
        const int sl = !has ? 0 : lo.n_adapters <= M ? id : m;  // slot: id, or row
        const int ttile = (m / BM) + (n_tn + sl / APT) * n_tm;
        tsrc = partial + (size_t)ttile * BM * kBN + (m % BM) * kBN + (sl % APT) * RM;
        t_stride = stride;
        n_t = n_splits;
    } else {
        tsrc = lo.tpart + (size_t)m * RM;
        t_stride = (size_t)M * RM;
        n_t = lo.n_chunks;
    }
    // t[m, j] = sum over parts c, in order: the block loads the n_t x RM values at once (one
    // or a few per thread) into LDS, then thread j adds its column in order (for very many
    // parts, thread j reads its column directly)
    __shared__ float s_tp[kTpartMax];
    const int nv = n_t * RM;
    const bool staged = nv <= kTpartMax;
    if (has && staged)
        for (int v = threadIdx.x; v < nv; v += 256) s_tp[v] = tsrc[(v / RM) * t_stride + v % RM];
    __syncthreads();
    if (has && threadIdx.x < RM) {
        float t = 0.0f;
        if (staged) {
            for (int c = 0; c < n_t; ++c) t += s_tp[c * RM + threadIdx.x];
        } else {
            for (int c = 0; c < n_t; ++c) t += tsrc[c * t_stride + threadIdx.x];
        }
        s_t[threadIdx.x] = t;
    }
    __syncthreads();

    float4 acc = pv[0];
#pragma unroll
    for (int sp = 1; sp < kMaxSplits; ++sp) {
        if (sp < n_splits) {
            acc.x += pv[sp].x; acc.y += pv[sp].y; acc.z += pv[sp].z; acc.w += pv[sp].w;
        }
    }
    if (has) {
        float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
        // chunk j0 is multiplied while chunk j0 + BCH is being loaded (r is uniform in the
        // block; rows past the rank add nothing)
#pragma unroll
        for (int j0 = 0; j0 < RM; j0 += BCH) {
            if (j0 >= r) break;
            uint2 nb[BCH];
            const bool more = RM > BCH && j0 + BCH < r;
            if (more) {
#pragma unroll
                for (int j = 0; j < BCH; ++j)
                    nb[j] = j0 + BCH + j < r ? *reinterpret_cast<const uint2 *>(bp + (size_t)(j0 + BCH + j) * N)
                                             : make_uint2(0, 0);
            }
#pragma unroll
            for (int j = 0; j < BCH; ++j) {
                const float tj = j0 + j < r ? s_t[j0 + j] : 0.0f;
                d0 = fmaf(tj, bf16_lo(bv[j].x), d0);
                d1 = fmaf(tj, bf16_hi(bv[j].x), d1);
                d2 = fmaf(tj, bf16_lo(bv[j].y), d2);
                d3 = fmaf(tj, bf16_hi(bv[j].y), d3);
            }
            if (more) {
#pragma unroll
                for (int j = 0; j < BCH; ++j) bv[j] = nb[j];
            }
        }
        const float sc = lo.scale[a];
        acc.x = fmaf(sc, d0, acc.x); acc.y = fmaf(sc, d1, acc.y);
        acc.z = fmaf(sc, d2, acc.z); acc.w = fmaf(sc, d3, acc.w);
    }
    if (!col_ok) return;
    if constexpr (YF32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + (size_t)m * N + n) = acc;
    } else {
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + (size_t)m * N + n) =
            make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    }
}

// The decode reduction for batches of 129-256 rows (t comes from the segment-path shrink's
// chunk sums; the rows arrive grouped by adapter).  Work item = up to
// kSubRows consecutive positions of one adapter's segment (a quarter of a segment tile) x
// kSegCols columns; base-only positions form items of their own.  Each 16-rank-row chunk of
// the adapter's B slice is loaded once per item and applied to every row of it, so B is read
// once per item instead of once per row, and unpacked once for all its rows.  Per row the
// arithmetic is reduce_lora_kernel's: the split partials added in split order, t summed over
// the chunks in chunk order, d the fmaf chain over rank rows in ascending order (chunks of
// 16, zero terms past the rank), one fmaf with the scale, one rounding; so both kernels give
// the same bits.  Two columns per thread keep a rank-64 item's FMA chain (4 rows x 2 columns
// x 64 per lane) short.
// Items are numbered densely: the tiles cover the LoRA positions in order, so tile t holds
// (first position of tile t + 1, or the LoRA row count) - (its first position) rows and
// ceil(rows / 4) items; every block reads all tiles at once and finds its own by a scan.
// Block y takes item y; the grid is sized for the most items a batch of M rows and n
// adapters can have, and blocks past the batch's count exit after that first round.
constexpr int kSubRows = 4;
constexpr int kSegCpt = 2;               // columns per thread
constexpr int kSegCols = 256 * kSegCpt;  // columns per item
constexpr int kSegMaxTiles = 512;        // tiles a block scans (lora_max_tiles at M <= 256)
template <int RM, bool YF32, int MS, bool PADRM>
__global__ __launch_bounds__(256) void reduce_seg_kernel(const float *__restrict__ partial,
                                                         int M, int N, int n_tm, int n_tn,
                                                         int bm_log2, int n_splits,
                                                         int max_tiles, DecodeLora lo, Seg seg,
                                                         void *__restrict__ y) {
    constexpr int SUB = kSubRows;
    constexpr int TPT = kSegMaxTiles / 256;  // tiles per thread in the scan
    static_assert(SUB * RM <= 256, "one thread per (row, rank column) sums t");
    static_assert(kSegCpt == 2, "two columns per thread");
    __shared__ int s_p0[kSegMaxTiles + 1];
    __shared__ int s_wave[4];
    __shared__ int s_own[3];  // tile, first item of that tile, adapter
    __shared__ __attribute__((aligned(16))) float s_t[SUB][RM];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    // round 1: meta and every tile's (first position, adapter)
    // (clamped: the counts index this block's LDS)
    const int n_tiles = min(max(seg.meta[3], 0), max_tiles);
    const int lora_rows = min(max(seg.meta[1], 0), M);
    int2 te[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int t = tid * TPT + u;
        te[u] = t < max_tiles ? reinterpret_cast<const int2 *>(seg.tiles)[t] : make_int2(0, 0);
    }
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int t = tid * TPT + u;
        if (t < n_tiles) s_p0[t] = te[u].x;
    }
    if (tid == 0) s_p0[n_tiles] = lora_rows;
    __syncthreads();
    int nsub[TPT], mine = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int t = tid * TPT + u;
        nsub[u] = t < n_tiles ? (s_p0[t + 1] - te[u].x + SUB - 1) / SUB : 0;
        mine += nsub[u];
    }
    // exclusive scan of the item counts over threads (tiles in order)
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
    }
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    int before = incl - mine, n_sub = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int c = s_wave[w];
        if (w < wv) before += c;
        n_sub += c;
    }
    const int item = blockIdx.y;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        if (item >= before && item < before + nsub[u]) {
            s_own[0] = tid * TPT + u;
            s_own[1] = before;
            s_own[2] = te[u].y;
        }
        before += nsub[u];
    }
    const int n_items = n_sub + (M - lora_rows + SUB - 1) / SUB;
    if (item >= n_items) return;  // uniform in the block
    __syncthreads();
    int p0, nr, a;
    // (a tile naming no adapter of the pool, possible only in segments a caller built, adds
    // nothing: its rows keep the base output)
    const bool has = item < n_sub && s_own[2] >= 0 && s_own[2] < lo.n_adapters;
    if (item < n_sub) {
        const int t = s_own[0];
        p0 = s_p0[t] + SUB * (item - s_own[1]);
        nr = max(min(SUB, s_p0[t + 1] - p0), 1);
        a = has ? s_own[2] : 0;
    } else {
        p0 = lora_rows + SUB * (item - n_sub);
        nr = min(SUB, M - p0);
        a = 0;
    }
    int m[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) m[i] = seg.perm[min(max(p0 + min(i, nr - 1), 0), M - 1)];

    const int n = (blockIdx.x * 256 + tid) * kSegCpt;
    const bool col_ok = n < N;  // N % 4 == 0: a thread's pair is all in or all out
    const int nc = col_ok ? n : 0;
    const int bm = 1 << bm_log2;
    const size_t stride = (size_t)n_tm * n_tn * bm * kBN;  // one split of the partial tiles
    const float *pp[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        const int tile = (m[i] >> bm_log2) + (nc / kBN) * n_tm;
        pp[i] = partial + (size_t)tile * bm * kBN + (m[i] & (bm - 1)) * kBN + (nc % kBN);
    }
    const int width = PADRM || lo.roff ? RM : lo.pstride;
    int r = !has ? 0 : lo.ranks ? min(max(lo.ranks[a], 1), width) : width;
    const int row0 = PADRM ? a * RM : adapter_row0(lo.roff, lo.pool_rows, a, lo.pstride, r);
    const uint16_t *bp = lo.B + (size_t)row0 * N + nc;

    // Issued together: every row's split partials (up to eight splits), the first TB chunk
    // sums of t (thread (i, j) of the first SUB x RM reads column j of row i; columns at or
    // beyond the rank are not read and stay zero) and the first two 16-row chunks of B.
    constexpr bool EARLY = MS <= 8;
    float2 pv[EARLY ? SUB : 1][EARLY ? MS : 1];
    if constexpr (EARLY) {
#pragma unroll
        for (int i = 0; i < SUB; ++i)
#pragma unroll
            for (int sp = 0; sp < MS; ++sp)
                if (sp < n_splits) pv[i][sp] = *reinterpret_cast<const float2 *>(pp[i] + sp * stride);
    }
    constexpr int TB = 32;
    const int ti = tid / RM, tj = tid % RM;
    const bool tmine = has && tid < SUB * RM && tj < r;
    const float *ts = lo.tpart + (size_t)seg.perm[min(max(p0 + min(ti, nr - 1), 0), M - 1)] * RM + tj;
    const size_t cs = (size_t)M * RM;
    float tv[TB];
#pragma unroll
    for (int c = 0; c < TB; ++c) tv[c] = tmine && c < lo.n_chunks ? ts[c * cs] : 0.0f;

    constexpr int BCH = RM <= 16 ? RM : 16;
    constexpr int NCH = RM / BCH;
    uint32_t bq[NCH][BCH];
    // a padded pool at r_max <= 16 holds every row (the padding rows exist): loaded without
    // waiting for the rank; otherwise rows at or beyond it are zeros, not loads
#define SEG_LOAD_CHUNK(CI)                                                                        \
    do {                                                                                          \
        if (RM <= 16 && PADRM) {                                                                  \
            _Pragma("unroll") for (int j = 0; j < BCH; ++j) bq[CI][j] =                           \
                *reinterpret_cast<const uint32_t *>(bp + (size_t)((CI) * BCH + j) * N);           \
        } else {                                                                                  \
            _Pragma("unroll") for (int j = 0; j < BCH; ++j) bq[CI][j] =                           \
                (CI) * BCH + j < r ? *reinterpret_cast<const uint32_t *>(bp + (size_t)((CI) * BCH + j) * N) \
                                   : 0u;                                                          \
        }                                                                                         \
    } while (0)
#pragma unroll
    for (int c = 0; c < (NCH < 2 ? NCH : 2); ++c)
        if (c * BCH < r) SEG_LOAD_CHUNK(c);

    float2 acc[SUB];
    if constexpr (EARLY) {
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            acc[i] = pv[i][0];
#pragma unroll
            for (int sp = 1; sp < MS; ++sp) {
                if (sp < n_splits) { acc[i].x += pv[i][sp].x; acc[i].y += pv[i][sp].y; }
            }
        }
    }
    // t[m_i, j] = sum over the shrink's chunks, in chunk order (zero at or beyond the rank)
    if (has) {
        float t = 0.0f;
        if (tmine) {
#pragma unroll
            for (int c = 0; c < TB; ++c)
                if (c < lo.n_chunks) t += tv[c];
            for (int c0 = TB; c0 < lo.n_chunks; c0 += 8) {
                float v[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) v[c] = c0 + c < lo.n_chunks ? ts[(c0 + c) * cs] : 0.0f;
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    if (c0 + c < lo.n_chunks) t += v[c];
            }
        }
        if (tid < SUB * RM) s_t[ti][tj] = t;
        __syncthreads();
    }

    // d[i] = sum over rank rows j (ascending, in chunks of 16; zero terms past the rank) of
    // t[m_i, j] B_a[j, cols]; chunk c + 2 is loaded while chunk c is multiplied
    float d[SUB][2];
#pragma unroll
    for (int i = 0; i < SUB; ++i) d[i][0] = d[i][1] = 0.0f;
    if (has) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int j0 = c * BCH;
            if (j0 >= r) break;
            if (c + 2 < NCH && j0 + 2 * BCH < r) SEG_LOAD_CHUNK(c + 2);
#pragma unroll
            for (int j = 0; j < BCH; ++j) {
                const float b0 = bf16_lo(bq[c][j]), b1 = bf16_hi(bq[c][j]);
#pragma unroll
                for (int i = 0; i < SUB; ++i) {
                    const float tt = s_t[i][j0 + j];
                    d[i][0] = fmaf(tt, b0, d[i][0]);
                    d[i][1] = fmaf(tt, b1, d[i][1]);
                }
            }
        }
    }
#undef SEG_LOAD_CHUNK
    const float sc = has ? lo.scale[a] : 0.0f;
    if constexpr (!EARLY) {
        // more than eight splits: every row's partials, issued together once B is no longer
        // held, then added in split order
        float2 pr[SUB][MS];
#pragma unroll
        for (int i = 0; i < SUB; ++i)
#pragma unroll
            for (int sp = 0; sp < MS; ++sp)
                if (sp < n_splits) pr[i][sp] = *reinterpret_cast<const float2 *>(pp[i] + sp * stride);
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            acc[i] = pr[i][0];
#pragma unroll
            for (int sp = 1; sp < MS; ++sp) {
                if (sp < n_splits) { acc[i].x += pr[i][sp].x; acc[i].y += pr[i][sp].y; }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        float2 o = acc[i];
        if (has) {
            o.x = fmaf(sc, d[i][0], o.x);
            o.y = fmaf(sc, d[i][1], o.y);
        }
        if (!col_ok || i >= nr) continue;
        if constexpr (YF32) {
            *reinterpret_cast<float2 *>(reinterpret_cast<float *>(y) + (size_t)m[i] * N + n) = o;
        } else {
            *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(y) + (size_t)m[i] * N + n) =
                pack_bf16x2(o.x, o.y);
        }
    }
}

struct DecPlan {
    int bm, n_tm, n_tn, n_lt, ks, k_per_split;  // ks splits of K per tile
};

// Adapter tiles of a fused call (0 when the call has none).
int adapter_tiles(int M, int r_max, int n_adapters) {
    const int apt = kBN / r_max;
    const int slots = n_adapters < M ? n_adapters : M;
    return (slots + apt - 1) / apt;
}

// Splits of K per tile so that tiles x splits fills the 256 CUs once (at most 16 splits).
DecPlan dec_plan(int M, int K, int N, int n_lt) {
    DecPlan p;
    p.bm = M <= 32 ? 32 : 64;
    p.n_tm = (M + p.bm - 1) / p.bm;
    p.n_tn = (N + kBN - 1) / kBN;
    p.n_lt = n_lt;
    const long tiles = (long)p.n_tm * (p.n_tn + n_lt);
    const int kq = (K + kBKW * kWaves - 1) / (kBKW * kWaves);  // 64-deep quanta (a step per wave)
    int ks = (int)(256 / tiles);
    if (ks < 1) ks = 1;
    if (ks > kq) ks = kq;
    if (ks > 16) ks = 16;
    const int q_per = (kq + ks - 1) / ks;
    p.k_per_split = q_per * kBKW * kWaves;
    p.ks = (K + p.k_per_split - 1) / p.k_per_split;  // <= ks <= 16, what the reduction adds
    return p;
}

bool rank_ok(int r_max) { return r_max == 8 || r_max == 16 || r_max == 32 || r_max == 64; }

}  // namespace

bool decode_gemm_supported(int M, int K, int N) {
    return M >= 1 && M <= kDecodeGemmMaxRows && K % 32 == 0 && K >= 128 && N >= 8 &&
           N % 4 == 0;
}

bool decode_fused_supported(int M, int K, int N) {
    return decode_gemm_supported(M, K, N) && M <= kDecodeMaxRows;
}

size_t decode_gemm_partial_floats(int M, int K, int N, int r_max, int n_adapters) {
    if (!decode_gemm_supported(M, K, N)) return 0;
    // every plan a call of these sizes may run: without adapter tiles (batches of 129-256
    // rows, rank-compact pools, strides that are not a rank bucket, the fp8 base), and with
    // them (the fused small-batch path); the latter has more tiles but may have fewer splits
    const DecPlan p0 = dec_plan(M, K, N, 0);
    size_t f = (size_t)p0.ks * p0.n_tm * p0.n_tn * p0.bm * kBN;
    // (adapter slots r_max wide, the fp8 base's, or fused_tile_rank(r_max) wide, the bf16's)
    if (rank_ok(r_max) && decode_fused_supported(M, K, N)) {
        for (const int rs : {r_max, fused_tile_rank(r_max)}) {
            const DecPlan p = dec_plan(M, K, N, adapter_tiles(M, rs, n_adapters));
            const size_t fa = (size_t)p.ks * p.n_tm * (p.n_tn + p.n_lt) * p.bm * kBN;
            if (fa > f) f = fa;
        }
    }
    return f;
}

hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, const uint16_t *A, int M,
                              int K, int N, const DecodeLora &lo, bool adapters, float *partial,
                              const SegBuild *build, hipStream_t s) {
    if (!decode_gemm_supported(M, K, N) || partial == nullptr || !rank_ok(lo.r_max) ||
        (adapters && (M > kDecodeMaxRows || A == nullptr || lo.ids == nullptr ||
                      (lo.roff == nullptr && (lo.pstride % 8 != 0 || lo.pstride < 8 ||
                                              lo.pstride > lo.r_max)))))
        return hipErrorInvalidValue;
    const int n_lt = adapters ? adapter_tiles(M, lo.r_max, lo.n_adapters) : 0;
    const DecPlan p = dec_plan(M, K, N, n_lt);
    if (build && (build->ids == nullptr || build->n_adapters < 1 || build->n_adapters > LORA_MAX_ADAPTERS))
        return hipErrorInvalidValue;
    const int n_gemm = p.n_tm * (p.n_tn + p.n_lt) * p.ks;
    const dim3 grid(n_gemm + (build ? 1 : 0));
    const SegBuild bld = build ? *build : SegBuild{nullptr, 1, Seg{}};
    // adapter tiles whose adapters' rows are not r_max wide (a rank-compact pool, or a padded
    // pool of another stride) read each adapter at its own row stride
    const bool cpt = adapters && (lo.roff != nullptr || lo.pstride != lo.r_max);
#define GEMM_LAUNCH(BM, RMX)                                                                  \
    if (build)                                                                                \
        launch((decode_gemm_kernel<Dec<BM>, RMX, true, false>), grid, dim3(kThreads), 0, s, x, W, \
               A, M, K, N, p.n_tm, p.n_tn, p.n_lt, p.k_per_split, partial, lo, n_gemm, bld);   \
    else if (cpt)                                                                             \
        launch((decode_gemm_kernel<Dec<BM>, RMX, false, true>), grid, dim3(kThreads), 0, s, x, W, \
               A, M, K, N, p.n_tm, p.n_tn, p.n_lt, p.k_per_split, partial, lo, n_gemm, bld);   \
    else                                                                                      \
        launch((decode_gemm_kernel<Dec<BM>, RMX, false, false>), grid, dim3(kThreads), 0, s, x,  \
               W, A, M, K, N, p.n_tm, p.n_tn, p.n_lt, p.k_per_split, partial, lo, n_gemm, bld)
#define GEMM_RANK(BM)                                                                         \
    switch (lo.r_max) {                                                                       \
        case 8: GEMM_LAUNCH(BM, 8); break;                                                    \
        case 16: GEMM_LAUNCH(BM, 16); break;                                                  \
        case 32: GEMM_LAUNCH(BM, 32); break;                                                  \
        default: GEMM_LAUNCH(BM, 64); break;                                                  \
    }
    if (p.bm == 32) {
        GEMM_RANK(32)
    } else {
        GEMM_RANK(64)
    }
#undef GEMM_RANK
#undef GEMM_LAUNCH
    return hipGetLastError();
}

hipError_t launch_decode_gemm_fp8(const uint16_t *x, const uint8_t *W8, const float *w_scale,
                                  int M, int K, int N, float *partial, const SegBuild *build,
                                  hipStream_t s) {
    if (!decode_gemm_supported(M, K, N) || N % 8 != 0 || partial == nullptr || w_scale == nullptr)
        return hipErrorInvalidValue;
    if (build && (build->ids == nullptr || build->n_adapters < 1 || build->n_adapters > LORA_MAX_ADAPTERS))
        return hipErrorInvalidValue;
    const DecPlan p = dec_plan(M, K, N, 0);
    const int n_gemm = p.n_tm * p.n_tn * p.ks;
    const dim3 grid(n_gemm + (build ? 1 : 0));
    const SegBuild bld = build ? *build : SegBuild{nullptr, 1, Seg{}};
#define F8_LAUNCH(BM)                                                                          \
    if (build)                                                                                 \
        launch((decode_gemm_fp8_kernel<DecF8<BM>, true>), grid, dim3(kThreads), 0, s, x, W8,     \
               w_scale, M, K, N, p.n_tm, p.n_tn, p.k_per_split, partial, n_gemm, bld);          \
    else                                                                                       \
        launch((decode_gemm_fp8_kernel<DecF8<BM>, false>), grid, dim3(kThreads), 0, s, x, W8,    \
               w_scale, M, K, N, p.n_tm, p.n_tn, p.k_per_split, partial, n_gemm, bld)
    if (p.bm == 32) {
        F8_LAUNCH(32);
    } else {
        F8_LAUNCH(64);
    }
#undef F8_LAUNCH
    return hipGetLastError();
}

hipError_t launch_decode_gemm_fp8_lora(const uint16_t *x, const uint8_t *W8, const float *w_scale,
                                       const uint16_t *A, int M, int K, int N,
                                       const DecodeLora &lo, float *partial, hipStream_t s) {
    if (!decode_fused_supported(M, K, N) || N % 8 != 0 || partial == nullptr ||
        w_scale == nullptr || A == nullptr || lo.ids == nullptr || !rank_ok(lo.r_max) ||
        lo.n_adapters < 1)
        return hipErrorInvalidValue;
    const int n_lt = adapter_tiles(M, lo.r_max, lo.n_adapters);
    const DecPlan p = dec_plan(M, K, N, n_lt);
    const int n_gemm = p.n_tm * (p.n_tn + n_lt) * p.ks;
#define F8L_ONE(BM, RMX)                                                                        \
    launch((decode_gemm_fp8_lora_kernel<DecF8<BM>, Dec<BM>, RMX>), dim3(n_gemm), dim3(kThreads), \
           0, s, x, W8, w_scale, A, M, K, N, p.n_tm, p.n_tn, n_lt, p.k_per_split, partial, lo,   \
           n_gemm)
#define F8L_RANK(BM)                                                                            \
    switch (lo.r_max) {                                                                         \
        case 8: F8L_ONE(BM, 8); break;                                                          \
        case 16: F8L_ONE(BM, 16); break;                                                        \
        case 32: F8L_ONE(BM, 32); break;                                                        \
        default: F8L_ONE(BM, 64); break;                                                        \
    }
    if (p.bm == 32) {
        F8L_RANK(32)
    } else {
        F8L_RANK(64)
    }
#undef F8L_RANK
#undef F8L_ONE
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const float *partial, int M, int K, int N, void *y, bool y_f32,
                                const DecodeLora &lo, bool adapters, const Seg *seg,
                                hipStream_t s) {
    if (!decode_gemm_supported(M, K, N) || partial == nullptr || !rank_ok(lo.r_max) ||
        (!adapters && (lo.tpart == nullptr || lo.n_chunks < 1)))
        return hipErrorInvalidValue;
    const int n_lt = adapters ? adapter_tiles(M, lo.r_max, lo.n_adapters) : 0;
    const DecPlan p = dec_plan(M, K, N, n_lt);
    const bool padrm = lo.roff == nullptr && lo.pstride == lo.r_max;
    // (at most kDecodeMaxRows rows the rows of an adapter are too few to share B; there the
    // row kernel's shorter chain wins)
    if (!adapters && seg != nullptr && M > kDecodeMaxRows &&
        lora_max_tiles(M, lo.n_adapters) <= kSegMaxTiles) {
        // one block per (item, kSegCols columns), as many items as a batch of M rows and
        // n adapters can have
        const int max_tiles = lora_max_tiles(M, lo.n_adapters);
        const int n_cc = (N + kSegCols - 1) / kSegCols;
        const int n_seg = M < lo.n_adapters ? M : lo.n_adapters;
        // sum over segments of ceil(rows / 4), plus ceil(base rows / 4), is at most
        // (M + 3 (segments + 1)) / 4
        const long max_items = ((long)M + 3L * n_seg + 6) / kSubRows;
        const dim3 sgrid((unsigned)n_cc, (unsigned)max_items);
        const int bl = p.bm == 32 ? 5 : 6;
#define SEG_ONE(RMX, YF, MSX)                                                                   \
    if (padrm)                                                                                  \
        launch((reduce_seg_kernel<RMX, YF, MSX, true>), sgrid, dim3(256), 0, s, partial, M, N,  \
               p.n_tm, p.n_tn, bl, p.ks, max_tiles, lo, *seg, y);                                \
    else                                                                                        \
        launch((reduce_seg_kernel<RMX, YF, MSX, false>), sgrid, dim3(256), 0, s, partial, M, N, \
               p.n_tm, p.n_tn, bl, p.ks, max_tiles, lo, *seg, y)
#define SEG_LAUNCH(RMX, YF)                                                                     \
    if (p.ks <= 2) {                                                                            \
        SEG_ONE(RMX, YF, 2);                                                                    \
    } else if (p.ks <= 4) {                                                                     \
        SEG_ONE(RMX, YF, 4);                                                                    \
    } else if (p.ks <= 8) {                                                                     \
        SEG_ONE(RMX, YF, 8);                                                                    \
    } else {                                                                                    \
        SEG_ONE(RMX, YF, 16);                                                                   \
    }
#define SEG_RANK(YF)                                                                            \
    switch (lo.r_max) {                                                                         \
        case 8: SEG_LAUNCH(8, YF); break;                                                       \
        case 16: SEG_LAUNCH(16, YF); break;                                                     \
        case 32: SEG_LAUNCH(32, YF); break;                                                     \
        default: SEG_LAUNCH(64, YF); break;                                                     \
    }
        if (y_f32) { SEG_RANK(true) } else { SEG_RANK(false) }
#undef SEG_RANK
#undef SEG_LAUNCH
#undef SEG_ONE
        return hipGetLastError();
    }
    const dim3 rgrid((unsigned)((N + 1023) / 1024), (unsigned)M);
#define RED_ONE(BM, RMX, YF, MSX)                                                           \
    if (padrm)                                                                              \
        launch((reduce_lora_kernel<BM, RMX, YF, MSX, true>), rgrid, dim3(256), 0, s, partial, M,\
               N, p.n_tm, p.n_tn, p.n_lt, p.ks, lo, y);                                      \
    else                                                                                    \
        launch((reduce_lora_kernel<BM, RMX, YF, MSX, false>), rgrid, dim3(256), 0, s, partial, \
               M, N, p.n_tm, p.n_tn, p.n_lt, p.ks, lo, y)
#define RED_LAUNCH(BM, RMX, YF)                                                             \
    if (p.ks <= 4) {                                                                        \
        RED_ONE(BM, RMX, YF, 4);                                                            \
    } else {                                                                                \
        RED_ONE(BM, RMX, YF, 16);                                                           \
    }
#define RED_RANK(BM, YF)                                                                    \
    switch (lo.r_max) {                                                                     \
        case 8: RED_LAUNCH(BM, 8, YF); break;                                               \
        case 16: RED_LAUNCH(BM, 16, YF); break;                                             \
        case 32: RED_LAUNCH(BM, 32, YF); break;                                             \
        default: RED_LAUNCH(BM, 64, YF); break;                                             \
    }
    if (p.bm == 32) {
        if (y_f32) { RED_RANK(32, true) } else { RED_RANK(32, false) }
    } else {
        if (y_f32) { RED_RANK(64, true) } else { RED_RANK(64, false) }
    }
#undef RED_RANK
#undef RED_LAUNCH
#undef RED_ONE
    return hipGetLastError();
}

}  // namespace lora

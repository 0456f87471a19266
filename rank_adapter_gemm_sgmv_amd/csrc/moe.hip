// moe.hip -- MoE-LoRA: a routed expert layer in which every expert carries the batch's
// adapters, as two launches (an expert-routed split-K GEMM with the shrink folded in as extra
// column tiles, then one reduction with the expand and the routing weight).
//
// Source: "Multi-LoRA Serving: Sharing One GPU Across Adapters" (cloudai.pt), "MoE Models
// Raise the Bar" (each adapted projection of each expert has its own low-rank pair; the
// adapter's shrink and expand are folded into the expert-routed kernel, with split-K for the
// skinny products); the layer: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU"
// (dev.to), "Why can't you just merge LoRA weights into the base model?".
//
//   y[m][j][:] = topk_w[m][j] * ( x[m] W[e] + scale_i (x[m] A[i][e]) B[i][e] )
//   with e = topk_ids[m][j] (no expert, -1: a zero row) and i = ids[m] (-1: no adapter term).
//
// gfx950 design, for decode batches (a few (token, slot) pairs per expert; W of every
// routed expert is read once from HBM, which is the bound).
//  * moe_gemm_kernel, workgroup (K split, expert e, column tile).  It finds its expert's
//    pairs itself -- ballots over topk_ids, in pair order, into LDS -- so no routing launch
//    precedes it; a workgroup whose expert has no pair ends at once.  Column tiles
//    0 .. n_tn-1 stream 128 columns of W[e] over the split's K through the per-wave
//    direct-load ring of decode_tiles.h, the x row of each pair gathered per lane.  Column
//    tiles n_tn .. are adapter tiles: the distinct adapters of the expert's pairs (ascending
//    id, found with an LDS bitmap), 128 / RM of them side by side, each A[i][e] streamed the
//    same way -- the shrink runs at the rate of W in the same launch and every touched
//    A[i][e] is read once.  Pairs are taken in blocks of BM rows; a block writes
//    partial[split][pair][column] (W tiles) or tpart[split][pair][0 .. RM) (adapter tiles,
//    each pair only its own adapter's columns).
//  * moe_reduce_kernel, block (column chunk, pair): the splits added in order, t summed over
//    the splits in order, scale_i t B[i][e] added, the routing weight applied, rounded once
//    into y.  No atomics: results do not depend on scheduling.
#include "decode_tiles.h"

namespace lora {

namespace {

constexpr int kBitWords = LORA_MAX_ADAPTERS / 32;

// The expert's pairs (pair order) and, in adapter tiles, the bitmap of their adapters.
struct MoeShared {
    uint16_t rows[LORA_MOE_MAX_PAIRS];
    uint32_t bits[kBitWords];
    int32_t wpre[kBitWords];  // set bits in the words before each word
    int32_t tile_ad[16];      // this adapter tile's adapters (-1: none)
    int32_t wc[kWaves];
};

__device__ __forceinline__ int moe_slot(const MoeShared &sh, int i) {
    const int w = i >> 5;
    return sh.wpre[w] + __popc(sh.bits[w] & ((1u << (i & 31)) - 1u));
}

template <class C, int RM>
__global__ __launch_bounds__(kThreads) void moe_gemm_kernel(MoeGemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint4 lds[kWaves * C::WAVE];
    __shared__ MoeShared sh;
    constexpr int APT = AdapterTiles<RM>::APT;
    static_assert(APT <= 16, "tile_ad holds the adapters of one tile");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_cols = a.n_tn + a.n_lt;
    const int lin = blockIdx.x;
    const int ct = lin % n_cols;
    const int e = (lin / n_cols) % a.E;
    const int split = lin / (n_cols * a.E);
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));

    // 1. this expert's pairs, in pair order (count is uniform in the workgroup)
    int count = 0;
    for (int p0 = 0; p0 < a.P; p0 += kThreads) {
        const int p = p0 + tid;
        const bool hit = p < a.P && a.topk_ids[p] == e;
        const uint64_t bal = __ballot(hit);
        if (lane == 0) sh.wc[wave] = __popcll(bal);
        __syncthreads();
        int base = count, tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = sh.wc[w];
            base += w < wave ? c : 0;
            tot += c;
        }
        if (hit) sh.rows[base + __popcll(bal & below)] = (uint16_t)p;
        count += tot;
        __syncthreads();  // wc is rewritten by the next round; rows complete after the last
    }
    if (count == 0) return;  // whole workgroup

    // 2. adapter tiles: the expert's adapters, ascending, and this tile's share of them
    const bool adapter_tile = ct >= a.n_tn;
    const int lt = ct - a.n_tn;
    if (adapter_tile) {
        const int nw = (a.n_adapters + 31) >> 5;  // <= kBitWords = 2 kThreads
        for (int w = tid; w < nw; w += kThreads) sh.bits[w] = 0u;
        __syncthreads();
        for (int j = tid; j < count; j += kThreads) {
            const int i = a.ids[sh.rows[j] / a.top_k];
            if (i >= 0 && i < a.n_adapters) atomicOr(&sh.bits[i >> 5], 1u << (i & 31));
        }
        __syncthreads();
        const int w0 = 2 * tid;
        const int c0 = w0 < nw ? __popc(sh.bits[w0]) : 0;
        const int c1 = w0 + 1 < nw ? __popc(sh.bits[w0 + 1]) : 0;
        int v = c0 + c1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(v, d, 64);
            if (lane >= d) v += u;
        }
        if (lane == 63) sh.wc[wave] = v;
        __syncthreads();
        int wb = 0, T = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = sh.wc[w];
            wb += w < wave ? c : 0;
            T += c;
        }
        const int excl = wb + v - c0 - c1;
        if (w0 < nw) sh.wpre[w0] = excl;
        if (w0 + 1 < nw) sh.wpre[w0 + 1] = excl + c0;
        if (lt * APT >= T) return;  // no adapter of this expert in this tile (whole workgroup)
        __syncthreads();
        if (tid < APT) {
            const int s = lt * APT + tid;
            int ad = -1;
            if (s < T) {
                // the word holding slot s: the last word whose prefix is <= s
                int lo = 0, hi = nw - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (sh.wpre[mid] <= s) lo = mid;
                    else hi = mid - 1;
                }
                uint32_t bw = sh.bits[lo];
                for (int k = s - sh.wpre[lo]; k > 0; --k) bw &= bw - 1u;
                ad = 32 * lo + __ffs(bw) - 1;
            }
            sh.tile_ad[tid] = ad;
        }
        __syncthreads();
    }

    // 3. per-lane sources: W[e] (row stride N), or the tile's A[i][e] (row stride r_stride);
    //    direct load q of a W stage: lane l fills position l % 16 of row 4 q + l / 16
    DecSrc<C> src;
    size_t ldw;
    const int n0 = ct * kBN;
    if (!adapter_tile) {
        const uint16_t *We = a.W + (size_t)e * a.K * a.N;
#pragma unroll
        for (int q = 0; q < C::WINS; ++q) {
            const int r = 4 * q + (lane >> 4);
            const int lc = (lane & 15) ^ wsw(r);
            src.wp[q] = We + (size_t)r * a.N + min(n0 + lc * 8, a.N - 8);
        }
        ldw = (size_t)a.N;
    } else {
#pragma unroll
        for (int q = 0; q < C::WINS; ++q) {
            const int r = 4 * q + (lane >> 4);
            const int col = ((lane & 15) ^ wsw(r)) * 8;
            int ad = sh.tile_ad[col / RM];
            if (ad < 0) ad = sh.tile_ad[0];  // an empty slot reads a valid adapter, unused
            int cc = col % RM;
            if (cc >= a.r_stride) cc = 0;     // bucket columns past r_max: unused
            src.wp[q] = a.A + (((size_t)ad * a.E + e) * a.K + r) * a.r_stride + cc;
        }
        ldw = (size_t)a.r_stride;
    }

    const int ks0 = split * a.k_per_split;
    const int ks1 = min(a.K, ks0 + a.k_per_split);
    const int per_wave = a.k_per_split / kWaves;  // multiple of 16
    const int kw0 = min(ks1, ks0 + wave * per_wave);
    const int kw1 = min(ks1, kw0 + per_wave);
    const int nst = (kw1 - kw0) / kBKW;
    const int n_rb = (count + C::BM - 1) / C::BM;
    const int col = tid & 127;

    for (int rb = 0; rb < n_rb; ++rb) {
        // x load q of an x stage: lane l fills position l % 8 of row 8 q + l / 8 (chunk
        // (l % 8) ^ (l / 8)); rows past the expert's last pair repeat it
#pragma unroll
        for (int q = 0; q < C::XINS; ++q) {
            const int row = 8 * q + (lane >> 3);
            const int lc = (lane & 7) ^ (lane >> 3);
            const int p = sh.rows[min(rb * C::BM + row, count - 1)];
            src.xp[q] = a.x + (size_t)(p / a.top_k) * a.K + lc * 8;
        }
        f32x16_t acc[C::TM][C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        dec_kloop<C>(acc, src, lds + wave * C::WAVE, kw0, nst, a.K, ldw, lane);
        wait_vm<0>();     // the ring's last loads have landed
        __syncthreads();  // every wave is done with its stages

        float4 *const red = reinterpret_cast<float4 *>(lds);
        reduce_waves_put<C>(acc, red + wave * (C::TILE / 4), lane);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < C::BM / 8; ++q) {
            const int g = (tid >> 7) + 2 * q;  // rows 4 g .. 4 g + 3 of the block
            const float4 s = reduce_waves_group<C>(red, g, col);
            const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int j = rb * C::BM + 4 * g + v;
                if (j >= count) continue;
                const int p = sh.rows[j];
                if (!adapter_tile) {
                    a.partial[((size_t)split * a.P + p) * a.np + n0 + col] = sv[v];
                } else {
                    const int i = a.ids[p / a.top_k];
                    if (i < 0 || i >= a.n_adapters) continue;
                    const int sl = moe_slot(sh, i) - lt * APT;
                    if (sl == col / RM) a.tpart[((size_t)split * a.P + p) * RM + col % RM] = sv[v];
                }
            }
        }
        __syncthreads();  // the next block's ring overwrites red
    }
}

// y[p, n .. n+3] = topk_w[p] * ( sum over splits of partial[s][p][n ..]
//                               + scale_i sum_{j < rank_i} t[p, j] B[i][e][j][n ..] )
// t[p, j] = sum over splits of tpart[s][p][j]; e = topk_ids[p], i = ids[p / top_k].  Block
// (column chunk of 1024, pair p), 256 threads x 4 columns.  MS: the most splits (4 or 16).
template <int RM, bool YF32, int MS>
__global__ __launch_bounds__(256) void moe_reduce_kernel(MoeReduceArgs a) {
    __shared__ float s_t[RM];
    const int p = blockIdx.y;
    const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
    const bool col_ok = n < a.N;
    const int nc = col_ok ? n : 0;
    const int e = a.topk_ids[p];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (e >= 0 && e < a.E) {  // uniform in the block
        const int i = a.ids[p / a.top_k];
        const bool has = i >= 0 && i < a.n_adapters;
        float4 pv[MS];
#pragma unroll
        for (int sp = 0; sp < MS; ++sp)
            if (sp < a.ks)
                pv[sp] = *reinterpret_cast<const float4 *>(a.partial + ((size_t)sp * a.P + p) * a.np + nc);
        int r = 0;
        const uint16_t *bp = nullptr;
        if (has) {
            r = a.ranks ? min(max(a.ranks[i], 0), a.r_stride) : a.r_stride;
            bp = a.B + ((size_t)i * a.E + e) * a.r_stride * a.N + nc;
        }
        constexpr int BCH = RM <= 16 ? RM : 16;
        uint2 bv[BCH];
#pragma unroll
        for (int j = 0; j < BCH; ++j)
            bv[j] = j < r ? *reinterpret_cast<const uint2 *>(bp + (size_t)j * a.N) : make_uint2(0, 0);
        if (has && threadIdx.x < RM) {
            float t = 0.0f;
            for (int sp = 0; sp < a.ks; ++sp) t += a.tpart[((size_t)sp * a.P + p) * RM + threadIdx.x];
            s_t[threadIdx.x] = t;
        }
        __syncthreads();
        acc = pv[0];
#pragma unroll
        for (int sp = 1; sp < MS; ++sp) {
            if (sp < a.ks) {
                acc.x += pv[sp].x; acc.y += pv[sp].y; acc.z += pv[sp].z; acc.w += pv[sp].w;
            }
        }
        if (has) {
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
            for (int j0 = 0; j0 < RM; j0 += BCH) {
                if (j0 >= r) break;
                if (j0 > 0) {
#pragma unroll
                    for (int j = 0; j < BCH; ++j)
                        bv[j] = j0 + j < r ? *reinterpret_cast<const uint2 *>(bp + (size_t)(j0 + j) * a.N)
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
            }
            const float sc = a.scale[i];
            acc.x = fmaf(sc, d0, acc.x); acc.y = fmaf(sc, d1, acc.y);
            acc.z = fmaf(sc, d2, acc.z); acc.w = fmaf(sc, d3, acc.w);
        }
        if (a.topk_w) {
            const float w = a.topk_w[p];
            acc.x *= w; acc.y *= w; acc.z *= w; acc.w *= w;
        }
    }
    if (!col_ok) return;
    if constexpr (YF32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.y) + (size_t)p * a.N + n) = acc;
    } else {
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.y) + (size_t)p * a.N + n) =
            make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    }
}

}  // namespace

MoePlan moe_plan(int M, int top_k, int E, int K, int N, int r_max, int n_adapters) {
    MoePlan p;
    const int P = M * top_k;
    p.rm = rank_bucket(r_max);
    p.bm = 32;
    p.n_tn = (N + kBN - 1) / kBN;
    p.np = p.n_tn * kBN;
    const int apt = kBN / p.rm;
    const int distinct = n_adapters < M ? n_adapters : M;  // adapters per expert at most
    p.n_lt = (distinct + apt - 1) / apt;
    // splits of K so that the W tiles of the experts that can be routed to fill the chip
    // about twice (at most 16 splits, each a multiple of 64 deep)
    const long active = (long)(E < P ? E : P) * p.n_tn;
    int ks = (int)((512 + active - 1) / active);
    const int kq = (K + kBKW * kWaves - 1) / (kBKW * kWaves);
    if (ks < 1) ks = 1;
    if (ks > 16) ks = 16;
    if (ks > kq) ks = kq;
    p.k_per_split = (kq + ks - 1) / ks * kBKW * kWaves;
    p.ks = (K + p.k_per_split - 1) / p.k_per_split;
    return p;
}

size_t moe_partial_floats(const MoePlan &p, int P) { return (size_t)p.ks * P * p.np; }
size_t moe_tpart_floats(const MoePlan &p, int P) { return (size_t)p.ks * P * p.rm; }

hipError_t launch_moe_gemm(const MoePlan &p, const MoeGemmArgs &args, hipStream_t s) {
    if (args.P < 1 || args.P > LORA_MOE_MAX_PAIRS || args.K % 32 != 0 || args.K < 128 ||
        args.N < 8 || args.N % 8 != 0 || args.r_stride % 8 != 0 || args.r_stride > p.rm ||
        args.n_adapters > LORA_MAX_ADAPTERS || p.bm != 32)
        return hipErrorInvalidValue;
    MoeGemmArgs a = args;
    a.n_tn = p.n_tn;
    a.n_lt = p.n_lt;
    a.k_per_split = p.k_per_split;
    a.np = p.np;
    const dim3 grid((unsigned)((long)p.ks * a.E * (p.n_tn + p.n_lt)));
    switch (p.rm) {
        case 8: launch(moe_gemm_kernel<Dec<32>, 8>, grid, dim3(kThreads), 0, s, a); break;
        case 16: launch(moe_gemm_kernel<Dec<32>, 16>, grid, dim3(kThreads), 0, s, a); break;
        case 32: launch(moe_gemm_kernel<Dec<32>, 32>, grid, dim3(kThreads), 0, s, a); break;
        default: launch(moe_gemm_kernel<Dec<32>, 64>, grid, dim3(kThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_moe_reduce(const MoePlan &p, const MoeReduceArgs &args, bool y_f32,
                             hipStream_t s) {
    if (args.P < 1 || args.N % 4 != 0 || args.r_stride > p.rm || p.ks < 1 || p.ks > 16)
        return hipErrorInvalidValue;
    MoeReduceArgs a = args;
    a.ks = p.ks;
    a.np = p.np;
    const dim3 grid((unsigned)((a.N + 1023) / 1024), (unsigned)a.P);
#define MOE_RED(RMX, YF)                                                                      \
    if (p.ks <= 4) launch(moe_reduce_kernel<RMX, YF, 4>, grid, dim3(256), 0, s, a);           \
    else launch(moe_reduce_kernel<RMX, YF, 16>, grid, dim3(256), 0, s, a)
#define MOE_RANK(YF)                                                                          \
    switch (p.rm) {                                                                           \
        case 8: MOE_RED(8, YF); break;                                                        \
        case 16: MOE_RED(16, YF); break;                                                      \
        case 32: MOE_RED(32, YF); break;                                                      \
        default: MOE_RED(64, YF); break;                                                      \
    }
    if (y_f32) {
        MOE_RANK(true)
    } else {
        MOE_RANK(false)
    }
#undef MOE_RANK
#undef MOE_RED
    return hipGetLastError();
}

}  // namespace lora

// decode_gemm.hip -- y = x W + (x A_i) B_i * scale_i for small (decode) batches: the shared
// GEMM streamed from HBM with the LoRA expand as one more K split, then an ordered split-K
// reduction.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Why can't you
// just merge LoRA weights into the base model?" (the layer; x W is one GEMM over the batch)
// and "How does one batch run 30 different adapters at once?" (at decode every request adds
// one row, and the cost is the weight bytes read from HBM); "Multi-LoRA Serving: Sharing One
// GPU Across Adapters" (cloudai.pt), "MoE Models Raise the Bar" (split-K for skinny products,
// the expand step).
//
// gfx950 design.  With one row per request, x W is bound by reading W once from HBM.
// Needs the shrink's chunk sums of t (decode_shrink.hip); groups the rows by adapter itself.
//  * Output tile = BM rows (all of a small batch) x 64 columns; the K range of each tile is
//    split over `ksplit` workgroups, and inside a workgroup over its four waves.  Each wave
//    streams its own K sub-range through its own 4-stage LDS ring filled by direct
//    global->LDS loads, so the K loop has no workgroup barrier at all: only this wave's
//    s_waitcnt orders its loads and reads.  Three stages (24 KiB per wave) are in flight.
//  * x tile [BM][32] and W tile [32][64] per stage, XOR-swizzled as in the large GEMM; the
//    W operand is read with the transposing LDS read (ds_read_b64_tr_b16).
//  * The LoRA expand is one more split of each tile: the K-extension [x | s t] [W ; B_a].
//    Its k runs over (adapter of the batch, rank), its W rows are the stacked B_a rows of
//    the batch's adapters (streamed once per column tile by the same DMA ring), and its x
//    rows hold scale_a * t[m, :] for the rows of adapter a and zero elsewhere.  So every
//    touched B_a is read from HBM once, and the delta lands in the same fp32 sums as x W.
//  * The four waves' partial tiles are added through LDS in wave order and each workgroup
//    writes its partial tile; a second small kernel adds the partials in split order and
//    rounds once into y, so the result does not depend on scheduling.
#include "batch_adapters.h"

namespace lora {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kBN = 64;
constexpr int kBK = 32;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int BM_>
struct Dec {
    static constexpr int BM = BM_;
    static constexpr int TM = BM / 32, TN = kBN / 32;
    static constexpr int XSLOT = BM * kBK * 2 / 16;  // uint4 per wave per stage (x)
    static constexpr int WSLOT = kBK * kBN * 2 / 16; // uint4 per wave per stage (W)
    static constexpr int XINS = XSLOT / 64;          // DMA instructions per wave per stage
    static constexpr int WINS = WSLOT / 64;
    static constexpr int PER = XINS + WINS;
    static constexpr int TILE = BM * kBN;             // floats per tile
    static_assert(BM == 32 || BM == 64, "decode tile rows");
    static_assert(TILE <= kWaves * WSLOT * 4, "a wave's partial tile fits one W stage array");
};

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// W tile rows are 128 bytes (8 chunks of 16 bytes); chunk c of row r is stored at
// c ^ (4 ((r / 2) % 2)), so the 4 rows x 32 bytes of one transposing read of 16 lanes, and
// the two 16-lane groups read together, fall on distinct banks.
__device__ __forceinline__ int wsw(int r) { return ((r >> 1) & 1) << 2; }

template <class C>
__device__ __forceinline__ void dec_mfma(f32x16_t (&acc)[C::TM][C::TN], const uint4 *__restrict__ xs,
                                         const uint4 *__restrict__ ws, int lane) {
    const lds_char_t *wsb = (const lds_char_t *)(ws);
    const int g = lane >> 4, li = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t af[C::TM], bfr[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int row = 32 * i + (lane & 31);
            const int lc = 2 * kk + (lane >> 5);
            af[i] = *reinterpret_cast<const bf16x8_t *>(&xs[row * 4 + (lc ^ ((row >> 2) & 3))]);
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = 32 * j + 16 * (g & 1) + 4 * (li & 3);
            const int lc = col >> 3, half = (col >> 2) & 1;
            const int r = 16 * kk + 8 * (g >> 1) + (li >> 2);
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
}

template <class C>
struct DecSrc {
    const uint16_t *xp[C::XINS];
    const uint16_t *wp[C::WINS];
};

// One stage of this wave: x[rows][k0 .. k0+31] and W[k0 .. k0+31][tile columns].
template <class C>
__device__ __forceinline__ void dec_issue(const DecSrc<C> &src, uint4 *__restrict__ xslot,
                                          uint4 *__restrict__ wslot, int k0, int N) {
#pragma unroll
    for (int q = 0; q < C::XINS; ++q)
        __builtin_amdgcn_global_load_lds((const void *)(src.xp[q] + k0), (lds_void_t *)&xslot[q * 64], 16, 0, 0);
#pragma unroll
    for (int q = 0; q < C::WINS; ++q)
        __builtin_amdgcn_global_load_lds((const void *)(src.wp[q] + (size_t)k0 * N), (lds_void_t *)&wslot[q * 64], 16, 0, 0);
}

// Cross-wave reduction: each wave's accumulators go to LDS (accumulator layout, lane-minor)
// and are added in wave order into row-major elements; thread tid owns rows tid/64 + 4q
// and column tid % 64.
template <class C>
__device__ __forceinline__ void reduce_waves(const f32x16_t (&acc)[C::TM][C::TN], float *red_mine,
                                             const float *r0, const float *r1, const float *r2,
                                             const float *r3, int lane, int wave,
                                             float (&sum)[C::BM / 4]) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) red_mine[((i * C::TN + j) * 16 + v) * 64 + lane] = acc[i][j][v];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < C::BM / 4; ++q) {
        const int r = wave + 4 * q, c = lane;
        const int i = r >> 5, rr = r & 31, j = c >> 5, cc = c & 31;
        const int e = ((i * C::TN + j) * 16 + (rr >> 3) * 4 + (rr & 3)) * 64 + ((rr >> 2) & 1) * 32 + cc;
        sum[q] = ((r0[e] + r1[e]) + r2[e]) + r3[e];
    }
}

// Workgroup (tile, split).  Splits 0 .. ks_base-1 cover K; split ks_base (the extension
// split) multiplies the LoRA K-extension [s t] [B stacked over the batch's adapters]: its
// k runs over (adapter slot s, rank j), its x rows hold scale_a * t[m, j] for the rows m of
// the slot's adapter a (zero for other rows) and its W rows are B_a[j, tile columns].
// Each split writes its partial tile; reduce_partials_kernel adds them in split order.
template <class C>
__global__ __launch_bounds__(kThreads) void decode_gemm_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ W, int M, int K, int N, int n_tm,
    int n_tn, int ks_base, int k_per_split, float *__restrict__ partial, DecodeLora lo) {
    // stage s of wave w: X{s}[w * XSLOT ..], W{s}[w * WSLOT ..]
    __shared__ __attribute__((aligned(1024))) uint4 XS0[kWaves * C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 XS1[kWaves * C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 XS2[kWaves * C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 XS3[kWaves * C::XSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 WS0[kWaves * C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 WS1[kWaves * C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 WS2[kWaves * C::WSLOT];
    __shared__ __attribute__((aligned(1024))) uint4 WS3[kWaves * C::WSLOT];
    // extension split only: the batch's adapters, and t / scale / slot of the tile's rows
    __shared__ BatchAdapters ba;
    __shared__ __attribute__((aligned(16))) float s_t[C::BM * 64];
    __shared__ float s_scale[C::BM];
    __shared__ int32_t s_slot[C::BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_tiles = n_tm * n_tn;
    // block -> (tile, split): the splits of one tile are n_tiles apart
    const int tile = blockIdx.x % n_tiles, split = blockIdx.x / n_tiles;
    const int tm = tile % n_tm, tn = tile / n_tm;
    const int m0 = tm * C::BM, n0 = tn * kBN;
    const bool ext = split == ks_base;

    DecSrc<C> src;
#pragma unroll
    for (int q = 0; q < C::XINS; ++q) {
        const int row = 16 * q + (lane >> 2);
        const int lc = (lane & 3) ^ ((lane >> 4) & 3);
        const int m = min(m0 + row, M - 1);
        src.xp[q] = x + (size_t)m * K + lc * 8;
    }
    int wrow[C::WINS], wcol[C::WINS];
#pragma unroll
    for (int q = 0; q < C::WINS; ++q) {
        const int r = 8 * q + (lane >> 3);
        const int lc = (lane & 7) ^ wsw(r);
        wrow[q] = r;
        wcol[q] = min(n0 + lc * 8, N - 8);
        src.wp[q] = W + (size_t)r * N + wcol[q];
    }

    f32x16_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const int xo = wave * C::XSLOT, wo = wave * C::WSLOT;

    if (!ext) {
        // ---- base term: this wave's part of the split's K range --------------------------
        const int ks0 = split * k_per_split;
        const int ks1 = min(K, ks0 + k_per_split);
        const int per_wave = k_per_split / kWaves;  // multiple of 32
        const int kw0 = min(ks1, ks0 + wave * per_wave);
        const int kw1 = min(ks1, kw0 + per_wave);
        const int nst = (kw1 - kw0) / kBK;
        // k of stage s (stages past the last reload the last one; an empty range loads k=0)
#define KLOAD(S) (nst > 0 ? kw0 + min((S), nst - 1) * kBK : 0)
        dec_issue<C>(src, XS0 + xo, WS0 + wo, KLOAD(0), N);
        dec_issue<C>(src, XS1 + xo, WS1 + wo, KLOAD(1), N);
        dec_issue<C>(src, XS2 + xo, WS2 + wo, KLOAD(2), N);
#define DEC_STEP(SS, XC, WC, XN, WN)                                   \
        wait_vm<2 * C::PER>();                                         \
        wait_lgkm0();                                                  \
        dec_issue<C>(src, XN + xo, WN + wo, KLOAD((SS) + 3), N);       \
        if ((SS) < nst) dec_mfma<C>(acc, XC + xo, WC + wo, lane);
        for (int s = 0; s < nst; s += 4) {
            DEC_STEP(s, XS0, WS0, XS3, WS3)
            DEC_STEP(s + 1, XS1, WS1, XS0, WS0)
            DEC_STEP(s + 2, XS2, WS2, XS1, WS1)
            DEC_STEP(s + 3, XS3, WS3, XS2, WS2)
        }
#undef DEC_STEP
#undef KLOAD
        wait_vm<0>();
    } else {
        // ---- LoRA K-extension -------------------------------------------------------------
        const int RM = lo.r_max;
        const int lr = 31 - __clz(RM);  // r_max is a power of two
        batch_adapters(ba, lo.ids, M, lo.n_adapters);
        const int T = ba.T;
        for (int r = tid; r < C::BM; r += kThreads) {
            const int m = m0 + r;
            const int sl = m < M ? ba.slot[m] : -1;
            s_slot[r] = sl;
            s_scale[r] = sl >= 0 ? lo.scale[ba.id[m]] : 0.0f;
        }
        // t of the tile's rows: the shrink's chunk sums added in chunk order
        for (int cq = tid; cq < C::BM * (RM / 4); cq += kThreads) {
            const int r = cq / (RM / 4), j = (cq % (RM / 4)) * 4;
            const int m = m0 + r;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m < M && ba.slot[m] >= 0) {
                const float *tp = lo.tpart + (size_t)m * RM + j;
                const size_t cs = (size_t)M * RM;
                for (int c0 = 0; c0 < lo.n_chunks; c0 += 8) {  // 8 loads in flight, added in order
                    float4 u[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        u[i] = c0 + i < lo.n_chunks ? *reinterpret_cast<const float4 *>(tp + (c0 + i) * cs)
                                                    : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        v.x += u[i].x; v.y += u[i].y; v.z += u[i].z; v.w += u[i].w;
                    }
                }
            }
            *reinterpret_cast<float4 *>(&s_t[r * RM + j]) = v;
        }
        __syncthreads();
        const int ES = (T * RM + kBK - 1) / kBK;  // extension steps
        const int pe = (ES + kWaves - 1) / kWaves;
        const int e0 = wave * pe;
        const int nst = max(0, min(ES, e0 + pe) - e0);
        // W rows of extension step e: stacked row k = 32 e + r -> (adapter slot s, rank j)
        auto issue_ext = [&](uint4 *__restrict__ xslot, uint4 *__restrict__ wslot, int step) {
            const int e = e0 + (nst > 0 ? min(step, nst - 1) : 0);
#pragma unroll
            for (int q = 0; q < C::XINS; ++q)  // placeholder x (overwritten before use)
                __builtin_amdgcn_global_load_lds((const void *)src.xp[q], (lds_void_t *)&xslot[q * 64], 16, 0, 0);
#pragma unroll
            for (int q = 0; q < C::WINS; ++q) {
                const int k = e * kBK + wrow[q];
                const int sl = k >> lr, j = k & (RM - 1);
                const int a = sl < T ? ba.list[sl] : 0;
                const uint16_t *p = lo.B + ((size_t)a * RM + j) * N + wcol[q];
                __builtin_amdgcn_global_load_lds((const void *)p, (lds_void_t *)&wslot[q * 64], 16, 0, 0);
            }
        };
        // x rows of extension step e: scale_a * t[m, j .. j+7] where the row's adapter is the
        // step's adapter slot, else zero
        auto fill_ext = [&](uint4 *__restrict__ xslot, int step) {
            const int e = e0 + step;
#pragma unroll
            for (int i = 0; i < C::BM * 4 / 64; ++i) {
                const int c = lane + 64 * i;
                const int row = c >> 2, lc = c & 3;
                const int k = e * kBK + lc * 8;
                const int sl = k >> lr, j = k & (RM - 1);
                uint4 v = make_uint4(0, 0, 0, 0);
                if (sl < T && s_slot[row] == sl) {
                    const float sc = s_scale[row];
                    const float4 t0 = *reinterpret_cast<const float4 *>(&s_t[row * RM + j]);
                    const float4 t1 = *reinterpret_cast<const float4 *>(&s_t[row * RM + j + 4]);
                    v = make_uint4(pack_bf16x2(sc * t0.x, sc * t0.y), pack_bf16x2(sc * t0.z, sc * t0.w),
                                   pack_bf16x2(sc * t1.x, sc * t1.y), pack_bf16x2(sc * t1.z, sc * t1.w));
                }
                xslot[row * 4 + (lc ^ ((row >> 2) & 3))] = v;
            }
        };
        issue_ext(XS0 + xo, WS0 + wo, 0);
        issue_ext(XS1 + xo, WS1 + wo, 1);
        issue_ext(XS2 + xo, WS2 + wo, 2);
#define EXT_STEP(SS, XC, WC, XN, WN)                                   \
        wait_vm<2 * C::PER>();                                         \
        wait_lgkm0();                                                  \
        issue_ext(XN + xo, WN + wo, (SS) + 3);                         \
        if ((SS) < nst) {                                              \
            fill_ext(XC + xo, (SS));                                   \
            dec_mfma<C>(acc, XC + xo, WC + wo, lane);                  \
        }
        for (int s = 0; s < nst; s += 4) {
            EXT_STEP(s, XS0, WS0, XS3, WS3)
            EXT_STEP(s + 1, XS1, WS1, XS0, WS0)
            EXT_STEP(s + 2, XS2, WS2, XS1, WS1)
            EXT_STEP(s + 3, XS3, WS3, XS2, WS2)
        }
#undef EXT_STEP
        wait_vm<0>();
    }
    __syncthreads();

    float sum[C::BM / 4];
    float *red = reinterpret_cast<float *>(wave == 0 ? WS0 : wave == 1 ? WS1 : wave == 2 ? WS2 : WS3);
    reduce_waves<C>(acc, red, reinterpret_cast<const float *>(WS0), reinterpret_cast<const float *>(WS1),
                    reinterpret_cast<const float *>(WS2), reinterpret_cast<const float *>(WS3), lane,
                    wave, sum);
    float *mine = partial + ((size_t)split * n_tiles + tile) * C::TILE;
#pragma unroll
    for (int q = 0; q < C::BM / 4; ++q) mine[(wave + 4 * q) * kBN + lane] = sum[q];
}

// y[m][n] = sum over splits (in order) of the partial tiles; 4 columns per thread.
template <int BM, bool YF32>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ partial,
                                                              int M, int N, int n_tm, int n_tn,
                                                              int n_splits, void *__restrict__ y) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int nq = (N + 3) / 4;
    if (idx >= (long)M * nq) return;
    const int m = (int)(idx / nq), n = (int)(idx % nq) * 4;
    const int tile = (m / BM) + (n / kBN) * n_tm;
    const int off = (m % BM) * kBN + (n % kBN);
    const size_t stride = (size_t)n_tm * n_tn * BM * kBN;
    const float *p = partial + (size_t)tile * BM * kBN + off;
    float4 acc = *reinterpret_cast<const float4 *>(p);
    for (int sp = 1; sp < n_splits; ++sp) {
        const float4 v = *reinterpret_cast<const float4 *>(p + sp * stride);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if constexpr (YF32) {
        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + (size_t)m * N + n) = acc;
    } else {
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + (size_t)m * N + n) =
            make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    }
}

struct DecPlan {
    int bm, n_tm, n_tn, ks_base, k_per_split;
};

// ks_base splits of K per tile plus the extension split, aiming at one workgroup per CU.
DecPlan dec_plan(int M, int K, int N) {
    DecPlan p;
    p.bm = M <= 32 ? 32 : 64;
    p.n_tm = (M + p.bm - 1) / p.bm;
    p.n_tn = (N + kBN - 1) / kBN;
    const long tiles = (long)p.n_tm * p.n_tn;
    const int kq = K / (kBK * kWaves);  // whole 128-deep quanta
    int ks = (int)(256 / tiles) - 1;
    if (ks < 1) ks = 1;
    if (ks > kq) ks = kq > 0 ? kq : 1;
    if (ks > 16) ks = 16;
    const int q_per = (kq + ks - 1) / ks;
    p.k_per_split = (q_per > 0 ? q_per : 1) * kBK * kWaves;
    p.ks_base = (K + p.k_per_split - 1) / p.k_per_split;
    return p;
}

}  // namespace

bool decode_gemm_supported(int M, int K, int N) {
    return M >= 1 && M <= kDecodeMaxRows && K % kBK == 0 && K >= kBK * kWaves && N >= 8 && N % 4 == 0;
}

size_t decode_gemm_partial_floats(int M, int K, int N) {
    if (!decode_gemm_supported(M, K, N)) return 0;
    const DecPlan p = dec_plan(M, K, N);
    return (size_t)(p.ks_base + 1) * p.n_tm * p.n_tn * p.bm * kBN;
}

hipError_t launch_decode_gemm(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y,
                              bool y_f32, const DecodeLora &lo, float *partial, hipStream_t s) {
    if (!decode_gemm_supported(M, K, N) || partial == nullptr || lo.tpart == nullptr)
        return hipErrorInvalidValue;
    const DecPlan p = dec_plan(M, K, N);
    const int n_tiles = p.n_tm * p.n_tn;
    const dim3 grid(n_tiles * (p.ks_base + 1));
    if (p.bm == 32)
        launch((decode_gemm_kernel<Dec<32>>), grid, dim3(kThreads), 0, s, x, W, M, K, N,
                           p.n_tm, p.n_tn, p.ks_base, p.k_per_split, partial, lo);
    else
        launch((decode_gemm_kernel<Dec<64>>), grid, dim3(kThreads), 0, s, x, W, M, K, N,
                           p.n_tm, p.n_tn, p.ks_base, p.k_per_split, partial, lo);
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const float *partial, int M, int K, int N, void *y, bool y_f32,
                                hipStream_t s) {
    if (!decode_gemm_supported(M, K, N) || partial == nullptr) return hipErrorInvalidValue;
    const DecPlan p = dec_plan(M, K, N);
    const long threads = (long)M * ((N + 3) / 4);
    const dim3 rgrid((unsigned)((threads + 255) / 256));
#define RED_LAUNCH(BM, YF)                                                                     \
    launch((reduce_partials_kernel<BM, YF>), rgrid, dim3(256), 0, s, partial, M, N, \
                       p.n_tm, p.n_tn, p.ks_base + 1, y)
    if (p.bm == 32) {
        if (y_f32) RED_LAUNCH(32, true); else RED_LAUNCH(32, false);
    } else {
        if (y_f32) RED_LAUNCH(64, true); else RED_LAUNCH(64, false);
    }
#undef RED_LAUNCH
    return hipGetLastError();
}

}  // namespace lora

// gemm.hip -- the shared base term y = x W on bf16 MFMA (gfx950) for the decode shapes no
// other GEMM of the library takes (split-K tilings), and the dispatch between the GEMMs.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Why can't you
// just merge LoRA weights into the base model?": the x W term is one big GEMM across the
// whole batch; "How does one batch run 30 different adapters at once?": prefill is
// compute-bound and the delta is small next to x W.
//
// Operands: x[M][K] (K contiguous) and W[K][N] (N contiguous), bf16.  The gfx950 MFMA
// v_mfma_f32_32x32x16_bf16 takes, per lane, 8 consecutive-k values of one row of the left
// operand and 8 consecutive-k values of one column of the right operand.  x tiles go to LDS
// as they are ([row][k]).  W tiles are loaded as 8x8 blocks (8 k rows x 16 bytes), transposed
// in registers with byte permutes and stored to LDS as [n][k], so both operands are read
// from LDS with one 16-byte read per lane per MFMA.  LDS rows are padded by 16 bytes.
//
// Pipeline: LDS double buffer, one barrier per 64-deep k step; the global loads of step
// k+1 are in flight while step k's MFMAs run.
//
// Tilings: 64 x 64, 128 x 64 or 128 x 128 with split-K partial sums reduced by a second
// kernel in split order.  Tiles are mapped XCD-aware: workgroup b runs on XCD b % 8, so
// each XCD is handed compact groups of 4 tile rows and its L2 serves the x and W panels those
// tiles share (without it, the row tiles of a decode W panel land on four XCDs and W is
// fetched from HBM about four times).

#include "common.h"

namespace lora {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;  // LDS row length in bf16 (16-byte pad)

// 8x8 bf16 transpose: in[kk] = 8 consecutive n at row kk (4 dwords, low half = even n);
// out[nn] = 8 consecutive k at column nn.
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
    const uint32_t *r = reinterpret_cast<const uint32_t *>(in);
    uint32_t *o = reinterpret_cast<uint32_t *>(out);
#pragma unroll
    for (int p = 0; p < 4; ++p) {      // dword p of a row holds columns 2p, 2p+1
#pragma unroll
        for (int q = 0; q < 4; ++q) {  // dword q of a column holds rows 2q, 2q+1
            const uint32_t lo = r[(2 * q) * 4 + p], hi = r[(2 * q + 1) * 4 + p];
            o[(2 * p) * 4 + q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);      // even column
            o[(2 * p + 1) * 4 + q] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // odd column
        }
    }
}

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int XCH = BM * (kBK / 8) / NT;           // x 16-byte chunks per thread
    static constexpr int WBL = (kBK / 8) * (BN / 8);          // 8x8 W blocks per tile
    static constexpr int WB = (WBL + NT - 1) / NT;            // W blocks per thread
    static_assert(TM >= 1 && TN >= 1 && XCH >= 1, "tile shape");
    static_assert(BM * (kBK / 8) % NT == 0, "x chunks must divide evenly");
};

// Tile order: XCD-major, then groups of 4 tile rows, column-major inside a group.
__device__ __forceinline__ void tile_coords(int b, int n_tm, int n_tn, bool xcd_remap, int &tm,
                                            int &tn) {
    const int T = n_tm * n_tn;
    int lin = b;
    if (xcd_remap && (T % 8) == 0) lin = (b % 8) * (T / 8) + b / 8;
    constexpr int G = 4;
    const int group = lin / (G * n_tn);
    const int first = group * G;
    const int gsz = min(n_tm - first, G);
    const int in = lin % (G * n_tn);
    tm = first + in % gsz;
    tn = in / gsz;
}

// One 16-deep MFMA step of a wave's TM x TN block of 32x32 accumulators; operands from LDS.
template <class C>
__device__ __forceinline__ void mfma_step(f32x16_t (&acc)[C::TM][C::TN], const uint16_t *as,
                                          const uint16_t *bs, int wm0, int wn0, int lane, int kk) {
    const int koff = kk * 16 + (lane >> 5) * 8;
    bf16x8_t af[C::TM], bf[C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t *>(&as[(wm0 + i * 32 + (lane & 31)) * kLDK + koff]);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const bf16x8_t *>(&bs[(wn0 + j * 32 + (lane & 31)) * kLDK + koff]);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// Global loads of one 64-deep k step: x chunks (16 bytes) and 8x8 W blocks.
template <class C>
__device__ __forceinline__ void load_tile(uint4 (&xr)[C::XCH], uint4 (&wr)[C::WB][8],
                                          const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ W, const int (&xrow)[C::XCH],
                                          int tid, int k0, int kz1, int K, int N, int n0) {
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
        const int kc = ((tid + i * C::NT) % (kBK / 8)) * 8;
        xr[i] = (xrow[i] >= 0 && k0 + kc < kz1) ? ld16(x + (size_t)xrow[i] * K + k0 + kc)
                                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::WB; ++j) {
        const int b = tid + j * C::NT;
        const int kb = b % 8, nb = b / 8;
        const int n = n0 + nb * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int k = k0 + kb * 8 + kk;
            wr[j][kk] = (b < C::WBL && n < N && k < kz1) ? ld16(W + (size_t)k * N + n)
                                                         : make_uint4(0, 0, 0, 0);
        }
    }
}

template <class C>
__device__ __forceinline__ void store_tile(const uint4 (&xr)[C::XCH], const uint4 (&wr)[C::WB][8],
                                           uint16_t *as, uint16_t *bs, int tid) {
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
        const int c = tid + i * C::NT;
        st16(&as[(c / (kBK / 8)) * kLDK + (c % (kBK / 8)) * 8], xr[i]);
    }
#pragma unroll
    for (int j = 0; j < C::WB; ++j) {
        const int b = tid + j * C::NT;
        if (b < C::WBL) {
            const int kb = b % 8, nb = b / 8;
            uint4 t8[8];
            transpose8x8(wr[j], t8);
#pragma unroll
            for (int nn = 0; nn < 8; ++nn) st16(&bs[(nb * 8 + nn) * kLDK + kb * 8], t8[nn]);
        }
    }
}

template <class C, bool YF32>
__global__ __launch_bounds__(C::NT) void gemm_kernel(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ W, int M, int K,
                                                     int N, void *__restrict__ y,
                                                     float *__restrict__ partial, int k_per_split,
                                                     int n_tm, int n_tn) {
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kLDK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / C::WN) * C::WTM, wn0 = (wave % C::WN) * C::WTN;

    int tmi, tni;
    tile_coords(blockIdx.x, n_tm, n_tn, true, tmi, tni);
    const int row0 = tmi * BM, n0 = tni * BN;
    const int split = blockIdx.y;
    const int kz0 = split * k_per_split;
    const int kz1 = min(K, kz0 + k_per_split);

    // rows of x this thread loads (fixed over the k loop); -1 = beyond M
    int xrow[C::XCH];
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
        const int rr = row0 + (tid + i * NT) / (kBK / 8);
        int m = -1;
        if (rr < M) m = rr;
        xrow[i] = m;
    }

    uint4 xr[C::XCH];
    uint4 wr[C::WB][8];
    f32x16_t acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = (kz1 - kz0 + kBK - 1) / kBK;
    if (nk > 0) {
        load_tile<C>(xr, wr, x, W, xrow, tid, kz0, kz1, K, N, n0);
        store_tile<C>(xr, wr, As[0], Bs[0], tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tile<C>(xr, wr, x, W, xrow, tid, kz0 + (kt + 1) * kBK, kz1, K, N, n0);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) mfma_step<C>(acc, As[cur], Bs[cur], wm0, wn0, lane, kk);
        if (kt + 1 < nk) store_tile<C>(xr, wr, As[cur ^ 1], Bs[cur ^ 1], tid);
        __syncthreads();
    }

    // store: accumulator register v of a 32x32 block holds row (v/4)*8 + (lane/32)*4 + v%4,
    // column lane%32
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn0 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int rr = row0 + wm0 + i * 32 + (v / 4) * 8 + (lane >> 5) * 4 + (v % 4);
                if (rr < M && col < N) {
                    const int m = rr;
                    const float val = acc[i][j][v];
                    if (partial != nullptr) {
                        partial[((size_t)split * M + m) * N + col] = val;
                    } else if constexpr (YF32) {
                        reinterpret_cast<float *>(y)[(size_t)m * N + col] = val;
                    } else {
                        reinterpret_cast<uint16_t *>(y)[(size_t)m * N + col] = (uint16_t)f32_to_bf16_rne(val);
                    }
                }
            }
        }
    }
}

// y[m][n] = sum over splits (ascending) of partial[split][m][n]; 4 columns per thread.
template <bool YF32>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partial,
                                                            int M, int N, int ksplit,
                                                            void *__restrict__ y) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long total = (long)M * N / 4;
    if (idx >= total) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z = 0; z < ksplit; ++z) {
        const float4 v = reinterpret_cast<const float4 *>(partial + (size_t)z * M * N)[idx];
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    if constexpr (YF32) {
        reinterpret_cast<float4 *>(y)[idx] = acc;
    } else {
        uint2 o = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
        reinterpret_cast<uint2 *>(y)[idx] = o;
    }
}

using CfgD64 = Cfg<64, 64, 2, 2>;
using CfgD128x64 = Cfg<128, 64, 2, 2>;
using CfgD128 = Cfg<128, 128, 2, 2>;

// Decode batches with enough 128 x 128 output tiles to cover every CU use the large-tile
// MFMA kernel (no split-K); smaller ones the split-K tilings below.
bool use_big(int M, int N) { return (long)((M + 127) / 128) * ((N + 127) / 128) >= 256; }

struct DecodePlan {
    int bm, bn, ksplit, k_per_split;
};

DecodePlan decode_plan(int M, int K, int N) {
    DecodePlan p;
    if (M <= 64) { p.bm = 64; p.bn = 64; }
    else if (M <= 256) { p.bm = 128; p.bn = 64; }
    else { p.bm = 128; p.bn = 128; }
    const long tiles = (long)((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
    const int ksteps = (K + kBK - 1) / kBK;
    int ks = (int)((512 + tiles - 1) / tiles);  // aim at about two workgroups per CU
    ks = ks < 1 ? 1 : ks;
    const int max_ks = ksteps / 4 > 0 ? ksteps / 4 : 1;  // at least 4 k steps per split
    if (ks > max_ks) ks = max_ks;
    if (ks > 16) ks = 16;
    const int steps_per = (ksteps + ks - 1) / ks;
    p.k_per_split = steps_per * kBK;
    p.ksplit = (K + p.k_per_split - 1) / p.k_per_split;
    return p;
}

template <class C>
hipError_t launch_cfg(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y, bool y_f32,
                      float *partial, int ksplit, int k_per_split, hipStream_t s) {
    const int n_tm = (M + C::BM - 1) / C::BM, n_tn = (N + C::BN - 1) / C::BN;
    dim3 grid(n_tm * n_tn, ksplit);
    if (y_f32)
        launch((gemm_kernel<C, true>), grid, dim3(C::NT), 0, s, x, W, M, K, N, y, partial,
               k_per_split, n_tm, n_tn);
    else
        launch((gemm_kernel<C, false>), grid, dim3(C::NT), 0, s, x, W, M, K, N, y, partial,
               k_per_split, n_tm, n_tn);
    return hipGetLastError();
}

}  // namespace

size_t gemm_partial_floats(int M, int K, int N) {
    const SkPlan sp = sk_plan(M, K, N);
    if (sp.use) return sk_partial_floats(sp);
    if (use_big(M, N)) return 0;
    const DecodePlan p = decode_plan(M, K, N);
    return p.ksplit > 1 ? (size_t)p.ksplit * M * N : 0;
}

hipError_t launch_gemm(const uint16_t *x, const uint16_t *W, int M, int K, int N, void *y,
                       bool y_f32, bool prefill, Seg seg, const LoraEpilogue *lora,
                       float *ws_partial, size_t ws_partial_floats, int *ksplit_out,
                       hipStream_t s) {
    *ksplit_out = 1;
    if (prefill) return launch_gemm_big(x, W, M, K, N, y, y_f32, seg, lora, s);
    const SkPlan sp = sk_plan(M, K, N);
    if (sp.use) {
        if (sk_partial_floats(sp) > ws_partial_floats || ws_partial == nullptr)
            return hipErrorInvalidValue;
        *ksplit_out = -1;
        SkProj pj{};
        pj.W[0] = W;
        return launch_gemm_sk(x, pj, M, K, N, sp, ws_partial, s);
    }
    if (use_big(M, N)) return launch_gemm_big(x, W, M, K, N, y, y_f32, seg, nullptr, s);

    const DecodePlan p = decode_plan(M, K, N);
    float *partial = nullptr;
    if (p.ksplit > 1) {
        if ((size_t)p.ksplit * M * N > ws_partial_floats || ws_partial == nullptr)
            return hipErrorInvalidValue;
        partial = ws_partial;
    }
    *ksplit_out = p.ksplit;
    if (p.bm == 64)
        return launch_cfg<CfgD64>(x, W, M, K, N, y, y_f32, partial, p.ksplit, p.k_per_split, s);
    if (p.bn == 64)
        return launch_cfg<CfgD128x64>(x, W, M, K, N, y, y_f32, partial, p.ksplit, p.k_per_split, s);
    return launch_cfg<CfgD128>(x, W, M, K, N, y, y_f32, partial, p.ksplit, p.k_per_split, s);
}

hipError_t launch_splitk_reduce(const float *partial, int M, int N, int ksplit, void *y, bool y_f32,
                                hipStream_t s) {
    const long threads = (long)M * N / 4;
    const int grid = (int)((threads + 255) / 256);
    if (y_f32)
        launch(splitk_reduce_kernel<true>, dim3(grid), dim3(256), 0, s, partial, M, N, ksplit, y);
    else
        launch(splitk_reduce_kernel<false>, dim3(grid), dim3(256), 0, s, partial, M, N, ksplit, y);
    return hipGetLastError();
}

}  // namespace lora

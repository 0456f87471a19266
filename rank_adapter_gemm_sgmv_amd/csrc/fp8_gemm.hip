// fp8_gemm.hip -- x W_eff for decode batches whose shared base weight is stored as 8-bit
// floating point: W_eff[k, n] = w_scale[n] * dec(W8[n, k]), with W8 the E4M3 codes of the
// OCP 8-bit floating point format, one fp32 scale per output column.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), "Where does
// multi-LoRA serving actually break?", item 4 (a quantized base served beside higher-precision
// adapters: the delta runs in another type than the base, and the base, the denominator of
// the overhead, gets cheaper), and "How does one batch run 30 different adapters at once?"
// (at decode the cost is the weight bytes read from HBM -- halved here).
//
// gfx950 design.  Only the base GEMM changes; the LoRA delta is the bf16 decode path's
// (segment shrink, then the reduction that adds this kernel's split partials and the expand).
//  * The split plan and partial-tile layout are decode_splits': tile = BM rows x 128 columns,
//    K cut into ks splits so that tiles x splits fills the 256 CUs once; partial tiles
//    [split][tile][BM][128] fp32, already multiplied by the column's scale.
//  * The four waves of a workgroup split the tile's columns (32 each) and share its x: the
//    split's x rows are staged in LDS (up to 512 k at a time; 16-byte chunk c of row r is
//    stored at c ^ (r % 16), so the 16 rows a read serves at once fall on all 64 banks).
//  * Each lane streams the codes of one output column, W8[n, k .. k+31] (two 16-byte loads
//    per 64 k, every 128-byte line of a column consumed by the two halves of one wave in one
//    step), four steps ahead in registers.
//  * Codes become bf16 with v_cvt_scalef32_pk_bf16_fp8 (scale 1: exact, every E4M3 value is a
//    bf16 value) and meet x on v_mfma_f32_32x32x16_bf16.  For a 64-k step, lane half g holds
//    k = 32 g .. 32 g + 31 of its column; MFMA q (0..3) takes k = 32 g + 8 q .. + 7 from both
//    operands, so the four MFMAs cover the 64 k once each.
#include "segments_block.h"

namespace lora {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 128;      // columns of a tile (the decode plan's)
constexpr int kStepK = 64;    // k per streamed step of W8
constexpr int kSlabK = 512;   // k of x staged in LDS at a time
constexpr int kAhead = 4;     // W8 steps in flight per lane
constexpr int kThreads = 256;
constexpr int kBuildLds = (LORA_MAX_ADAPTERS + 1 + 15) / 16 * 64 + 64 * 4 + 64;  // builder tables

template <int BM>
struct Fp8Cfg {
    static constexpr int TM = BM / 32;                         // 32-row MFMA blocks
    static constexpr int SLAB_CHUNKS = kSlabK / 8;             // 16-byte chunks per x row
    static constexpr int SLAB_BYTES = BM * kSlabK * 2;
    static constexpr int LDS16 = (SLAB_BYTES > kBuildLds ? SLAB_BYTES : kBuildLds) / 16;
};

// 8 codes (two dwords) -> 8 bf16
__device__ __forceinline__ bf16x8_t dec8(uint32_t lo, uint32_t hi) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Workgroup (tile, split): rows m0 .. m0 + BM of x, columns n0 .. n0 + 127, k in the split.
// BUILD: one more workgroup (the last) builds the segments instead.
template <int BM, bool BUILD>
__global__ __launch_bounds__(kThreads) void decode_gemm_fp8_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ W8, const float *__restrict__ w_scale,
    int M, int K, int N, int n_tm, int n_tn, int k_per_split, float *__restrict__ partial,
    int n_gemm_blocks, SegBuild build) {
    using C = Fp8Cfg<BM>;
    __shared__ __attribute__((aligned(1024))) uint4 lds[C::LDS16];

    if (BUILD && (int)blockIdx.x >= n_gemm_blocks) {
        int32_t *cnt = reinterpret_cast<int32_t *>(lds);
        int32_t(*wave_tot)[kThreads / 64] =
            reinterpret_cast<int32_t(*)[kThreads / 64]>(cnt + ((build.n_adapters + 1 + 15) & ~15));
        build_segments_block<kThreads>(build.ids, M, build.n_adapters, build.seg, cnt, wave_tot,
                                       &wave_tot[3][0]);
        return;
    }

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_tiles = n_tm * n_tn;
    // block -> (split, tile); with several row tiles, row tile fastest over consecutive blocks
    // of one XCD (workgroup b runs on XCD b % 8), so they read a W8 panel through one L2
    int lin = blockIdx.x;
    if (n_tm > 1 && (n_gemm_blocks & 7) == 0) lin = (blockIdx.x & 7) * (n_gemm_blocks >> 3) + (blockIdx.x >> 3);
    const int tile = lin % n_tiles, split = lin / n_tiles;
    const int tm = tile % n_tm, tn = tile / n_tm;
    const int m0 = tm * BM, n0 = tn * kBN;
    const int ks0 = split * k_per_split, ks1 = min(K, ks0 + k_per_split);
    const int nsteps = (ks1 - ks0) / kStepK;  // K % 64 == 0 and k_per_split % 256 == 0

    // this lane's column (columns past N read the last one; their sums are never used) and
    // half of each 64-k step
    const int col = n0 + 32 * wave + (lane & 31);
    const int g = lane >> 5;
    const uint8_t *wcol = W8 + (size_t)min(col, N - 1) * K + ks0 + 32 * g;

    // W8 ring: step s in slot s % kAhead
    uint4 wr[kAhead][2];
#pragma unroll
    for (int s = 0; s < kAhead; ++s) {
        const int ss = min(s, nsteps - 1);
        wr[s][0] = ld16(wcol + (size_t)ss * kStepK);
        wr[s][1] = ld16(wcol + (size_t)ss * kStepK + 16);
    }

    f32x16_t acc[C::TM];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;

    constexpr int kSlabSteps = kSlabK / kStepK;  // a multiple of kAhead
    for (int sk = 0; sk < nsteps; sk += kSlabSteps) {
        // x[m0 .. m0 + BM, ks0 + sk * 64 .. + 512) into LDS (rows past the batch repeat its
        // last row; k past the split's end is not read by any step)
        const int kx0 = ks0 + sk * kStepK;
        const int kx_len = min(kSlabK, ks1 - kx0);
        __syncthreads();  // the previous slab's reads are done
#pragma unroll 8
        for (int v = tid; v < BM * C::SLAB_CHUNKS; v += kThreads) {
            const int row = v / C::SLAB_CHUNKS, c = v % C::SLAB_CHUNKS;
            const int m = min(m0 + row, M - 1);
            const uint4 val = c * 8 < kx_len ? ld16(x + (size_t)m * K + kx0 + c * 8) : make_uint4(0, 0, 0, 0);
            lds[row * C::SLAB_CHUNKS + (c ^ (row & 15))] = val;
        }
        __syncthreads();
        const int s_end = min(nsteps, sk + kSlabSteps);
        // step s is in ring slot (s - sk) % kAhead = j
#pragma unroll 1
        for (int s0 = sk; s0 < s_end; s0 += kAhead) {
#pragma unroll
            for (int j = 0; j < kAhead; ++j) {
                const int s = s0 + j;
                if (s < s_end) {
                    const uint4 w0 = wr[j][0], w1 = wr[j][1];
                    // refill the slot with step s + kAhead (steps past the last reload the last)
                    const int sn = min(s + kAhead, nsteps - 1);
                    wr[j][0] = ld16(wcol + (size_t)sn * kStepK);
                    wr[j][1] = ld16(wcol + (size_t)sn * kStepK + 16);
                    const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
                    const int kc0 = (s - sk) * (kStepK / 8) + 4 * g;  // this half's first chunk
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bf16x8_t b = dec8(wd[2 * q], wd[2 * q + 1]);
#pragma unroll
                        for (int i = 0; i < C::TM; ++i) {
                            const int row = 32 * i + (lane & 31);
                            const bf16x8_t av = *reinterpret_cast<const bf16x8_t *>(
                                &lds[row * C::SLAB_CHUNKS + ((kc0 + q) ^ (row & 15))]);
                            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[i], 0, 0, 0);
                        }
                    }
                }
            }
        }
    }

    // the scaled partial tile: element v of block i is row 32 i + (v / 4) * 8 + g * 4 + v % 4,
    // column lane % 32 of this wave's 32
    const float sc = w_scale[min(col, N - 1)];
    float *P = partial + ((size_t)split * n_tiles + tile) * BM * kBN + 32 * wave + (lane & 31);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) P[(size_t)(32 * i + (v / 4) * 8 + g * 4 + v % 4) * kBN] = sc * acc[i][v];
}

}  // namespace

hipError_t launch_decode_gemm_fp8(const uint16_t *x, const uint8_t *W8, const float *w_scale,
                                  int M, int K, int N, float *partial, const SegBuild *build,
                                  hipStream_t s) {
    if (M < 1 || M > kDecodeGemmMaxRows || K % kStepK != 0 || K < 128 || N < 8 || N % 8 != 0 ||
        partial == nullptr || w_scale == nullptr)
        return hipErrorInvalidValue;
    if (build && (build->ids == nullptr || build->n_adapters < 1 || build->n_adapters > LORA_MAX_ADAPTERS))
        return hipErrorInvalidValue;
    const DecodeSplits p = decode_splits(M, K, N);
    if (p.k_per_split % kStepK != 0) return hipErrorInvalidValue;
    const int n_gemm = p.n_tm * p.n_tn * p.ks;
    const dim3 grid(n_gemm + (build ? 1 : 0));
    const SegBuild bld = build ? *build : SegBuild{nullptr, 1, Seg{}};
#define FP8_LAUNCH(BM)                                                                         \
    if (build)                                                                                 \
        launch((decode_gemm_fp8_kernel<BM, true>), grid, dim3(kThreads), 0, s, x, W8, w_scale, M, \
               K, N, p.n_tm, p.n_tn, p.k_per_split, partial, n_gemm, bld);                      \
    else                                                                                       \
        launch((decode_gemm_fp8_kernel<BM, false>), grid, dim3(kThreads), 0, s, x, W8, w_scale, M,\
               K, N, p.n_tm, p.n_tn, p.k_per_split, partial, n_gemm, bld)
    if (p.bm == 32) {
        FP8_LAUNCH(32);
    } else {
        FP8_LAUNCH(64);
    }
#undef FP8_LAUNCH
    return hipGetLastError();
}

}  // namespace lora

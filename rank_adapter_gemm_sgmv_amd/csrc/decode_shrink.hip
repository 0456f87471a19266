// decode_shrink.hip -- t = x A_i for a small (decode) batch in one launch, without a
// separate segment-building kernel.
//
// Source: the adapter "shrink" of "Multi-LoRA Serving: Sharing One GPU Across Adapters"
// (cloudai.pt), "MoE Models Raise the Bar" (split-K for these skinny products); the
// [B, 4096] x [4096, r] product of "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU"
// (dev.to), "How does one batch run 30 different adapters at once?", bound by reading the
// adapter weights.
//
// Workgroup (k-chunk c, adapter slot s): the workgroup groups the batch's rows by adapter in
// LDS (batch_adapters.h), takes the s-th distinct adapter a, holds A_a[chunk, 0:r_max] in
// registers (each lane one k-slice x 8 rank columns, 16-byte loads; all r_max columns, the
// pool's padding being zero) and multiplies every row of adapter a with it: 8 fp32 sums per
// lane, then an xor butterfly across the k-slices.  So each touched A_a is read from HBM
// exactly once per batch and untouched adapters cost nothing.  The chunk sums go to
// tpart[c][m][0:r_max] (rows without an adapter are not written); the consumer adds the
// chunks in ascending order.
#include "batch_adapters.h"

namespace lora {

namespace {

constexpr int kThreads = 128;  // 2 waves; >= kDecodeMaxRows for the grouping

template <int RM>
struct ShrinkCfg {
    static constexpr int KC = RM == 64 ? 128 : 256;  // k per chunk
    static constexpr int JG = RM / 8;                // 8-column groups per lane row
    static constexpr int KSUB = 64 / JG;             // k-slices across the lanes of a wave
    static constexpr int SL = KC / KSUB;             // k per slice (4, 8, 16 or 16)
};

template <int RM>
__global__ __launch_bounds__(kThreads) void decode_shrink_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ A, const int32_t *__restrict__ ids,
    const int32_t *__restrict__ ranks, int M, int K, int n_adapters, int n_chunks,
    float *__restrict__ tpart) {
    using C = ShrinkCfg<RM>;
    __shared__ BatchAdapters ba;
    const int c = blockIdx.x % n_chunks, s = blockIdx.x / n_chunks;
    batch_adapters(ba, ids, M, n_adapters);
    if (s >= ba.T) return;  // uniform across the workgroup
    const int a = ba.list[s];
    (void)ranks;  // all r_max columns are read: the pool's padded columns are zero

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ks = lane % C::KSUB, g = lane / C::KSUB;
    const int k0 = c * C::KC + ks * C::SL;

    // A_a[k0 .. k0+SL][8g .. 8g+7] -> registers.  The loads are unconditional (k beyond K
    // reads the last row; those terms are dropped below), so they issue back to back.
    uint4 araw[C::SL];
    const uint16_t *Ap = A + ((size_t)a * K + k0) * RM + g * 8;
    const uint16_t *Alast = A + ((size_t)a * K + (K - 1)) * RM + g * 8;
#pragma unroll
    for (int kk = 0; kk < C::SL; ++kk) araw[kk] = ld16(k0 + kk < K ? Ap + (size_t)kk * RM : Alast);

    // rows of adapter a with row parity == wave, from a ballot mask; the next row's x is
    // loaded while the current one is multiplied
    uint64_t mk0 = __ballot(lane < M && ba.slot[lane] == s && (lane & 1) == wave);
    uint64_t mk1 = __ballot(lane + 64 < M && ba.slot[lane + 64] == s && (lane & 1) == wave);
    auto next_row = [&]() -> int {
        if (mk0) {
            const int b = __ffsll((unsigned long long)mk0) - 1;
            mk0 &= mk0 - 1;
            return b;
        }
        if (mk1) {
            const int b = __ffsll((unsigned long long)mk1) - 1;
            mk1 &= mk1 - 1;
            return b + 64;
        }
        return -1;
    };
    constexpr int XV = C::SL >= 8 ? C::SL / 8 : 1;  // 16-byte x loads per row and lane
    // x[m][k0 ..]: unconditional loads from in-bounds addresses (row 0 for no row, the last
    // k for k beyond K); the terms beyond K are dropped in the sums
    auto load_x = [&](int m, uint4 (&xv)[XV]) {
        const uint16_t *xr = x + (size_t)(m < 0 ? 0 : m) * K;
        if constexpr (C::SL >= 8) {
#pragma unroll
            for (int v = 0; v < XV; ++v) xv[v] = ld16(xr + min(k0 + 8 * v, K - 8));
        } else {  // 4 k per slice: one 8-byte load
            const uint2 h = *reinterpret_cast<const uint2 *>(xr + min(k0, K - 4));
            xv[0] = make_uint4(h.x, h.y, 0, 0);
        }
    };
    int m = next_row();
    uint4 xc[XV];
    load_x(m, xc);
    while (m >= 0) {
        const int mn = next_row();
        uint4 xn[XV];
        load_x(mn, xn);
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            float xf[8];
            unpack8(xc[v], xf);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (8 * v + u < C::SL && k0 + 8 * v + u < K) {
                    float av[8];
                    unpack8(araw[8 * v + u], av);
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[j] = fmaf(xf[u], av[j], acc[j]);
                }
            }
        }
#pragma unroll
        for (int off = 1; off < C::KSUB; off <<= 1) {
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] += __shfl_xor(acc[j], off, 64);
        }
        if (ks == 0) {
            float *dst = tpart + ((size_t)c * M + m) * RM + g * 8;
            *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        }
        m = mn;
#pragma unroll
        for (int v = 0; v < XV; ++v) xc[v] = xn[v];
    }
}

}  // namespace

int decode_shrink_chunks(int K, int r_max) {
    const int kc = r_max == 64 ? 128 : 256;
    return (K + kc - 1) / kc;
}

hipError_t launch_decode_shrink(const uint16_t *x, const uint16_t *A, const int32_t *ids,
                                const int32_t *ranks, int M, int K, int r_max, int n_adapters,
                                float *tpart, hipStream_t s) {
    if (M < 1 || M > kDecodeMaxRows) return hipErrorInvalidValue;
    const int n_chunks = decode_shrink_chunks(K, r_max);
    const int slots = M < n_adapters ? M : n_adapters;
    const dim3 grid(n_chunks * slots);
    switch (r_max) {
        case 8:
            launch(decode_shrink_kernel<8>, grid, dim3(kThreads), 0, s, x, A, ids, ranks, M, K, n_adapters, n_chunks, tpart);
            break;
        case 16:
            launch(decode_shrink_kernel<16>, grid, dim3(kThreads), 0, s, x, A, ids, ranks, M, K, n_adapters, n_chunks, tpart);
            break;
        case 32:
            launch(decode_shrink_kernel<32>, grid, dim3(kThreads), 0, s, x, A, ids, ranks, M, K, n_adapters, n_chunks, tpart);
            break;
        case 64:
            launch(decode_shrink_kernel<64>, grid, dim3(kThreads), 0, s, x, A, ids, ranks, M, K, n_adapters, n_chunks, tpart);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace lora

// decode_shrink.h -- the shrink t = x A_i of a small (decode) batch, as work items that the
// decode GEMM's workgroups run before their K loop (no launch of its own).
//
// Source: the adapter "shrink" of "Multi-LoRA Serving: Sharing One GPU Across Adapters"
// (cloudai.pt), "MoE Models Raise the Bar" (split-K for these skinny products); the
// [B, 4096] x [4096, r] product of "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU"
// (dev.to), "How does one batch run 30 different adapters at once?", bound by reading the
// adapter weights.
//
// Work item (k-chunk c, adapter a), taken by a pair of waves: the pair holds
// A_a[chunk, 0:r_max] in registers (each lane one k-slice x 8 rank columns, 16-byte loads;
// all r_max columns, the pool's padding being zero) and multiplies every row of adapter a
// with it -- each wave takes the rows of one parity, given as ballot masks over the batch's
// rows (at most kDecodeMaxRows) -- with 8 fp32 sums per lane and an xor butterfly across
// the k-slices.  The
// caller names the adapters either directly (item = (chunk, adapter id), rows found by a
// ballot over ids) or through the batch's distinct adapters grouped in LDS
// (batch_adapters.h).  So each touched A_a is read from HBM
// exactly once per batch and untouched adapters cost nothing.  The chunk sums go to
// tpart[c][m][0:r_max] (rows without an adapter are not written); the consumer adds the
// chunks in ascending order.
#pragma once

#include "batch_adapters.h"

namespace lora {

template <int RM>
struct DecodeShrinkCfg {
    static constexpr int KC = RM == 64 ? 128 : 256;  // k per chunk
    static constexpr int JG = RM / 8;                // 8-column groups per lane row
    static constexpr int KSUB = 64 / JG;             // k-slices across the lanes of a wave
    static constexpr int SL = KC / KSUB;             // k per slice (4, 8, 16 or 16)
    static constexpr int XV = SL >= 8 ? SL / 8 : 1;  // 16-byte x loads per row and lane
};

inline int decode_shrink_chunk_k(int r_max) { return r_max == 64 ? 128 : 256; }

// Row masks of one wave: bit i of word q is row 64 q + i.
constexpr int kRowWords = kDecodeMaxRows / 64;
struct RowMask {
    uint64_t w[kRowWords];
};

template <int RM>
__device__ __forceinline__ void decode_shrink_item(const uint16_t *__restrict__ x,
                                                   const uint16_t *__restrict__ A, int M, int K,
                                                   int c, int a, RowMask mk, int lane,
                                                   float *__restrict__ tpart) {
    using C = DecodeShrinkCfg<RM>;
    const int ks = lane % C::KSUB, g = lane / C::KSUB;
    const int k0 = c * C::KC + ks * C::SL;

    // A_a[k0 .. k0+SL][8g .. 8g+7] -> registers.  The loads are unconditional (k beyond K
    // reads the last row; those terms are dropped below), so they issue back to back.
    uint4 araw[C::SL];
    const uint16_t *Ap = A + ((size_t)a * K + k0) * RM + g * 8;
    const uint16_t *Alast = A + ((size_t)a * K + (K - 1)) * RM + g * 8;
#pragma unroll
    for (int kk = 0; kk < C::SL; ++kk) araw[kk] = ld16(k0 + kk < K ? Ap + (size_t)kk * RM : Alast);

    // this wave's rows, lowest first; the next row's x is loaded while the current one is
    // multiplied
    auto next_row = [&]() -> int {
#pragma unroll
        for (int q = 0; q < kRowWords; ++q) {
            if (mk.w[q]) {
                const int b = __ffsll((unsigned long long)mk.w[q]) - 1;
                mk.w[q] &= mk.w[q] - 1;
                return b + 64 * q;
            }
        }
        return -1;
    };
    // x[m][k0 ..]: unconditional loads from in-bounds addresses (row 0 for no row, the last
    // k for k beyond K); the terms beyond K are dropped in the sums
    auto load_x = [&](int m, uint4 (&xv)[C::XV]) {
        const uint16_t *xr = x + (size_t)(m < 0 ? 0 : m) * K;
        if constexpr (C::SL >= 8) {
#pragma unroll
            for (int v = 0; v < C::XV; ++v) xv[v] = ld16(xr + min(k0 + 8 * v, K - 8));
        } else {  // 4 k per slice: one 8-byte load
            const uint2 h = *reinterpret_cast<const uint2 *>(xr + min(k0, K - 4));
            xv[0] = make_uint4(h.x, h.y, 0, 0);
        }
    };
    int m = next_row();
    uint4 xc[C::XV];
    load_x(m, xc);
    while (m >= 0) {
        const int mn = next_row();
        uint4 xn[C::XV];
        load_x(mn, xn);
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int v = 0; v < C::XV; ++v) {
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
        for (int v = 0; v < C::XV; ++v) xc[v] = xn[v];
    }
}

}  // namespace lora

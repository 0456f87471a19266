// batch_adapters.h -- the distinct adapters of a small decode batch, found by one
// workgroup in LDS (no separate segment-building launch).
//
// For a batch of at most kDecodeMaxRows rows, every workgroup that needs the grouping of
// rows by adapter recomputes it: adapters are numbered by the first row that uses them
// ("slots" 0 .. T-1), and each row learns its slot.  The numbering depends only on ids, so
// every workgroup of every kernel of a call agrees on it.  Rows with id -1 or an id outside
// [0, n_adapters) get slot -1 (base only).
#pragma once

#include "common.h"

namespace lora {

struct alignas(16) BatchAdapters {
    int32_t id[kDecodeMaxRows];     // row -> valid adapter id, or -1
    int32_t slot[kDecodeMaxRows];   // row -> slot, or -1
    int32_t fslot[kDecodeMaxRows];  // first row of an adapter -> its slot
    int32_t list[kDecodeMaxRows];   // slot -> adapter id
    int32_t wcount[kDecodeMaxRows / 64];
    int32_t T;                      // number of distinct adapters
};
static_assert(kDecodeMaxRows % 64 == 0, "whole waves of rows");

// Fill `ba` (in LDS) from ids[0 .. M); M <= kDecodeMaxRows.  Every thread of the workgroup
// must call it (blockDim.x >= kDecodeMaxRows, whole waves); it contains three barriers.
// Row t is handled by thread t: its first occurrence is found by an unrolled scan of the
// ids in LDS (independent reads), slots by a wave ballot prefix count.
__device__ __forceinline__ void batch_adapters(BatchAdapters &ba, const int32_t *__restrict__ ids,
                                               int M, int n_adapters) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const bool mine = t < kDecodeMaxRows;
    int a = -1;
    if (t < M) {
        a = ids[t];
        if (a < 0 || a >= n_adapters) a = -1;
    }
    if (mine) ba.id[t] = a;
    __syncthreads();
    int f = -1;
    if (mine && a >= 0) {
        f = t;
        const int4 *v4 = reinterpret_cast<const int4 *>(ba.id);
#pragma unroll
        for (int q = 0; q < kDecodeMaxRows / 4; ++q) {
            const int4 v = v4[q];
            const int j = 4 * q;
            if (v.w == a && j + 3 < f) f = j + 3;
            if (v.z == a && j + 2 < f) f = j + 2;
            if (v.y == a && j + 1 < f) f = j + 1;
            if (v.x == a && j < f) f = j;
        }
    }
    const bool first = mine && a >= 0 && f == t;
    const uint64_t bal = __ballot(first);
    if (mine && lane == 0) ba.wcount[w] = __popcll(bal);
    __syncthreads();
    if (mine) {
        int base = 0;
        for (int q = 0; q < w; ++q) base += ba.wcount[q];
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        if (first) {
            const int sl = base + __popcll(bal & below);
            ba.fslot[t] = sl;
            ba.list[sl] = a;
        }
    }
    if (t == 0) {
        int T = 0;
        for (int q = 0; q < kDecodeMaxRows / 64; ++q) T += ba.wcount[q];
        ba.T = T;
    }
    __syncthreads();
    if (mine) ba.slot[t] = (t < M && a >= 0) ? ba.fslot[f] : -1;
    __syncthreads();
}

}  // namespace lora

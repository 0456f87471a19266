// segments.hip -- group the rows of a mixed batch by adapter, on the device, in one launch.
//
// Source: "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to), section "How does
// one batch run 30 different adapters at once?": one pass over the full batch, an index
// vector mapping rows to adapter ids and a stacked adapter tensor, with no per-adapter host
// loop and no padding of the token dimension.  Grouping the rows by adapter is what lets
// every adapter's weights be read once per batch ("Serving Many LoRA Adapters From One Base
// Model", "Going deeper": grouping by adapter).
//
// Output (see lora_segments_t): a stable counting sort of row indices by adapter id, ids
// ascending, base-only rows (id -1, and invalid ids, which are counted) last; the prefix
// offsets; the compact list of adapters present; the segments cut into tiles of
// LORA_TILE_ROWS positions; and meta = {segments, LoRA rows, invalid ids, tiles}.
//
// One workgroup of 1024 threads (16 wave64s).  Every wave finds the lanes that share its
// bucket with one ballot per bit of the bucket number (a peer mask), so a row's rank among
// equal ids inside 64 rows is a popcount.  One block-wide exclusive scan of three per-bucket
// quantities (rows, "has rows", tiles) gives the offsets.  Two kernels differ in how the
// waves are ordered for the stable scatter:
//   * M > 1024 and n_adapters < 960 (build_segments_small_kernel): wave w owns a contiguous chunk of
//     rows and counts its rows per bucket into an LDS table pos[w][bucket]; a per-bucket
//     scan over the waves turns the table into each wave's first position per bucket, and
//     every wave then scatters its chunk independently.
//   * otherwise (build_segments_kernel): histogram by LDS atomics (counts do not depend
//     on order), then 1024 rows per round, the waves of a round taking their slots from the
//     per-bucket cursors strictly in wave order.
// No order-dependent atomic reaches perm: the result is identical on every run, and the
// same for both kernels.
#include "segments_block.h"

namespace lora {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Any n.  The stable scatter takes 1024 rows per round and the waves of a round in order.
__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t *__restrict__ ids,
                                                                  int M, int n, Seg seg) {
    // cnt (dynamic LDS, n + 1 entries): see build_segments_block
    extern __shared__ int32_t dyn[];
    __shared__ int32_t wave_tot[3][kWaves];
    __shared__ int32_t bad_total;
    build_segments_block<kThreads>(ids, M, n, seg, dyn, wave_tot, &bad_total);
}

// n < kSmallN.  Wave w owns the contiguous rows [w C, (w+1) C), C a multiple of 64, and
// walks them in order twice: first counting its rows per bucket into pos[w][b], then -- once
// pos[w][b] has become the first perm position of bucket b's rows in wave w (bucket start
// plus the counts of waves < w) -- writing perm.  Rows of one bucket thus keep their order
// inside a wave and across waves, with no order-dependent step shared between waves, and
// the workgroup needs only the barriers of the scans.
// Dynamic LDS: cnt[n + 1], then pos[kWaves][n + 1] (row stride n + 1); at most 64 KiB.
constexpr int kSmallN = 960;

__global__ __launch_bounds__(kThreads) void build_segments_small_kernel(
    const int32_t *__restrict__ ids, int M, int n, Seg seg) {
    extern __shared__ int32_t dyn[];
    const int nb = n + 1;
    int32_t *cnt = dyn;
    int32_t *pos = dyn + nb;
    __shared__ int32_t wave_tot[3][kWaves];
    __shared__ int32_t bad_total;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < kWaves * nb; i += kThreads) pos[i] = 0;
    if (tid == 0) bad_total = 0;
    __syncthreads();

    const int C = ((M + kWaves - 1) / kWaves + 63) & ~63;
    const int r0 = wave * C, r1 = min(r0 + C, M);
    const int nbits = 32 - __clz(n);
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

    // 1. per-wave histogram (one writer per (wave, bucket) per block of 64 rows: the peer
    //    group's lowest lane; a wave's LDS instructions execute in order).  The ids of four
    //    blocks are loaded together.
    // A wave whose chunk is one pass (C <= 256 rows: M <= 4096) keeps its buckets and peer
    // masks in registers for the scatter instead of reloading its ids.
    const bool one_pass = r1 - r0 <= 4 * 64;
    int kb[4];
    uint64_t kp[4];
    int bad = 0;
    for (int c0 = r0; c0 < r1; c0 += 4 * 64) {
        int bq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = c0 + 64 * q + lane;
            const int id = m < r1 ? ids[m] : -1;
            bq[q] = bucket_of(id, n);
            bad += (id != -1 && bq[q] == n);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool valid = c0 + 64 * q + lane < r1;
            const uint64_t peers = peer_mask(bq[q], valid, nbits);
            if (valid && __popcll(peers & lanes_below) == 0) pos[wave * nb + bq[q]] += __popcll(peers);
            kb[q] = bq[q];
            kp[q] = peers;
        }
    }
    if (bad) atomicAdd(&bad_total, bad);
    __syncthreads();

    // per bucket: totals, and pos[w][b] = rows of bucket b in waves < w
    for (int b = tid; b <= n; b += kThreads) {
        int c[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) c[w] = pos[w * nb + b];  // all reads first
        int run = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            pos[w * nb + b] = run;
            run += c[w];
        }
        cnt[b] = run;
    }
    __syncthreads();

    // 2. offsets, segments, tiles; cnt[b] becomes the first position of bucket b
    scan_buckets<kThreads>(cnt, wave_tot, n, bad_total, seg);

    // 3. scatter: the same walk as step 1
    for (int c0 = r0; c0 < r1; c0 += 4 * 64) {
        int bq[4];
        uint64_t pq[4];
        if (one_pass) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bq[q] = kb[q];
                pq[q] = kp[q];
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = c0 + 64 * q + lane;
                bq[q] = m < r1 ? bucket_of(ids[m], n) : n;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) pq[q] = peer_mask(bq[q], c0 + 64 * q + lane < r1, nbits);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int m = c0 + 64 * q + lane;
            const bool valid = m < r1;
            const uint64_t peers = pq[q];
            const int rank = __popcll(peers & lanes_below);
            if (valid) {
                const int base = cnt[bq[q]] + pos[wave * nb + bq[q]];
                if (rank == 0) pos[wave * nb + bq[q]] += __popcll(peers);
                seg.perm[base + rank] = m;
            }
        }
    }
}

}  // namespace

hipError_t launch_build_segments(const int32_t *ids, int M, int n_adapters, Seg seg,
                                 hipStream_t s) {
    const uint32_t nb = (uint32_t)n_adapters + 1;
    // up to 1024 rows the scatter is one round of at most 16 wave steps, which costs less
    // than the table's extra pass
    if (n_adapters < kSmallN && M > kThreads)
        launch(build_segments_small_kernel, dim3(1), dim3(kThreads), (kWaves + 1) * nb * 4, s, ids, M,
               n_adapters, seg);
    else
        launch(build_segments_kernel, dim3(1), dim3(kThreads), nb * 4, s, ids, M, n_adapters, seg);
    return hipGetLastError();
}

}  // namespace lora

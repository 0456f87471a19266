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
#include "common.h"

namespace lora {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Step 2 of both kernels: cnt[0..n) holds the row count of every bucket (cnt[n] is not
// read).  Writes offsets, seg_adapter, tiles and meta, and leaves cnt[b] = first position of
// bucket b in perm (cnt[n] = first base-only position).  Contains three barriers; every
// thread of the workgroup must call it.
__device__ void scan_buckets(int32_t *cnt, int32_t (*wave_tot)[kWaves], int n, int bad_total,
                             Seg seg) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // exclusive scans over buckets 0..n-1 of (rows, present, tiles); each thread owns a
    // contiguous run of buckets
    const int per = (n + kThreads - 1) / kThreads;
    const int b0 = min(tid * per, n), b1 = min(b0 + per, n);
    int rows = 0, segs = 0, tiles = 0;
    for (int b = b0; b < b1; ++b) {
        const int c = cnt[b];
        rows += c;
        segs += (c > 0);
        tiles += (c + kTileRows - 1) / kTileRows;
    }
    const int ir = wave_inclusive_scan(rows, lane);
    const int is = wave_inclusive_scan(segs, lane);
    const int it = wave_inclusive_scan(tiles, lane);
    if (lane == 63) {
        wave_tot[0][wave] = ir;
        wave_tot[1][wave] = is;
        wave_tot[2][wave] = it;
    }
    __syncthreads();
    int wr = 0, ws = 0, wt = 0, tr = 0, tsg = 0, ttl = 0;
    for (int w = 0; w < kWaves; ++w) {  // 16 entries: every thread scans them itself
        const int r_ = wave_tot[0][w], s_ = wave_tot[1][w], t_ = wave_tot[2][w];
        if (w < wave) { wr += r_; ws += s_; wt += t_; }
        tr += r_; tsg += s_; ttl += t_;
    }
    int pos = wr + ir - rows;   // first perm position of bucket b0
    int sgi = ws + is - segs;   // first seg_adapter slot
    int tli = wt + it - tiles;  // first tile slot
    __syncthreads();  // all reads of cnt[] as counts are done before it becomes a cursor

    for (int b = b0; b < b1; ++b) {
        const int c = cnt[b];
        seg.offsets[b] = pos;
        cnt[b] = pos;
        if (c > 0) {
            seg.seg_adapter[sgi++] = b;
            for (int j = 0; j < c; j += kTileRows) {
                seg.tiles[2 * tli] = pos + j;
                seg.tiles[2 * tli + 1] = b;
                ++tli;
            }
        }
        pos += c;
    }
    if (tid == 0) {
        seg.offsets[n] = tr;
        cnt[n] = tr;
        seg.meta[0] = tsg;
        seg.meta[1] = tr;
        seg.meta[2] = bad_total;
        seg.meta[3] = ttl;
    }
    __syncthreads();
}

// bucket of a row: its adapter, or n for base-only and invalid ids
__device__ __forceinline__ int bucket_of(int id, int n) { return (id < 0 || id >= n) ? n : id; }

// Lanes of this wave whose bucket equals mine (valid lanes only): one ballot per bit.
__device__ __forceinline__ uint64_t peer_mask(int b, bool valid, int nbits) {
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (b >> bit) & 1;
        const uint64_t bal = __ballot(valid && set);
        peers &= set ? bal : ~bal;
    }
    return peers;
}

// Any n.  The stable scatter takes 1024 rows per round and the waves of a round in order.
__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t *__restrict__ ids,
                                                                  int M, int n, Seg seg) {
    // cnt[b] (dynamic LDS, n + 1 entries): count of bucket b (b = n collects base-only and
    // invalid ids), later the next free position of bucket b in perm.
    extern __shared__ int32_t dyn[];
    int32_t *cnt = dyn;
    __shared__ int32_t wave_tot[3][kWaves];
    __shared__ int32_t bad_total;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int b = tid; b <= n; b += kThreads) cnt[b] = 0;
    if (tid == 0) bad_total = 0;
    __syncthreads();

    // 1. histogram
    int bad = 0;
    for (int m = tid; m < M; m += kThreads) {
        const int id = ids[m];
        bad += (id != -1 && (id < 0 || id >= n));
        atomicAdd(&cnt[bucket_of(id, n)], 1);
    }
    if (bad) atomicAdd(&bad_total, bad);
    __syncthreads();

    // 2. offsets, segments, tiles
    scan_buckets(cnt, wave_tot, n, bad_total, seg);

    // 3. stable scatter
    const int nbits = 32 - __clz(n);  // bits of the largest bucket number, n
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < M; c0 += kThreads) {
        const int m = c0 + tid;
        const bool valid = m < M;
        const int b = valid ? bucket_of(ids[m], n) : 0;
        const uint64_t peers = peer_mask(b, valid, nbits);
        const int rank = __popcll(peers & lanes_below);
        const int same = __popcll(peers);
        const int waves_used = min(kWaves, (M - c0 + 63) / 64);
        for (int w = 0; w < waves_used; ++w) {
            if (wave == w && valid) {
                // Every lane of this wave reads its bucket's cursor before the lowest lane
                // of each bucket advances it: one LDS read instruction precedes one LDS
                // write instruction in the same wave, and LDS executes a wave's
                // instructions in order.
                const int base = cnt[b];
                if (rank == 0) cnt[b] = base + same;
                seg.perm[base + rank] = m;
            }
            __syncthreads();
        }
    }
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
    scan_buckets(cnt, wave_tot, n, bad_total, seg);

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

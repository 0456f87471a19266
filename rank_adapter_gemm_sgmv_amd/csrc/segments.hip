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
// One workgroup of 1024 threads (16 wave64s):
//   1. histogram of bucket ids into LDS with LDS atomics (counts do not depend on order);
//   2. one block-wide exclusive scan of three per-bucket quantities at once: rows, "has
//      rows" and tiles; each thread owns a contiguous run of buckets;
//   3. stable scatter, 1024 rows per round: every wave finds the lanes that share its
//      bucket with one ballot per bit of the bucket number (a peer mask), so a row's rank
//      among equal ids in its wave is a popcount; the waves then take their slots from the
//      per-bucket cursors strictly in wave order, which keeps the sort stable without any
//      order-dependent atomic.
// The result is identical on every run.
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

__global__ __launch_bounds__(kThreads) void build_segments_kernel(const int32_t *__restrict__ ids,
                                                                  int M, int n, Seg seg) {
    // cnt[b]: count of bucket b (b = n collects base-only and invalid ids), later the
    // next free position of bucket b in perm.
    __shared__ int32_t cnt[LORA_MAX_ADAPTERS + 1];
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
        int b = id;
        if (id < 0 || id >= n) {
            b = n;
            bad += (id != -1);
        }
        atomicAdd(&cnt[b], 1);
    }
    if (bad) atomicAdd(&bad_total, bad);
    __syncthreads();

    // 2. exclusive scans over buckets 0..n-1 of (rows, present, tiles)
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

    // 3. stable scatter
    const int nbits = 32 - __clz(n);  // bits of the largest bucket number, n
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < M; c0 += kThreads) {
        const int m = c0 + tid;
        const bool valid = m < M;
        int b = 0;
        if (valid) {
            const int id = ids[m];
            b = (id < 0 || id >= n) ? n : id;
        }
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (b >> bit) & 1;
            const uint64_t bal = __ballot(valid && set);
            peers &= set ? bal : ~bal;
        }
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

}  // namespace

hipError_t launch_build_segments(const int32_t *ids, int M, int n_adapters, Seg seg,
                                 hipStream_t s) {
    launch(build_segments_kernel, dim3(1), dim3(kThreads), 0, s, ids, M, n_adapters,
                       seg);
    return hipGetLastError();
}

}  // namespace lora

// segments_block.h -- the segment builder's work for one workgroup of NT threads (NT a
// multiple of 64), shared by the builder's own launch (csrc/segments.hip, 1024 threads) and
// the extra workgroup of the medium-batch decode GEMM launch (csrc/decode_gemm.hip, 256
// threads), which builds the segments beside the GEMM.  Internal.
//
// The grouping: a stable counting sort of row indices by adapter id ("Multi-LoRA Serving:
// Why 100 Adapters Fit on One GPU" (dev.to), "How does one batch run 30 different adapters at
// once?"), see csrc/segments.hip.
#pragma once

#include "common.h"

namespace lora {

namespace {

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
template <int NT>
__device__ void scan_buckets(int32_t *cnt, int32_t (*wave_tot)[NT / 64], int n, int bad_total,
                             Seg seg) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // exclusive scans over buckets 0..n-1 of (rows, present, tiles); each thread owns a
    // contiguous run of buckets
    const int per = (n + NT - 1) / NT;
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
    for (int w = 0; w < NT / 64; ++w) {  // one entry per wave: every thread scans them itself
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

// Any n.  LDS (the caller's): cnt[n + 1], the count of bucket b (b = n collects base-only
// and invalid ids), later the next free position of bucket b in perm; wave_tot[3][NT / 64];
// *bad_total.  The stable scatter takes NT rows per round and the waves of a round in order.
// Every thread of the workgroup must call it (it contains barriers).
template <int NT>
__device__ __forceinline__ void build_segments_block(const int32_t *__restrict__ ids, int M, int n,
                                                     Seg seg, int32_t *cnt,
                                                     int32_t (*wave_tot)[NT / 64],
                                                     int32_t *bad_total) {
    static_assert(NT % 64 == 0 && NT >= 64 && NT <= 1024, "whole waves");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int b = tid; b <= n; b += NT) cnt[b] = 0;
    if (tid == 0) *bad_total = 0;
    __syncthreads();

    // 1. histogram
    int bad = 0;
    for (int m = tid; m < M; m += NT) {
        const int id = ids[m];
        bad += (id != -1 && (id < 0 || id >= n));
        atomicAdd(&cnt[bucket_of(id, n)], 1);
    }
    if (bad) atomicAdd(bad_total, bad);
    __syncthreads();

    // 2. offsets, segments, tiles
    scan_buckets<NT>(cnt, wave_tot, n, *bad_total, seg);

    // 3. stable scatter
    const int nbits = 32 - __clz(n);  // bits of the largest bucket number, n
    const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int c0 = 0; c0 < M; c0 += NT) {
        const int m = c0 + tid;
        const bool valid = m < M;
        const int b = valid ? bucket_of(ids[m], n) : 0;
        const uint64_t peers = peer_mask(b, valid, nbits);
        const int rank = __popcll(peers & lanes_below);
        const int same = __popcll(peers);
        const int waves_used = min(NT / 64, (M - c0 + 63) / 64);
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

}  // namespace lora

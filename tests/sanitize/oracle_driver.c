/* oracle_driver.c -- runs every entry point of oracle/oracle.c over many shapes, edge cases
 * and error paths, every buffer malloc'ed at exactly the size the entry point's contract
 * gives, so that an AddressSanitizer / UndefinedBehaviorSanitizer build of the two files
 * (tests/test_sanitizers.py) reports any access outside a buffer or any undefined operation.
 * Exit status 0 when every call returned the status expected of it.  Test infrastructure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_build_segments(const int32_t *ids, int32_t M, int32_t n_adapters, int32_t tile_rows,
                          int32_t *perm, int32_t *offsets, int32_t *seg_adapter, int32_t *tiles,
                          int32_t *meta);
int oracle_lora_shrink(const float *x, const float *A, const int32_t *ids, int32_t M, int32_t d_in,
                       int32_t r_max, int32_t n_adapters, float *t, int32_t n_threads);
int oracle_lora_expand(const float *t, const float *B, const float *alpha, const int32_t *ranks,
                       const int32_t *ids, int32_t M, int32_t d_out, int32_t r_max,
                       int32_t n_adapters, float *y, int32_t n_threads);
int oracle_lora_linear(const float *x, const float *W, const float *A, const float *B,
                       const float *alpha, const int32_t *ranks, const int32_t *ids, int32_t M,
                       int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
                       const int32_t *rows, int32_t n_rows, float *y, int32_t n_threads);
float oracle_fp8_e4m3_decode(uint8_t code);
void oracle_fp8_e4m3_decode_array(const uint8_t *codes, int64_t n, float *out);
int oracle_lora_linear_fp8w(const float *x, const uint8_t *W8, const float *w_scale,
                            const float *A, const float *B, const float *alpha,
                            const int32_t *ranks, const int32_t *ids, int32_t M, int32_t d_in,
                            int32_t d_out, int32_t r_max, int32_t n_adapters, const int32_t *rows,
                            int32_t n_rows, float *y, int32_t n_threads);
int oracle_moe_lora_linear(const float *x, const float *W, const float *A, const float *B,
                           const float *alpha, const int32_t *ranks, const int32_t *ids,
                           const int32_t *topk_ids, const float *topk_w, int32_t M, int32_t top_k,
                           int32_t n_experts, int32_t d_in, int32_t d_out, int32_t r_max,
                           int32_t n_adapters, float *y, int32_t n_threads);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float *fbuf(size_t n) { /* n >= 0; at least one element so malloc never returns NULL */
    float *p = (float *)malloc((n ? n : 1) * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = (float)((int)(rnd() % 2001) - 1000) / 1000.0f;
    return p;
}
static int32_t *ibuf(size_t n) { return (int32_t *)malloc((n ? n : 1) * sizeof(int32_t)); }

static int failures = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        int got_ = (call);                                                                  \
        if (got_ != (want)) {                                                               \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                    got_, (want));                                                          \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

static void ids_fill(int32_t *ids, int M, int n, int base_pct) {
    for (int m = 0; m < M; ++m) ids[m] = (int)(rnd() % 100) < base_pct ? -1 : (int32_t)(rnd() % n);
}

static void segments_case(int M, int n, int tile_rows, int base_pct) {
    int32_t *ids = ibuf(M);
    ids_fill(ids, M, n, base_pct);
    const int segs = M < n ? M : n;
    const int max_tiles = segs + M / tile_rows;
    int32_t *perm = ibuf(M), *off = ibuf(n + 1), *sa = ibuf(segs > 1 ? segs : 1),
            *tiles = ibuf(2 * (max_tiles > 1 ? max_tiles : 1)), *meta = ibuf(4);
    EXPECT(oracle_build_segments(ids, M, n, tile_rows, perm, off, sa, tiles, meta), 0);
    if (M > 0) { /* an id out of range is an error */
        ids[M - 1] = n;
        EXPECT(oracle_build_segments(ids, M, n, tile_rows, perm, off, sa, tiles, meta), 2);
    }
    free(ids); free(perm); free(off); free(sa); free(tiles); free(meta);
}

static void linear_case(int M, int d_in, int d_out, int r_max, int n, int threads) {
    float *x = fbuf((size_t)M * d_in), *W = fbuf((size_t)d_in * d_out),
          *A = fbuf((size_t)n * d_in * r_max), *B = fbuf((size_t)n * r_max * d_out),
          *alpha = fbuf(n), *t = fbuf((size_t)M * r_max), *y = fbuf((size_t)M * d_out);
    int32_t *ranks = ibuf(n), *ids = ibuf(M);
    for (int i = 0; i < n; ++i) ranks[i] = 1 + (int32_t)(rnd() % r_max);
    ids_fill(ids, M, n, 25);
    EXPECT(oracle_lora_shrink(x, A, ids, M, d_in, r_max, n, t, threads), 0);
    EXPECT(oracle_lora_expand(t, B, alpha, ranks, ids, M, d_out, r_max, n, y, threads), 0);
    EXPECT(oracle_lora_linear(x, W, A, B, alpha, ranks, ids, M, d_in, d_out, r_max, n, NULL, 0, y,
                              threads), 0);
    /* a sample of rows, into a buffer of exactly that many rows */
    const int nr = M < 5 ? M : 5;
    int32_t *rows = ibuf(nr);
    for (int q = 0; q < nr; ++q) rows[q] = (int32_t)(rnd() % (M ? M : 1));
    float *ys = fbuf((size_t)nr * d_out);
    EXPECT(oracle_lora_linear(x, W, A, B, alpha, ranks, ids, M, d_in, d_out, r_max, n, rows, nr, ys,
                              threads), 0);
    /* fp8 base of the same sizes */
    uint8_t *W8 = (uint8_t *)malloc((size_t)d_out * d_in);
    for (size_t i = 0; i < (size_t)d_out * d_in; ++i) {
        uint8_t c = (uint8_t)(rnd() & 0xFF);
        W8[i] = (c & 0x7F) == 0x7F ? 0 : c;
    }
    float *wsc = fbuf(d_out);
    EXPECT(oracle_lora_linear_fp8w(x, W8, wsc, A, B, alpha, ranks, ids, M, d_in, d_out, r_max, n,
                                   NULL, 0, y, threads), 0);
    EXPECT(oracle_lora_linear_fp8w(x, W8, wsc, A, B, alpha, ranks, ids, M, d_in, d_out, r_max, n,
                                   rows, nr, ys, threads), 0);
    /* error paths: a bad id, a bad row index, bad sizes */
    if (M > 0) {
        ids[0] = n;
        EXPECT(oracle_lora_linear(x, W, A, B, alpha, ranks, ids, M, d_in, d_out, r_max, n, NULL, 0, y,
                                  threads), 2);
        EXPECT(oracle_lora_shrink(x, A, ids, M, d_in, r_max, n, t, threads), 2);
        ids[0] = -1;
        if (nr > 0) {
            rows[0] = M;
            EXPECT(oracle_lora_linear(x, W, A, B, alpha, ranks, ids, M, d_in, d_out, r_max, n, rows,
                                      nr, ys, threads), 1);
        }
    }
    EXPECT(oracle_lora_linear(x, W, A, B, alpha, ranks, ids, -1, d_in, d_out, r_max, n, NULL, 0, y,
                              threads), 1);
    free(x); free(W); free(A); free(B); free(alpha); free(t); free(y); free(ranks); free(ids);
    free(rows); free(ys); free(W8); free(wsc);
}

static void moe_case(int M, int top_k, int E, int d_in, int d_out, int r_max, int n, int threads,
                     int weights) {
    const size_t P = (size_t)M * top_k;
    float *x = fbuf((size_t)M * d_in), *W = fbuf((size_t)E * d_in * d_out),
          *A = fbuf((size_t)n * E * d_in * r_max), *B = fbuf((size_t)n * E * r_max * d_out),
          *alpha = fbuf(n), *tw = fbuf(P), *y = fbuf(P * d_out);
    int32_t *ranks = ibuf(n), *ids = ibuf(M), *topk = ibuf(P);
    for (int i = 0; i < n; ++i) ranks[i] = 1 + (int32_t)(rnd() % r_max);
    ids_fill(ids, M, n, 20);
    for (size_t p = 0; p < P; ++p) topk[p] = (rnd() % 8 == 0) ? -1 : (int32_t)(rnd() % E);
    EXPECT(oracle_moe_lora_linear(x, W, A, B, alpha, ranks, ids, topk, weights ? tw : NULL, M,
                                  top_k, E, d_in, d_out, r_max, n, y, threads), 0);
    if (P > 0) {
        topk[P - 1] = E; /* an expert id out of range */
        EXPECT(oracle_moe_lora_linear(x, W, A, B, alpha, ranks, ids, topk, tw, M, top_k, E, d_in,
                                      d_out, r_max, n, y, threads), 2);
    }
    free(x); free(W); free(A); free(B); free(alpha); free(tw); free(y); free(ranks); free(ids);
    free(topk);
}

int main(void) {
    /* segments: empty, all base, one adapter, more adapters than rows, ragged tiles */
    const int seg_shapes[][4] = {{0, 1, 16, 0},   {1, 1, 16, 0},   {17, 3, 16, 100},
                                 {64, 1, 16, 0},  {33, 200, 4, 10}, {1000, 7, 16, 30},
                                 {5, 5, 1, 0},    {257, 64, 16, 50}};
    for (size_t i = 0; i < sizeof seg_shapes / sizeof seg_shapes[0]; ++i)
        segments_case(seg_shapes[i][0], seg_shapes[i][1], seg_shapes[i][2], seg_shapes[i][3]);
    /* the layer: empty batch, one row, ragged sizes, r_max 1 and 64, many adapters */
    const int lin_shapes[][6] = {{0, 8, 8, 4, 2, 1},    {1, 1, 1, 1, 1, 1},   {7, 13, 5, 3, 4, 2},
                                 {33, 64, 40, 16, 9, 4}, {5, 24, 72, 64, 3, 3}, {40, 16, 8, 8, 300, 8}};
    for (size_t i = 0; i < sizeof lin_shapes / sizeof lin_shapes[0]; ++i)
        linear_case(lin_shapes[i][0], lin_shapes[i][1], lin_shapes[i][2], lin_shapes[i][3],
                    lin_shapes[i][4], lin_shapes[i][5]);
    /* every fp8 code */
    uint8_t codes[256];
    float vals[256];
    for (int c = 0; c < 256; ++c) codes[c] = (uint8_t)c;
    oracle_fp8_e4m3_decode_array(codes, 256, vals);
    for (int c = 0; c < 256; ++c) {
        const float v = oracle_fp8_e4m3_decode((uint8_t)c);
        if ((c & 0x7F) == 0x7F ? !isnan(vals[c]) : vals[c] != v) {
            fprintf(stderr, "fp8 code %d decodes inconsistently\n", c);
            ++failures;
        }
    }
    /* MoE: empty batch, one expert, top_k 1 and 8, with and without routing weights */
    const int moe_shapes[][9] = {{0, 2, 3, 8, 8, 4, 2, 1, 1},     {1, 1, 1, 4, 4, 1, 1, 1, 0},
                                 {9, 2, 4, 24, 20, 4, 3, 2, 1},   {17, 8, 16, 16, 8, 8, 5, 4, 1},
                                 {6, 3, 5, 40, 28, 8, 40, 3, 0}};
    for (size_t i = 0; i < sizeof moe_shapes / sizeof moe_shapes[0]; ++i)
        moe_case(moe_shapes[i][0], moe_shapes[i][1], moe_shapes[i][2], moe_shapes[i][3],
                 moe_shapes[i][4], moe_shapes[i][5], moe_shapes[i][6], moe_shapes[i][7],
                 moe_shapes[i][8]);
    if (failures) {
        fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    printf("oracle driver: all calls returned the expected status\n");
    return 0;
}

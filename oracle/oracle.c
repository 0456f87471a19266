/*
 * oracle.c -- plain, slow CPU reference for the multi-LoRA batched linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The GPU library never links, includes or
 * calls it, and the two share no code: no kernels, headers, helpers or tables.
 *
 * Source pages, cited by title and section:
 *   [P1] "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to)
 *   [P2] "Serving Many LoRA Adapters From One Base Model" (ai-tldr.dev)
 *   [P3] "Multi-LoRA Serving: Sharing One GPU Across Adapters" (cloudai.pt)
 *
 * What is computed is the layer equation of [P1], section "Why can't you just merge LoRA
 * weights into the base model?":
 *
 *     y = x W + (x A_i) B_i * (alpha_i / r_i)
 *
 * evaluated one row at a time, each row with its own adapter i ([P2], "How it works",
 * "Batching across different adapters": the base term is shared, and each row gets its own
 * adapter correction).  An id of -1 means the bare base ([P2], "A worked example: the
 * memory math", the adapter=None request).
 *
 * Layout (row-major): x[M][d_in], W[d_in][d_out], A[n][d_in][r_max], B[n][r_max][d_out].
 * A_i is stored d_in x r_max and B_i is r_max x d_out (the transposes of [P1]'s
 * "A: r x d_in, B: d_out x r", same parameter count), so that the row-vector form
 * x A_i B_i reads directly.  Adapters are padded to r_max with zeros ([P1], "What does a
 * working multi-LoRA config look like?": every adapter is padded to the maximum rank);
 * the sums below run over all r_max stored columns, the zero padding adds nothing.
 *
 * Precision: every input arrives as float32 (bf16 inputs are widened exactly by the
 * caller); every product and sum is float32, accumulated in ascending index order.
 * Built with -ffp-contract=off, so no fused multiply-add changes the rounding.
 *
 * The segment builder is the definition of "group the rows by adapter" ([P1], "How does
 * one batch run 30 different adapters at once?": one launch over the full batch, an index
 * vector and a stacked adapter tensor; [P2], "Going deeper": grouping by adapter): a
 * stable counting sort of the rows by adapter id, base-only rows last.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_BAD_ID 2
#define ORACLE_ERR_NOMEM 3

static int ids_valid(const int32_t *ids, int32_t M, int32_t n_adapters) {
    for (int32_t m = 0; m < M; ++m)
        if (ids[m] < -1 || ids[m] >= n_adapters) return 0;
    return 1;
}

/* ---------------------------------------------------------------------------------------
 * Segments: stable counting sort of row indices by adapter id.
 *
 *   offsets[i]     first position in perm of adapter i's rows (offsets[n] = #LoRA rows)
 *   perm           rows of adapter 0 in ascending row order, then adapter 1, ..., then the
 *                  id -1 rows in ascending row order
 *   seg_adapter    the adapters that have rows, ascending (meta[0] entries)
 *   tiles          each segment cut into runs of tile_rows positions of perm, in segment
 *                  order: pairs {first perm position, adapter}
 *   meta           {segments, LoRA rows, invalid ids (always 0 here), tiles}
 * ------------------------------------------------------------------------------------- */
int oracle_build_segments(const int32_t *ids, int32_t M, int32_t n_adapters, int32_t tile_rows,
                          int32_t *perm, int32_t *offsets, int32_t *seg_adapter,
                          int32_t *tiles, int32_t *meta) {
    if (M < 0 || n_adapters < 1 || tile_rows < 1) return ORACLE_ERR_ARG;
    if (!ids_valid(ids, M, n_adapters)) return ORACLE_ERR_BAD_ID;

    int32_t *count = (int32_t *)calloc((size_t)n_adapters, sizeof(int32_t));
    int32_t *cursor = (int32_t *)calloc((size_t)n_adapters, sizeof(int32_t));
    if (!count || !cursor) { free(count); free(cursor); return ORACLE_ERR_NOMEM; }

    for (int32_t m = 0; m < M; ++m)
        if (ids[m] >= 0) count[ids[m]] += 1;

    int32_t running = 0;
    for (int32_t i = 0; i < n_adapters; ++i) {
        offsets[i] = running;
        cursor[i] = running;
        running += count[i];
    }
    offsets[n_adapters] = running;
    const int32_t n_lora_rows = running;

    int32_t base_pos = n_lora_rows;
    for (int32_t m = 0; m < M; ++m) {
        if (ids[m] >= 0) perm[cursor[ids[m]]++] = m;
        else perm[base_pos++] = m;
    }

    int32_t n_seg = 0, n_tiles = 0;
    for (int32_t i = 0; i < n_adapters; ++i) {
        if (count[i] == 0) continue;
        seg_adapter[n_seg++] = i;
        for (int32_t p = offsets[i]; p < offsets[i + 1]; p += tile_rows) {
            tiles[2 * n_tiles] = p;
            tiles[2 * n_tiles + 1] = i;
            n_tiles += 1;
        }
    }
    meta[0] = n_seg;
    meta[1] = n_lora_rows;
    meta[2] = 0;
    meta[3] = n_tiles;
    free(count);
    free(cursor);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------------------
 * Shrink: t[m][j] = sum_k x[m][k] * A[i][k][j] for a row with adapter i >= 0, and
 * t[m][j] = 0 for a base-only row.  The step that takes x down to the adapter rank
 * ([P3], "MoE Models Raise the Bar", the adapter "shrink"; [P1], "How does one batch run 30
 * different adapters at once?", the [B, 4096] x [4096, r] product).
 * ------------------------------------------------------------------------------------- */
int oracle_lora_shrink(const float *x, const float *A, const int32_t *ids, int32_t M,
                       int32_t d_in, int32_t r_max, int32_t n_adapters, float *t,
                       int32_t n_threads) {
    if (M < 0 || d_in < 1 || r_max < 1 || n_adapters < 1) return ORACLE_ERR_ARG;
    if (!ids_valid(ids, M, n_adapters)) return ORACLE_ERR_BAD_ID;
    (void)n_threads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
    for (int32_t m = 0; m < M; ++m) {
        float *trow = t + (size_t)m * r_max;
        for (int32_t j = 0; j < r_max; ++j) trow[j] = 0.0f;
        const int32_t i = ids[m];
        if (i < 0) continue;
        for (int32_t k = 0; k < d_in; ++k) {
            const float xv = x[(size_t)m * d_in + k];
            const float *arow = A + ((size_t)i * d_in + k) * r_max;
            for (int32_t j = 0; j < r_max; ++j) trow[j] += xv * arow[j];
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------------------------------
 * Expand: y[m][c] += (alpha_i / r_i) * sum_j t[m][j] * B[i][j][c] for a row with adapter
 * i >= 0; base-only rows are left untouched.  The step back up to d_out ([P3], "MoE Models
 * Raise the Bar", the adapter "expand"), scaled as in [P1]'s layer equation.
 * ------------------------------------------------------------------------------------- */
int oracle_lora_expand(const float *t, const float *B, const float *alpha, const int32_t *ranks,
                       const int32_t *ids, int32_t M, int32_t d_out, int32_t r_max,
                       int32_t n_adapters, float *y, int32_t n_threads) {
    if (M < 0 || d_out < 1 || r_max < 1 || n_adapters < 1) return ORACLE_ERR_ARG;
    if (!ids_valid(ids, M, n_adapters)) return ORACLE_ERR_BAD_ID;
    int status = ORACLE_OK;
    (void)n_threads;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
    {
        float *d = (float *)malloc((size_t)d_out * sizeof(float));
        if (!d) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int32_t m = 0; m < M; ++m) {
            const int32_t i = ids[m];
            if (i < 0 || !d) continue;
            const float s = alpha[i] / (float)ranks[i];
            for (int32_t c = 0; c < d_out; ++c) d[c] = 0.0f;
            for (int32_t j = 0; j < r_max; ++j) {
                const float tj = t[(size_t)m * r_max + j];
                const float *brow = B + ((size_t)i * r_max + j) * d_out;
                for (int32_t c = 0; c < d_out; ++c) d[c] += tj * brow[c];
            }
            float *yrow = y + (size_t)m * d_out;
            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];
        }
        free(d);
    }
    return status;
}

/* ---------------------------------------------------------------------------------------
 * The whole layer, row by row:
 *
 *   y[m][c] = sum_k x[m][k] W[k][c]                                  (shared base)
 *   if ids[m] = i >= 0:
 *       t[j]  = sum_k x[m][k] A[i][k][j]                             (x A_i)
 *       d[c]  = sum_j t[j] B[i][j][c]                                ((x A_i) B_i)
 *       y[m][c] += (alpha_i / r_i) * d[c]                             (* alpha / r)
 *
 * rows == NULL computes all M rows into y[M][d_out]; otherwise it computes only the
 * n_rows listed rows, into y[n_rows][d_out] in list order (every row is independent, so
 * a sample of rows is the same definition restricted to those rows).
 * ------------------------------------------------------------------------------------- */
int oracle_lora_linear(const float *x, const float *W, const float *A, const float *B,
                       const float *alpha, const int32_t *ranks, const int32_t *ids,
                       int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                       int32_t n_adapters, const int32_t *rows, int32_t n_rows, float *y,
                       int32_t n_threads) {
    if (M < 0 || d_in < 1 || d_out < 1 || r_max < 1 || n_adapters < 1) return ORACLE_ERR_ARG;
    if (!ids_valid(ids, M, n_adapters)) return ORACLE_ERR_BAD_ID;
    const int32_t count = rows ? n_rows : M;
    if (count < 0) return ORACLE_ERR_ARG;
    for (int32_t q = 0; rows && q < count; ++q)
        if (rows[q] < 0 || rows[q] >= M) return ORACLE_ERR_ARG;
    int status = ORACLE_OK;
    (void)n_threads;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
    {
        float *t = (float *)malloc((size_t)r_max * sizeof(float));
        float *d = (float *)malloc((size_t)d_out * sizeof(float));
        if (!t || !d) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int32_t q = 0; q < count; ++q) {
            if (!t || !d) continue;
            const int32_t m = rows ? rows[q] : q;
            const float *xrow = x + (size_t)m * d_in;
            float *yrow = y + (size_t)q * d_out;

            /* shared base term x W */
            for (int32_t c = 0; c < d_out; ++c) yrow[c] = 0.0f;
            for (int32_t k = 0; k < d_in; ++k) {
                const float xv = xrow[k];
                const float *wrow = W + (size_t)k * d_out;
                for (int32_t c = 0; c < d_out; ++c) yrow[c] += xv * wrow[c];
            }

            const int32_t i = ids[m];
            if (i == -1) continue; /* base only */

            /* x A_i */
            for (int32_t j = 0; j < r_max; ++j) t[j] = 0.0f;
            for (int32_t k = 0; k < d_in; ++k) {
                const float xv = xrow[k];
                const float *arow = A + ((size_t)i * d_in + k) * r_max;
                for (int32_t j = 0; j < r_max; ++j) t[j] += xv * arow[j];
            }

            /* (x A_i) B_i */
            for (int32_t c = 0; c < d_out; ++c) d[c] = 0.0f;
            for (int32_t j = 0; j < r_max; ++j) {
                const float tj = t[j];
                const float *brow = B + ((size_t)i * r_max + j) * d_out;
                for (int32_t c = 0; c < d_out; ++c) d[c] += tj * brow[c];
            }

            /* * alpha_i / r_i, added to the base term */
            const float s = alpha[i] / (float)ranks[i];
            for (int32_t c = 0; c < d_out; ++c) yrow[c] += s * d[c];
        }
        free(t);
        free(d);
    }
    return status;
}

/* ---------------------------------------------------------------------------------------
 * Quantized base ([P1], "Where does multi-LoRA serving actually break?", item 4: a base
 * stored at low precision served beside higher-precision adapters; the delta runs in a
 * different type than the base).  The base weight is held as 8-bit floating point codes of
 * the E4M3 format of the OCP 8-bit floating point specification ("E4M3FN"): 1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes the subnormals
 * m * 2^-9; the code whose exponent and mantissa bits are all ones is NaN; there is no
 * infinity.  The codes are laid out W8[d_out][d_in] (each output column's d_in codes
 * contiguous), with one fp32 scale per output column.
 * ------------------------------------------------------------------------------------- */
float oracle_fp8_e4m3_decode(uint8_t code) {
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -v : v;
}

void oracle_fp8_e4m3_decode_array(const uint8_t *codes, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp8_e4m3_decode(codes[i]);
}

/* The layer with the quantized base:
 *
 *   y[m][c] = w_scale[c] * sum_k x[m][k] dec(W8[c][k])              (shared base, k ascending)
 *   if ids[m] = i >= 0:  y[m][c] += (alpha_i / r_i) * sum_j (sum_k x[m][k] A[i][k][j]) B[i][j][c]
 *
 * i.e. x W_eff with W_eff[k][c] = w_scale[c] dec(W8[c][k]), the scale applied to the fp32
 * sum; the delta exactly as in oracle_lora_linear.  rows / n_rows as there. */
int oracle_lora_linear_fp8w(const float *x, const uint8_t *W8, const float *w_scale,
                            const float *A, const float *B, const float *alpha,
                            const int32_t *ranks, const int32_t *ids, int32_t M, int32_t d_in,
                            int32_t d_out, int32_t r_max, int32_t n_adapters, const int32_t *rows,
                            int32_t n_rows, float *y, int32_t n_threads) {
    if (M < 0 || d_in < 1 || d_out < 1 || r_max < 1 || n_adapters < 1) return ORACLE_ERR_ARG;
    if (!ids_valid(ids, M, n_adapters)) return ORACLE_ERR_BAD_ID;
    const int32_t count = rows ? n_rows : M;
    if (count < 0) return ORACLE_ERR_ARG;
    for (int32_t q = 0; rows && q < count; ++q)
        if (rows[q] < 0 || rows[q] >= M) return ORACLE_ERR_ARG;
    /* dec(W8) as an fp32 table Wd[k][c] (decoding is exact) */
    float *Wd = (float *)malloc((size_t)d_in * d_out * sizeof(float));
    if (!Wd) return ORACLE_ERR_NOMEM;
    for (int32_t c = 0; c < d_out; ++c)
        for (int32_t k = 0; k < d_in; ++k)
            Wd[(size_t)k * d_out + c] = oracle_fp8_e4m3_decode(W8[(size_t)c * d_in + k]);
    int status = ORACLE_OK;
    (void)n_threads;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
    {
        float *t = (float *)malloc((size_t)r_max * sizeof(float));
        float *d = (float *)malloc((size_t)d_out * sizeof(float));
        if (!t || !d) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int32_t q = 0; q < count; ++q) {
            if (!t || !d) continue;
            const int32_t m = rows ? rows[q] : q;
            const float *xrow = x + (size_t)m * d_in;
            float *yrow = y + (size_t)q * d_out;

            /* shared base term: sum_k x dec(W8), then times the column's scale */
            for (int32_t c = 0; c < d_out; ++c) yrow[c] = 0.0f;
            for (int32_t k = 0; k < d_in; ++k) {
                const float xv = xrow[k];
                const float *wdrow = Wd + (size_t)k * d_out;
                for (int32_t c = 0; c < d_out; ++c) yrow[c] += xv * wdrow[c];
            }
            for (int32_t c = 0; c < d_out; ++c) yrow[c] = w_scale[c] * yrow[c];

            const int32_t i = ids[m];
            if (i == -1) continue; /* base only */

            for (int32_t j = 0; j < r_max; ++j) t[j] = 0.0f;
            for (int32_t k = 0; k < d_in; ++k) {
                const float xv = xrow[k];
                const float *arow8 = A + ((size_t)i * d_in + k) * r_max;
                for (int32_t j = 0; j < r_max; ++j) t[j] += xv * arow8[j];
            }
            for (int32_t c = 0; c < d_out; ++c) d[c] = 0.0f;
            for (int32_t j = 0; j < r_max; ++j) {
                const float tj = t[j];
                const float *brow8 = B + ((size_t)i * r_max + j) * d_out;
                for (int32_t c = 0; c < d_out; ++c) d[c] += tj * brow8[c];
            }
            const float sc = alpha[i] / (float)ranks[i];
            for (int32_t c = 0; c < d_out; ++c) yrow[c] += sc * d[c];
        }
        free(t);
        free(d);
    }
    free(Wd);
    return status;
}

/* ---------------------------------------------------------------------------------------
 * MoE-LoRA ([P3], "MoE Models Raise the Bar": in a routed expert layer every adapted
 * projection of every expert carries the request's adapter, and the adapter's shrink and
 * expand run inside the expert routing kernel).  Token m is routed to top_k experts
 * (topk_ids[m][j], -1 = no expert in that slot) with routing weights topk_w[m][j]; it
 * carries adapter ids[m] (-1 = the bare base).  Expert e has its own base weight
 * W[e][d_in][d_out] and, for every adapter i, its own pair A[i][e][d_in][r_max],
 * B[i][e][r_max][d_out] (padded to r_max with zeros).  Per (token, slot), with e = topk_ids:
 *
 *   y[m][j][c] = topk_w[m][j] * ( sum_k x[m][k] W[e][k][c]
 *                                 + (alpha_i / r_i) sum_q (sum_k x[m][k] A[i][e][k][q]) B[i][e][q][c] )
 *
 * (the adapter term only when i = ids[m] >= 0), and y[m][j][:] = 0 for a slot with no
 * expert.  topk_w NULL means weight 1.  Sums ascending, fp32, as in oracle_lora_linear; the
 * routing weight multiplies the finished row.
 * ------------------------------------------------------------------------------------- */
int oracle_moe_lora_linear(const float *x, const float *W, const float *A, const float *B,
                           const float *alpha, const int32_t *ranks, const int32_t *ids,
                           const int32_t *topk_ids, const float *topk_w, int32_t M, int32_t top_k,
                           int32_t n_experts, int32_t d_in, int32_t d_out, int32_t r_max,
                           int32_t n_adapters, float *y, int32_t n_threads) {
    if (M < 0 || top_k < 1 || n_experts < 1 || d_in < 1 || d_out < 1 || r_max < 1 ||
        n_adapters < 1)
        return ORACLE_ERR_ARG;
    if (!ids_valid(ids, M, n_adapters)) return ORACLE_ERR_BAD_ID;
    for (int64_t p = 0; p < (int64_t)M * top_k; ++p)
        if (topk_ids[p] < -1 || topk_ids[p] >= n_experts) return ORACLE_ERR_BAD_ID;
    int status = ORACLE_OK;
    (void)n_threads;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
    {
        float *tq = (float *)malloc((size_t)r_max * sizeof(float));
        float *dq = (float *)malloc((size_t)d_out * sizeof(float));
        if (!tq || !dq) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t p = 0; p < (int64_t)M * top_k; ++p) {
            if (!tq || !dq) continue;
            const int32_t m = (int32_t)(p / top_k);
            const int32_t e = topk_ids[p];
            float *out = y + (size_t)p * d_out;
            for (int32_t c = 0; c < d_out; ++c) out[c] = 0.0f;
            if (e < 0) continue; /* empty slot */
            const float *xrow = x + (size_t)m * d_in;
            const float *We = W + (size_t)e * d_in * d_out;
            for (int32_t k = 0; k < d_in; ++k) {
                const float xv = xrow[k];
                const float *werow = We + (size_t)k * d_out;
                for (int32_t c = 0; c < d_out; ++c) out[c] += xv * werow[c];
            }
            const int32_t i = ids[m];
            if (i >= 0) {
                const float *Aie = A + ((size_t)i * n_experts + e) * d_in * r_max;
                const float *Bie = B + ((size_t)i * n_experts + e) * r_max * d_out;
                for (int32_t q = 0; q < r_max; ++q) tq[q] = 0.0f;
                for (int32_t k = 0; k < d_in; ++k) {
                    const float xv = xrow[k];
                    for (int32_t q = 0; q < r_max; ++q) tq[q] += xv * Aie[(size_t)k * r_max + q];
                }
                for (int32_t c = 0; c < d_out; ++c) dq[c] = 0.0f;
                for (int32_t q = 0; q < r_max; ++q) {
                    const float tv = tq[q];
                    for (int32_t c = 0; c < d_out; ++c) dq[c] += tv * Bie[(size_t)q * d_out + c];
                }
                const float sa = alpha[i] / (float)ranks[i];
                for (int32_t c = 0; c < d_out; ++c) out[c] += sa * dq[c];
            }
            if (topk_w) {
                const float wt = topk_w[p];
                for (int32_t c = 0; c < d_out; ++c) out[c] = wt * out[c];
            }
        }
        free(tq);
        free(dq);
    }
    return status;
}

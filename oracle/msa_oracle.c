/*
 * msa_oracle.c -- plain CPU oracle for the MiniMax-M3 lightning-indexer decode pass.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may load or run this library. It shares no code,
 * header, table or helper with the GPU library and must never be used to produce
 * a product result.
 *
 * It is written to be obviously correct, not fast: plain loops, fp64 arithmetic,
 * a library sort for the selection, OpenMP only over independent (row, block)
 * pairs. Every value it computes has a plain definition, which the code writes out.
 *
 * What it computes, per decode row b (one decode token) and index head h:
 *
 *   block score   S[b][h][j] = max over the valid tokens t of block j of
 *                              sum_d q[b][h][d] * k[page][t][d]
 *       - The four index heads share one index-K head, so one page is scored
 *         for all heads (vLLM PR #57832, "Problem"; SGLang PR #41488,
 *         "Motivation" and "Modifications": four heads, dim 128, 128-token
 *         blocks, max scoring).
 *       - A block's score is the max over its tokens; the max starts at -inf
 *         (TensorRT-LLM PR #17008, "Description" calls the pass a max-score
 *         pass; "Accuracy" seeds each per-tile max at -infinity).
 *       - The visible tokens of a single decode token are all seq_len context
 *         tokens: the causal clamp min(q_end + offset_q, kv_len) equals kv_len
 *         for the last query position (TensorRT-LLM PR #17008, "Description").
 *         Tokens of the partial last block past seq_len are not scored.
 *       - No positive scale is applied: top-k order does not change under one
 *         (vLLM blog "Following the Bottleneck", section 2, "What work repeats?").
 *       - Logical block j lives in physical page block_table[b][j]; a page holds
 *         128 tokens x 128 dims (vLLM PR #57832 runs with --block-size 128;
 *         vLLM blog section 3 maps selected logical blocks to physical pages).
 *
 *   selection     the top m = min(topk, nb) blocks of each (b, h), where nb is
 *                 the number of blocks in row b:
 *       - selection is per index head; heads are never mixed (vLLM PR #57832,
 *         "Solution" steps 3-4 and the withdrawn head-mixing design in
 *         "Test Result");
 *       - the first n_init blocks and the last n_local blocks are pinned and
 *         always selected (vLLM PR #57832, "Solution": forced init/sink and
 *         sliding-window blocks; SGLang PR #41488: initial/recent priorities);
 *       - order: pinned first, then higher score, then lower block id (ties
 *         broken by ascending id); scores compare numerically, so -0 == +0;
 *       - slots m .. topk-1 hold id -1 and score -inf; an empty row has none.
 *
 *   page table    for a sparse-attention consumer that reads 16-token pages (vLLM blog
 *                 "Following the Bottleneck", section 3 and Figure 5: each selected
 *                 128-token block resolves to its physical block, whose eight 16-token
 *                 pages make eight entries of a compact page table; the cache itself is
 *                 not copied). Per (b, h): the selected blocks in ascending logical order;
 *                 the i-th gives entries 8i .. 8i+7 = 8 * block_table[b][j] + t; entries
 *                 past the selected blocks are -1; the table's token count is the sum of
 *                 the selected blocks' valid tokens.
 *
 *   multi-token   a row that verifies Q draft tokens (speculative decoding) carries Q query
 *   decode        positions q[b][p], p < Q, the last Q tokens of its context (vLLM blog
 *                 "Following the Bottleneck", section 2: one workgroup per request scores all
 *                 draft positions; vLLM PR #57832, Test Plan: query_len 4 verifies). Under the
 *                 causal clamp min(q_end + offset_q, kv_len) of TensorRT-LLM PR #17008
 *                 ("Description"), position p sees the first L_p = L - (Q - 1 - p) tokens,
 *                 L the row's clamped length (L_p floored at 0). Each (b, p, h) is exactly the
 *                 single-token pass above with q[b][p] and length L_p.
 *
 *   fp8 cache     the index-K cache may hold FP8 E4M3 codes instead of bf16 (SGLang PR #41488,
 *                 Accuracy and Speed Tests: BF16 queries with an FP8 E4M3 index cache). The
 *                 pages fix no scale; the reading taken here: OCP E4M3 (the MI355X format:
 *                 exponent bias 7, three mantissa bits, subnormals, no infinities, S.1111.111
 *                 is NaN and outside the contract), one positive scale per cache, so the key
 *                 is k_scale * value(code). A positive scale cannot reorder blocks (vLLM blog,
 *                 section 2), so the selection does not depend on it.
 *
 * bf16 inputs are widened exactly (bits << 16 is the fp32 value; fp32 -> fp64
 * is exact), products of two bf16 values are exact in fp64, and the 128-term
 * sums are accumulated in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_HEADS 4
#define OR_DIM 128
#define OR_BLOCK 128

#define OR_OK 0
#define OR_ERR_ARG -1
#define OR_ERR_PAGE -2
#define OR_ERR_NONFINITE -3

static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal. */
static double widen_e4m3(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return sign ? -mag : mag;
}

static int64_t row_len(const int32_t *seq_lens, int32_t b, int32_t max_blocks)
{
    int64_t L = seq_lens[b];
    int64_t cap = (int64_t)max_blocks * OR_BLOCK;
    if (L < 0) L = 0;
    if (L > cap) L = cap;
    return L;
}

int msa_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads later calls use (for timing the oracle on one core and on all of them). */
void msa_oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Block scores, out[b][h][j] for j < max_blocks (fp64). Blocks at or past the
 * row's end hold -inf. Returns OR_ERR_PAGE if a block the row needs maps to a
 * page outside [0, num_pages).
 */
static int block_scores_impl(const uint16_t *q, const void *k_cache, int kv_fp8, double k_scale,
                             const int32_t *block_table, const int32_t *seq_lens,
                             int32_t batch, int32_t max_blocks, int32_t bt_stride,
                             int64_t num_pages, double *out)
{
    if (batch < 0 || max_blocks < 0 || bt_stride < max_blocks) return OR_ERR_ARG;
    int64_t total = (int64_t)batch * max_blocks;
    int status = OR_OK;

#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t bj = 0; bj < total; ++bj) {
        int32_t b = (int32_t)(bj / max_blocks);
        int32_t j = (int32_t)(bj % max_blocks);
        int64_t L = row_len(seq_lens, b, max_blocks);
        int64_t nb = (L + OR_BLOCK - 1) / OR_BLOCK;
        double best[OR_HEADS];
        for (int h = 0; h < OR_HEADS; ++h) best[h] = -INFINITY;

        if (j < nb) {
            int64_t page = block_table[(int64_t)b * bt_stride + j];
            if (page < 0 || page >= num_pages) {
#pragma omp atomic write
                status = OR_ERR_PAGE;
            } else {
                int64_t valid = L - (int64_t)j * OR_BLOCK;
                if (valid > OR_BLOCK) valid = OR_BLOCK;
                for (int64_t t = 0; t < valid; ++t) {
                    int64_t tok = (page * OR_BLOCK + t) * OR_DIM;
                    double kt[OR_DIM];
                    if (kv_fp8) {
                        const uint8_t *k8 = (const uint8_t *)k_cache + tok;
                        for (int d = 0; d < OR_DIM; ++d) kt[d] = k_scale * widen_e4m3(k8[d]);
                    } else {
                        const uint16_t *k16 = (const uint16_t *)k_cache + tok;
                        for (int d = 0; d < OR_DIM; ++d) kt[d] = widen_bf16(k16[d]);
                    }
                    for (int h = 0; h < OR_HEADS; ++h) {
                        const uint16_t *qh = q + ((int64_t)b * OR_HEADS + h) * OR_DIM;
                        double s = 0.0;
                        for (int d = 0; d < OR_DIM; ++d) s += widen_bf16(qh[d]) * kt[d];
                        if (s > best[h]) best[h] = s;
                    }
                }
                for (int h = 0; h < OR_HEADS; ++h) {
                    if (!isfinite(best[h])) {
#pragma omp atomic write
                        status = OR_ERR_NONFINITE;
                    }
                }
            }
        }
        for (int h = 0; h < OR_HEADS; ++h)
            out[((int64_t)b * OR_HEADS + h) * max_blocks + j] = best[h];
    }
    return status;
}

int msa_oracle_block_scores(const uint16_t *q, const uint16_t *k_cache,
                            const int32_t *block_table, const int32_t *seq_lens,
                            int32_t batch, int32_t max_blocks, int32_t bt_stride,
                            int64_t num_pages, double *out)
{
    return block_scores_impl(q, k_cache, 0, 1.0, block_table, seq_lens, batch, max_blocks,
                             bt_stride, num_pages, out);
}

/* Block scores over an FP8 E4M3 cache k_cache[page][token][dim] (one byte per element). */
int msa_oracle_block_scores_fp8(const uint16_t *q, const uint8_t *k_cache, double k_scale,
                                const int32_t *block_table, const int32_t *seq_lens,
                                int32_t batch, int32_t max_blocks, int32_t bt_stride,
                                int64_t num_pages, double *out)
{
    if (!(k_scale > 0.0) || !isfinite(k_scale)) return OR_ERR_ARG;
    return block_scores_impl(q, k_cache, 1, k_scale, block_table, seq_lens, batch, max_blocks,
                             bt_stride, num_pages, out);
}

typedef struct {
    int pinned;
    double score;
    int32_t id;
} cand_t;

/* pinned first, then higher score, then lower id */
static int cand_order(const void *pa, const void *pb)
{
    const cand_t *a = (const cand_t *)pa, *b = (const cand_t *)pb;
    if (a->pinned != b->pinned) return a->pinned ? -1 : 1;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id);
}

/*
 * Pinned top-k per (row, head) from block scores scores[b][h][j] (j < max_blocks).
 * Writes out_ids[b][h][i] and out_scores[b][h][i] for i < topk.
 */
int msa_oracle_select(const double *scores, const int32_t *seq_lens,
                      int32_t batch, int32_t max_blocks, int32_t topk,
                      int32_t n_init, int32_t n_local,
                      int32_t *out_ids, double *out_scores)
{
    if (batch < 0 || max_blocks < 0 || topk < 1 || n_init < 0 || n_local < 0)
        return OR_ERR_ARG;
    int status = OR_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)batch * OR_HEADS; ++bh) {
        int32_t b = (int32_t)(bh / OR_HEADS);
        int64_t L = row_len(seq_lens, b, max_blocks);
        int64_t nb = (L + OR_BLOCK - 1) / OR_BLOCK;
        int64_t m = nb < topk ? nb : topk;
        const double *row = scores + bh * max_blocks;
        cand_t *c = (cand_t *)malloc((size_t)(nb > 0 ? nb : 1) * sizeof(cand_t));
        if (!c) {
#pragma omp atomic write
            status = OR_ERR_ARG;
            continue;
        }
        for (int64_t j = 0; j < nb; ++j) {
            c[j].pinned = (j < n_init) || (j >= nb - n_local);
            c[j].score = row[j];
            c[j].id = (int32_t)j;
        }
        qsort(c, (size_t)nb, sizeof(cand_t), cand_order);
        for (int64_t i = 0; i < topk; ++i) {
            out_ids[bh * topk + i] = i < m ? c[i].id : -1;
            out_scores[bh * topk + i] = i < m ? c[i].score : -INFINITY;
        }
        free(c);
    }
    return status;
}

/* Both steps: block scores into scratch (caller-sized [batch][4][max_blocks]), then selection. */
int msa_oracle_decode(const uint16_t *q, const uint16_t *k_cache,
                      const int32_t *block_table, const int32_t *seq_lens,
                      int32_t batch, int32_t max_blocks, int32_t bt_stride,
                      int64_t num_pages, int32_t topk, int32_t n_init, int32_t n_local,
                      double *scratch_scores, int32_t *out_ids, double *out_scores)
{
    int rc = msa_oracle_block_scores(q, k_cache, block_table, seq_lens, batch, max_blocks,
                                     bt_stride, num_pages, scratch_scores);
    if (rc != OR_OK) return rc;
    return msa_oracle_select(scratch_scores, seq_lens, batch, max_blocks, topk, n_init,
                             n_local, out_ids, out_scores);
}

static int cmp_int(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * 16-token page tables from selections ids[b][h][i] (i < topk): pages[b][h][8*topk],
 * tokens[b][h]. An id outside [0, nb) stands for no block (-1 pads a short selection);
 * a repeated id is expanded each time it appears. The entry is 8 * page + t modulo 2^32.
 */
int msa_oracle_expand_pages(const int32_t *ids, const int32_t *block_table, const int32_t *seq_lens,
                            int32_t batch, int32_t max_blocks, int32_t bt_stride, int32_t topk,
                            int32_t *pages, int32_t *tokens)
{
    if (batch < 0 || max_blocks < 0 || bt_stride < max_blocks || topk < 1 || topk > 256)
        return OR_ERR_ARG;
    for (int64_t bh = 0; bh < (int64_t)batch * OR_HEADS; ++bh) {
        int32_t b = (int32_t)(bh / OR_HEADS);
        int64_t L = row_len(seq_lens, b, max_blocks);
        int64_t nb = (L + OR_BLOCK - 1) / OR_BLOCK;
        int32_t sel[256];
        int n = 0;
        for (int i = 0; i < topk; ++i) {
            int32_t j = ids[bh * topk + i];
            if (j >= 0 && j < nb) sel[n++] = j;
        }
        qsort(sel, (size_t)n, sizeof(int32_t), cmp_int);
        int32_t *row = pages + bh * topk * 8;
        for (int64_t e = 0; e < (int64_t)topk * 8; ++e) row[e] = -1;
        int64_t count = 0;
        for (int i = 0; i < n; ++i) {
            int32_t j = sel[i];
            int64_t page = block_table[(int64_t)b * bt_stride + j];
            for (int t = 0; t < 8; ++t) row[i * 8 + t] = (int32_t)(uint32_t)(page * 8 + t);
            int64_t valid = L - (int64_t)j * OR_BLOCK;
            count += valid > OR_BLOCK ? OR_BLOCK : valid;
        }
        tokens[bh] = (int32_t)count;
    }
    return OR_OK;
}

/*
 * Multi-token decode: q[b][p][h][d] for p < qlen; block scores out_blocks[b][p][h][j]
 * (j < max_blocks), selections out_ids / out_scores [b][p][h][topk]. Each position is run
 * through msa_oracle_decode with its own query and causal length.
 */
static int decode_multi_impl(const uint16_t *q, const void *k_cache, int kv_fp8, double k_scale,
                             const int32_t *block_table, const int32_t *seq_lens,
                             int32_t batch, int32_t max_blocks, int32_t bt_stride,
                             int64_t num_pages, int32_t qlen, int32_t topk, int32_t n_init,
                             int32_t n_local, double *out_blocks, int32_t *out_ids,
                             double *out_scores)
{
    if (batch < 0 || max_blocks < 0 || qlen < 1 || topk < 1) return OR_ERR_ARG;
    size_t nb_q = (size_t)batch * OR_HEADS * OR_DIM;
    size_t nb_s = (size_t)batch * OR_HEADS * (size_t)max_blocks;
    size_t nb_k = (size_t)batch * OR_HEADS * (size_t)topk;
    uint16_t *qp = (uint16_t *)malloc((nb_q ? nb_q : 1) * sizeof(uint16_t));
    int32_t *lens_p = (int32_t *)malloc((batch ? batch : 1) * sizeof(int32_t));
    double *sc = (double *)malloc((nb_s ? nb_s : 1) * sizeof(double));
    int32_t *ids = (int32_t *)malloc((nb_k ? nb_k : 1) * sizeof(int32_t));
    double *sel = (double *)malloc((nb_k ? nb_k : 1) * sizeof(double));
    int rc = (qp && lens_p && sc && ids && sel) ? OR_OK : OR_ERR_ARG;
    for (int32_t p = 0; p < qlen && rc == OR_OK; ++p) {
        for (int32_t b = 0; b < batch; ++b) {
            int64_t L = row_len(seq_lens, b, max_blocks) - (qlen - 1 - p);
            lens_p[b] = (int32_t)(L > 0 ? L : 0);
            memcpy(qp + (size_t)b * OR_HEADS * OR_DIM,
                   q + ((size_t)b * qlen + p) * OR_HEADS * OR_DIM,
                   OR_HEADS * OR_DIM * sizeof(uint16_t));
        }
        rc = block_scores_impl(qp, k_cache, kv_fp8, k_scale, block_table, lens_p, batch,
                               max_blocks, bt_stride, num_pages, sc);
        if (rc == OR_OK)
            rc = msa_oracle_select(sc, lens_p, batch, max_blocks, topk, n_init, n_local, ids, sel);
        for (int32_t b = 0; b < batch && rc == OR_OK; ++b) {
            size_t o = (size_t)b * qlen + p;
            memcpy(out_blocks + o * OR_HEADS * max_blocks, sc + (size_t)b * OR_HEADS * max_blocks,
                   (size_t)OR_HEADS * max_blocks * sizeof(double));
            memcpy(out_ids + o * OR_HEADS * topk, ids + (size_t)b * OR_HEADS * topk,
                   (size_t)OR_HEADS * topk * sizeof(int32_t));
            memcpy(out_scores + o * OR_HEADS * topk, sel + (size_t)b * OR_HEADS * topk,
                   (size_t)OR_HEADS * topk * sizeof(double));
        }
    }
    free(qp);
    free(lens_p);
    free(sc);
    free(ids);
    free(sel);
    return rc;
}

int msa_oracle_decode_multi(const uint16_t *q, const uint16_t *k_cache,
                            const int32_t *block_table, const int32_t *seq_lens,
                            int32_t batch, int32_t max_blocks, int32_t bt_stride,
                            int64_t num_pages, int32_t qlen, int32_t topk, int32_t n_init,
                            int32_t n_local, double *out_blocks, int32_t *out_ids,
                            double *out_scores)
{
    return decode_multi_impl(q, k_cache, 0, 1.0, block_table, seq_lens, batch, max_blocks,
                             bt_stride, num_pages, qlen, topk, n_init, n_local, out_blocks,
                             out_ids, out_scores);
}

/* Multi-token decode (qlen >= 1) over an FP8 E4M3 cache with scale k_scale > 0. */
int msa_oracle_decode_multi_fp8(const uint16_t *q, const uint8_t *k_cache, double k_scale,
                                const int32_t *block_table, const int32_t *seq_lens,
                                int32_t batch, int32_t max_blocks, int32_t bt_stride,
                                int64_t num_pages, int32_t qlen, int32_t topk, int32_t n_init,
                                int32_t n_local, double *out_blocks, int32_t *out_ids,
                                double *out_scores)
{
    if (!(k_scale > 0.0) || !isfinite(k_scale)) return OR_ERR_ARG;
    return decode_multi_impl(q, k_cache, 1, k_scale, block_table, seq_lens, batch, max_blocks,
                             bt_stride, num_pages, qlen, topk, n_init, n_local, out_blocks,
                             out_ids, out_scores);
}

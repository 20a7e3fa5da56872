/*
 * qsa_oracle.c -- plain, single-threaded CPU oracle of the QSA sparse-attention
 * decode step (indexer scoring, C4 block reduce, budgeted block selection,
 * page-table lookup, GQA softmax attention over the selected tokens).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this code. It shares nothing with the HIP library: no
 * header, no helper, no table. It is written for a reader who checks it by eye
 * against the pages, so it has no blocking, fusion or reordering: every sum runs
 * over its index in increasing order, in IEEE double, and results are rounded to
 * float only where they are stored.
 *
 * Sources:
 *  - "双卡RTX4090跑通Qwen3-Next" (kongchang.com), intro and the memory-ledger
 *    section: selection works on C4 blocks of 4 adjacent tokens, each QSA layer
 *    selects on its own, and logical token addresses are kept apart from
 *    physical cache slots (page table); attention anchors to the start of the
 *    sequence (sink) and a tail ring buffer exists.
 *  - "Оффлоадинг KV-кэша Qwen3.8-Flash-Next в RAM" (digest.ninitux.com), lead
 *    paragraph and the mechanism / efficiency sections: a GPU-resident index of
 *    compressed keys of 66 bytes per token per layer picks at most
 *    indexer_budget = 2048 positions; only those KV rows (2048 bytes per token
 *    per layer) are read.
 *  - The indexer score formula, dtypes and head geometry are not on the pages;
 *    the workload definition gives score = sum_h w_h * ReLU(q_h . k) over 4
 *    indexer heads of dim 64, fp8 e4m3 keys with one fp16 scale per token, and
 *    16 query heads over 2 KV heads of dim 256 in bf16.
 *
 * Readings taken where the pages are silent: the fp16 scale multiplies the
 * dot product inside the ReLU; e4m3 is the OCP "fn" variant (bias 7, max 448,
 * no infinities); a partial last block takes the max over its valid tokens
 * only; forced sink/tail blocks count inside the budget; ties break by lower
 * block index; the selection is returned in ascending block order; query head
 * h reads KV head h / (n_q_heads / n_kv_heads); the softmax scale is given by
 * the caller (1/sqrt(head_dim)), with no soft-cap; an empty token set gives a
 * zero output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there are
 * no infinities, so S.1111.110 = 448 is the largest finite magnitude. */
double qo_decode_e4m3(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* IEEE 754 binary16: 1 sign, 5 exponent bits (bias 15), 10 mantissa bits. */
double qo_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double mag;
    if (e == 31)
        mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m, -24);
    else
        mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double qo_decode_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------- indexer scoring */

/* Token scores of one sequence in one layer.
 *   keys   [L][idx_dim]  e4m3 codes (logical token order)
 *   scales [L]           fp16 bits, one dequantisation scale per token
 *   q_idx  [idx_heads][idx_dim] bf16 bits (indexer query)
 *   w      [idx_heads]   fp32 head weights
 *   out    [L]           fp32: s_t = sum_h w_h * max(0, sigma_t * (q_h . k_t))
 */
void qo_token_scores(int64_t L, int idx_heads, int idx_dim, const uint8_t *keys,
                     const uint16_t *scales, const uint16_t *q_idx, const float *w,
                     float *out)
{
    for (int64_t t = 0; t < L; t++) {
        double sigma = qo_decode_f16(scales[t]);
        double s = 0.0;
        for (int h = 0; h < idx_heads; h++) {
            double d = 0.0;
            for (int i = 0; i < idx_dim; i++)
                d += qo_decode_bf16(q_idx[h * idx_dim + i]) *
                     qo_decode_e4m3(keys[t * idx_dim + i]);
            double x = sigma * d;
            if (x < 0.0)
                x = 0.0;
            s += (double)w[h] * x;
        }
        out[t] = (float)s;
    }
}

/* C4 block reduce: block j covers tokens [bt*j, min(bt*j + bt, L)); its score
 * is the largest fp32 token score among those tokens. */
void qo_block_scores(int64_t L, int bt, const float *token_scores, float *block_scores)
{
    int64_t n_blk = (L + bt - 1) / bt;
    for (int64_t j = 0; j < n_blk; j++) {
        int64_t t0 = j * bt;
        int64_t t1 = t0 + bt < L ? t0 + bt : L;
        float best = token_scores[t0];
        for (int64_t t = t0 + 1; t < t1; t++)
            if (token_scores[t] > best)
                best = token_scores[t];
        block_scores[j] = best;
    }
}

/* ----------------------------------------------------------- selection */

/* Forced blocks: the first sink_blocks blocks (attention sink at the start of
 * the sequence) and, when tail_tokens > 0, every block that holds one of the
 * last tail_tokens tokens (the tail ring). mask[j] = 1 for forced block j. */
int64_t qo_forced_mask(int64_t L, int bt, int64_t sink_blocks, int64_t tail_tokens,
                       uint8_t *mask)
{
    int64_t n_blk = (L + bt - 1) / bt;
    int64_t count = 0;
    int64_t tail_first = n_blk;
    if (tail_tokens > 0) {
        int64_t first_tok = L - tail_tokens;
        if (first_tok < 0)
            first_tok = 0;
        tail_first = first_tok / bt;
    }
    for (int64_t j = 0; j < n_blk; j++) {
        mask[j] = (j < sink_blocks || j >= tail_first) ? 1 : 0;
        count += mask[j];
    }
    return count;
}

typedef struct {
    float score;
    int32_t index;
} qo_scored_block;

/* Order: higher score first; among equal scores, lower block index first. */
static int qo_cmp_blocks(const void *pa, const void *pb)
{
    const qo_scored_block *a = (const qo_scored_block *)pa;
    const qo_scored_block *b = (const qo_scored_block *)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->index > b->index) - (a->index < b->index);
}

static int qo_cmp_int32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/* Budgeted block selection. K = budget in blocks. Returns |S| (or -1 when the
 * forced blocks alone exceed K); writes S in ascending block order to sel[0..|S|)
 * and the score of the last non-forced block taken to *kth_score (NaN when no
 * non-forced block was taken, or when every block fits in the budget).
 *   S = all blocks                         if n_blk <= K
 *   S = F + the first K-|F| blocks of the rest sorted by (score desc, index asc)
 */
int64_t qo_select_blocks(int64_t n_blk, const float *block_scores, int64_t K,
                         const uint8_t *forced, int32_t *sel, float *kth_score)
{
    *kth_score = NAN;
    if (n_blk <= K) {
        for (int64_t j = 0; j < n_blk; j++)
            sel[j] = (int32_t)j;
        return n_blk;
    }
    int64_t n_forced = 0;
    for (int64_t j = 0; j < n_blk; j++)
        n_forced += forced ? forced[j] : 0;
    if (n_forced > K)
        return -1;

    qo_scored_block *rest = (qo_scored_block *)malloc(sizeof(qo_scored_block) * (size_t)n_blk);
    int64_t n_rest = 0, n_sel = 0;
    for (int64_t j = 0; j < n_blk; j++) {
        if (forced && forced[j])
            sel[n_sel++] = (int32_t)j;
        else {
            rest[n_rest].score = block_scores[j];
            rest[n_rest].index = (int32_t)j;
            n_rest++;
        }
    }
    qsort(rest, (size_t)n_rest, sizeof(qo_scored_block), qo_cmp_blocks);
    int64_t take = K - n_forced;
    for (int64_t i = 0; i < take; i++)
        sel[n_sel++] = rest[i].index;
    if (take > 0)
        *kth_score = rest[take - 1].score;
    free(rest);
    qsort(sel, (size_t)n_sel, sizeof(int32_t), qo_cmp_int32);
    return n_sel;
}

/* Tokens of the selected blocks, ascending: the union of [bt*j, min(bt*j+bt, L)). */
int64_t qo_tokens_of_blocks(int64_t L, int bt, const int32_t *sel, int64_t n_sel, int64_t *tokens)
{
    int64_t n = 0;
    for (int64_t i = 0; i < n_sel; i++) {
        int64_t t0 = (int64_t)sel[i] * bt;
        for (int64_t t = t0; t < t0 + bt && t < L; t++)
            tokens[n++] = t;
    }
    return n;
}

/* ----------------------------------------------------------- attention */

/* GQA softmax attention of one query over a set of cached tokens.
 *   tokens [n_tok]   logical token positions
 *   pt     [.]       logical token -> physical slot; NULL means slot = token
 *   pool   [n_slots][2 * n_kv_heads * head_dim] bf16 bits; a row holds the keys
 *                    of every KV head, then the values of every KV head
 *   q      [n_q_heads][head_dim] bf16 bits
 *   out    [n_q_heads][head_dim] fp32
 * For head h with KV head g = h / (n_q_heads / n_kv_heads):
 *   z_t = sm_scale * (q_h . K_{g,t}),  p_t = exp(z_t - max z) / sum exp(z - max z),
 *   out_h = sum_t p_t V_{g,t}.
 */
void qo_attention(int64_t n_tok, const int64_t *tokens, const int32_t *pt,
                  const uint16_t *pool, int n_q_heads, int n_kv_heads, int head_dim,
                  const uint16_t *q, double sm_scale, float *out)
{
    int64_t row = 2 * (int64_t)n_kv_heads * head_dim;
    int group = n_q_heads / n_kv_heads;
    double *z = (double *)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);
    for (int h = 0; h < n_q_heads; h++) {
        int g = h / group;
        if (n_tok == 0) {
            for (int i = 0; i < head_dim; i++)
                out[h * head_dim + i] = 0.0f;
            continue;
        }
        double zmax = -INFINITY;
        for (int64_t t = 0; t < n_tok; t++) {
            int64_t slot = pt ? (int64_t)pt[tokens[t]] : tokens[t];
            const uint16_t *k = pool + slot * row + (int64_t)g * head_dim;
            double d = 0.0;
            for (int i = 0; i < head_dim; i++)
                d += qo_decode_bf16(q[h * head_dim + i]) * qo_decode_bf16(k[i]);
            z[t] = sm_scale * d;
            if (z[t] > zmax)
                zmax = z[t];
        }
        double denom = 0.0;
        for (int i = 0; i < head_dim; i++)
            acc[i] = 0.0;
        for (int64_t t = 0; t < n_tok; t++) {
            int64_t slot = pt ? (int64_t)pt[tokens[t]] : tokens[t];
            const uint16_t *v = pool + slot * row + (int64_t)(n_kv_heads + g) * head_dim;
            double e = exp(z[t] - zmax);
            denom += e;
            for (int i = 0; i < head_dim; i++)
                acc[i] += e * qo_decode_bf16(v[i]);
        }
        for (int i = 0; i < head_dim; i++)
            out[h * head_dim + i] = (float)(acc[i] / denom);
    }
    free(acc);
    free(z);
}

/* ------------------------------------------------------ one layer, whole */

/* The decode step of one sequence in one QSA layer, in the order the method
 * takes: score every cached token, reduce to C4 blocks, select the budget,
 * expand to tokens, attend through the page table. Every output pointer may be
 * NULL except out. Returns |S| (blocks selected) or -1 on a forced-set overflow. */
int64_t qo_decode_layer(int64_t L, int idx_heads, int idx_dim, int bt, int64_t budget_tokens,
                        int64_t sink_blocks, int64_t tail_tokens,
                        const uint8_t *keys, const uint16_t *scales,
                        const uint16_t *q_idx, const float *w,
                        const uint16_t *q, const int32_t *pt, const uint16_t *pool,
                        int n_q_heads, int n_kv_heads, int head_dim, double sm_scale,
                        float *token_scores_out, float *block_scores_out,
                        int32_t *sel_out, float *kth_out, int64_t *n_tok_out, float *out)
{
    int64_t n_blk = (L + bt - 1) / bt;
    int64_t K = budget_tokens / bt;
    float *ts = (float *)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1));
    float *bs = (float *)malloc(sizeof(float) * (size_t)(n_blk > 0 ? n_blk : 1));
    uint8_t *mask = (uint8_t *)malloc((size_t)(n_blk > 0 ? n_blk : 1));
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_blk > 0 ? n_blk : 1));
    int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(L > 0 ? L : 1));
    float kth = NAN;

    qo_token_scores(L, idx_heads, idx_dim, keys, scales, q_idx, w, ts);
    qo_block_scores(L, bt, ts, bs);
    qo_forced_mask(L, bt, sink_blocks, tail_tokens, mask);
    int64_t n_sel = qo_select_blocks(n_blk, bs, K, mask, sel, &kth);
    int64_t n_tok = 0;
    if (n_sel >= 0) {
        n_tok = qo_tokens_of_blocks(L, bt, sel, n_sel, tok);
        qo_attention(n_tok, tok, pt, pool, n_q_heads, n_kv_heads, head_dim, q, sm_scale, out);
    }
    if (token_scores_out)
        memcpy(token_scores_out, ts, sizeof(float) * (size_t)L);
    if (block_scores_out)
        memcpy(block_scores_out, bs, sizeof(float) * (size_t)n_blk);
    if (sel_out && n_sel > 0)
        memcpy(sel_out, sel, sizeof(int32_t) * (size_t)n_sel);
    if (kth_out)
        *kth_out = kth;
    if (n_tok_out)
        *n_tok_out = n_tok;
    free(tok);
    free(sel);
    free(mask);
    free(bs);
    free(ts);
    return n_sel;
}

/* ------------------------------------------------------------ append step */

/* The new token of a decode step gets an index row and a KV row. Sources:
 * "双卡RTX4090跑通Qwen3-Next" (kongchang.com), memory-ledger section: the
 * index, its quantisation scales and the page layout are kept together, and
 * a new token's logical address maps to a physical cache slot; the workload
 * definition fixes fp8 e4m3 keys with one fp16 scale per token. Reading taken
 * where the pages are silent: the scale is the key's largest magnitude over
 * 448 (the largest e4m3 value), rounded to fp16, and every element is x / scale
 * rounded to the nearest e4m3 value; both divisions are done in binary32, the
 * precision the stored format implies (an fp32 key, an fp16 scale).
 *
 * The encoders below search every code for the nearest value instead of
 * manipulating bits, so they can be checked against the decoders by eye. */

/* Nearest binary16 value to a non-negative double, ties to the even code;
 * values of 65520 and above round to +infinity. Returns the bits. */
uint16_t qo_encode_f16(double x)
{
    if (!(x >= 0.0))
        return 0x7E00;                  /* NaN; negative inputs are not used */
    if (x >= 65520.0)
        return 0x7C00;
    uint16_t best = 0;
    double best_d = INFINITY;
    for (uint32_t c = 0; c < 0x7C00; c++) {
        double d = fabs(qo_decode_f16((uint16_t)c) - x);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = (uint16_t)c;
            best_d = d;
        }
    }
    return best;
}

/* Nearest e4m3 value to y, ties to the even code, magnitudes beyond 448
 * clamped to 448 (saturation); the sign follows y. */
uint8_t qo_encode_e4m3(double y)
{
    double a = fabs(y);
    uint8_t best = 0;
    if (a >= 448.0) {
        best = 0x7E;
    } else {
        double best_d = INFINITY;
        for (uint32_t c = 0; c <= 0x7E; c++) {
            double d = fabs(qo_decode_e4m3((uint8_t)c) - a);
            if (d < best_d || (d == best_d && (c & 1) == 0)) {
                best = (uint8_t)c;
                best_d = d;
            }
        }
    }
    return signbit(y) ? (uint8_t)(best | 0x80) : best;
}

/* Quantise one index key of n elements: scale bits and n e4m3 codes.
 *   sigma = f16(fl32(amax / 448)), code_i = e4m3(fl32(x_i / sigma)),
 * with all codes 0 when sigma is 0. */
void qo_quantise_key(int n, const float *x, uint8_t *codes, uint16_t *scale_bits)
{
    float amax = 0.0f;
    for (int i = 0; i < n; i++) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float ratio = amax / 448.0f;
    uint16_t s = qo_encode_f16((double)ratio);
    float sigma = (float)qo_decode_f16(s);
    for (int i = 0; i < n; i++) {
        if (sigma > 0.0f) {
            float y = x[i] / sigma;
            codes[i] = qo_encode_e4m3((double)y);
        } else {
            codes[i] = 0;
        }
    }
    *scale_bits = s;
}

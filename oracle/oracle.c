/*
 * CPU oracle for the candidate-consuming sparse MQA-logits indexer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the package's smoke() entry and the
 * CPU-baseline leg of bench.py may load this library.  The GPU product path
 * never calls it, and it shares no code, header or table with that path.
 *
 * What it computes (plain definitions, written out; no blocking, fusion or
 * reordering beyond what the definitions state):
 *
 *  - Decoding of the quantised formats, from their bit definitions in the OCP
 *    Microscaling Formats (MX) v1.0 specification: e2m1 (FP4) elements, UE8M0
 *    (E8M0) block scales with one scale per 32 elements, and OCP e4m3fn (FP8)
 *    elements.  The pages require the MXFP4 indexer K cache with power-of-two
 *    scales of granularity 32 (vLLM DeepSeek-V4.1 sparse indexer backend page,
 *    DeepseekV41SparseIndexerMetadataBuilder.__init__ checks).
 *
 *  - The candidate column set of a row: the candidate-source layer publishes
 *    candidate blocks, and a consuming layer scores only the tokens inside them
 *    (vllm.model_executor.layers.sparse_mqa_indexer page, module summary); the
 *    row's K range is [ks, ke) (same backend page, SparseMQARowsMetadata
 *    fields row_ks / row_ke).
 *
 *  - MQA logits with a per-head weighted head reduce (sparse_mqa_indexer page,
 *    SparseMQAIndexer.forward; rocm_paged_mxfp4_indexer page,
 *    RocmSparseMQAIndexer.weights_dtype: weights and logits are fp32 on gfx950):
 *        logit[t] = sum_h w[h] * max(q_h . k_t, 0),
 *    accumulated in fp64 and rounded once to fp32 (round to nearest even).
 *
 *  - Top-k selection: count = min(topk, |T|) tokens with the largest fp32
 *    logits, ties toward the lower token index, -0 equal to +0; chosen tokens
 *    are written in ascending token order and the slots after them hold -1
 *    (SparseMQAIndexer.forward fills the index buffer with -1 before scoring).
 *
 *  - The bf16 scoring variant, the SM100 layer's semantics: the per-head
 *    weights are bfloat16 (sparse_mqa_indexer page, SparseMQAIndexer
 *    weights_dtype) and the top-k runs on the kernels' bf16 logits with no fp32
 *    fallback (backend source page, DeepseekV41SparseIndexerMetadataBuilder
 *    __init__, the DeepSelect comment).  Reading: the weights are widened
 *    exactly, the logit is the same sum, and its exact value is rounded once to
 *    the nearest bf16 (ties to the even significand) before the selection,
 *    whose tie rule is unchanged.
 *
 *  - The candidate-source layer's publication of the candidate pool (the
 *    rocm_paged_mxfp4_indexer page: RocmSparseAttnIndexer, whose forward_hip
 *    hands candidate_blocks and candidate_write to the dense indexer; the
 *    sparse_mqa_indexer page's summary: the source layer publishes the top
 *    candidate blocks).  The pages give no pooling rule; the reading taken:
 *    the source scores every token of the row's [ks, ke) with the same
 *    per-token logit, a block of cbs tokens scores the largest logit among
 *    its tokens in [ks, ke), and the row publishes the NB blocks with the
 *    largest scores (ties toward the lower block id), ascending, then -1.
 *
 *  - The sparse-column schedule: each candidate block of cbs tokens becomes
 *    cbs/sbk sparse blocks of sbk tokens; sparse_indices lists the sparse
 *    blocks that hold a token of [ks, ke), ascending, padded with -1; end is
 *    the number of valid tokens (backend page: num_sparse_blocks computed in
 *    the builder __init__; SparseMQARowsMetadata.sparse_indices / .end).
 *
 * NaN inputs (the pages say nothing of them): ReLU maps a NaN dot product (from
 * a UE8M0 scale byte 0xFF or an e4m3 NaN code) to 0, as C's fmax and IEEE 754
 * maxNum do, so it contributes nothing; a NaN logit (a NaN or infinite weight)
 * ranks as -inf.
 *
 * Points the pages leave open are read as follows, each restated where used:
 * negative candidate ids are padding, repeated ids count once, element 2i of a
 * packed e2m1 vector is the low nibble of byte i, scale byte j covers elements
 * [32j, 32j+32), and a cache page holds its packed values [page][D/2] and its
 * scale bytes [page][D/32] at two independently strided base pointers.
 *
 * Parity pins: every function here is pinned by a CPU test against hand-worked
 * decodes and roundings, library decodes and conversions (torch float8_e4m3fn /
 * float8_e8m0fnu / bfloat16), closed forms, an independent dense-then-mask
 * brute force and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q_MXFP4 0
#define ORC_Q_FP8 1
#define ORC_SCORE_FP32 0
#define ORC_SCORE_BF16 1

/* ---- element and scale decoding (OCP MX v1.0) ------------------------------ */

/* e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0
 * encodes subnormals m * 2^-1.  No inf/NaN encodings.  Code 0x8 is -0. */
double orc_e2m1(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* UE8M0: an unsigned biased exponent, value 2^(b-127); 0xFF is NaN. */
double orc_ue8m0(int b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, b - 127);
}

/* e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; no infinities. */
double orc_e4m3fn(int b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double mag;
    if (e == 15 && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp(m / 8.0, -6);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* bf16 (bfloat16): 1 sign bit, 8 exponent bits (bias 127), 7 mantissa bits;
 * exponent field 0 encodes subnormals m/128 * 2^-126, field 255 infinity (m = 0)
 * or NaN. */
double orc_bf16(int code)
{
    int s = (code >> 15) & 1;
    int e = (code >> 7) & 255;
    int m = code & 127;
    double mag;
    if (e == 255)
        mag = m ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp(m / 128.0, -126);
    else
        mag = ldexp(1.0 + m / 128.0, e - 127);
    return s ? -mag : mag;
}

/* x rounded to the nearest bf16 value, ties to the even significand.  A bf16
 * value has 8 significant bits, so in the binade [2^(e-1), 2^e) its spacing is
 * 2^(e-8); below 2^-126 (subnormals) the spacing stays 2^-133.  A magnitude
 * that rounds to 2^128 or above is past the largest finite bf16 and becomes
 * infinity.  Zeros, infinities and NaN pass through. */
double orc_round_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    double a = fabs(x);
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int lsb = (e - 1) - 7;              /* exponent of the spacing */
    if (lsb < -133)
        lsb = -133;
    double q = ldexp(a, -lsb);          /* a in units of the spacing (exact) */
    double fl = floor(q), frac = q - fl;
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0))
        r = fl + 1.0;
    double v = ldexp(r, lsb);
    if (v >= ldexp(1.0, 128))
        v = INFINITY;
    return x < 0 ? -v : v;
}

/* Element d of a packed e2m1 vector: element 2i is the low nibble of byte i,
 * element 2i+1 the high nibble. */
static int nibble(const uint8_t *packed, int d)
{
    uint8_t b = packed[d / 2];
    return (d & 1) ? (b >> 4) : (b & 15);
}

/* ---- candidate token set ---------------------------------------------------- */

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Distinct candidate block ids >= 0, ascending.  Negative ids are padding and
 * repeated ids count once.  Returns how many were written to ids_out. */
static int distinct_blocks(const int32_t *cand, int nb, int32_t *ids_out)
{
    int n = 0;
    for (int i = 0; i < nb; i++)
        if (cand[i] >= 0)
            ids_out[n++] = cand[i];
    qsort(ids_out, n, sizeof(int32_t), cmp_i32);
    int m = 0;
    for (int i = 0; i < n; i++)
        if (m == 0 || ids_out[i] != ids_out[m - 1])
            ids_out[m++] = ids_out[i];
    return m;
}

/* T = union over distinct candidate blocks b of [b*cbs, (b+1)*cbs) cut to
 * [ks, ke), ascending.  Returns |T|. */
int32_t orc_candidate_tokens(const int32_t *cand, int nb, int cbs, int32_t ks, int32_t ke,
                             int32_t *tokens_out)
{
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (nb > 0 ? nb : 1));
    int m = distinct_blocks(cand, nb, ids);
    int32_t n = 0;
    for (int i = 0; i < m; i++) {
        int64_t lo = (int64_t)ids[i] * cbs, hi = lo + cbs;
        if (lo < ks)
            lo = ks;
        if (hi > ke)
            hi = ke;
        for (int64_t t = lo; t < hi; t++)
            tokens_out[n++] = (int32_t)t;
    }
    free(ids);
    return n;
}

/* Sparse-column schedule of one row: ascending sparse block ids that hold a
 * token of T, then -1 up to nsb_cap; *end_out = |T|.  Returns the number of
 * listed sparse blocks. */
int32_t orc_expand_row(const int32_t *cand, int nb, int cbs, int sbk, int32_t ks, int32_t ke,
                       int32_t *sparse_out, int32_t nsb_cap, int32_t *end_out)
{
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (nb > 0 ? nb : 1));
    int m = distinct_blocks(cand, nb, ids);
    int per = cbs / sbk;
    int32_t n = 0, valid = 0;
    for (int i = 0; i < m; i++) {
        for (int j = 0; j < per; j++) {
            int64_t sb = (int64_t)ids[i] * per + j;
            int64_t lo = sb * sbk, hi = lo + sbk;
            if (lo < ks)
                lo = ks;
            if (hi > ke)
                hi = ke;
            if (lo < hi) {
                if (n < nsb_cap)
                    sparse_out[n] = (int32_t)sb;
                n++;
                valid += (int32_t)(hi - lo);
            }
        }
    }
    for (int32_t i = n; i < nsb_cap; i++)
        sparse_out[i] = -1;
    *end_out = valid;
    free(ids);
    return n;
}

/* ---- logits ----------------------------------------------------------------- */

typedef struct {
    int num_heads, head_dim, page_size;
    const uint8_t *k_values;
    int64_t k_values_page_stride;
    const uint8_t *k_scales;
    int64_t k_scales_page_stride;
    const int32_t *table_row; /* the row's block-table row */
} orc_kview;

/* k[d] for token t: page = table_row[t / page_size], slot t % page_size; the
 * slot's packed values are D/2 bytes at slot*(D/2) in the page's value area,
 * its scales D/32 bytes at slot*(D/32) in the page's scale area, scale byte j
 * covering elements [32j, 32j+32). */
static void dequant_k(const orc_kview *kv, int32_t t, double *k)
{
    int D = kv->head_dim;
    int64_t page = kv->table_row[t / kv->page_size];
    int slot = t % kv->page_size;
    const uint8_t *v = kv->k_values + page * kv->k_values_page_stride + (int64_t)slot * (D / 2);
    const uint8_t *s = kv->k_scales + page * kv->k_scales_page_stride + (int64_t)slot * (D / 32);
    for (int d = 0; d < D; d++)
        k[d] = orc_e2m1(nibble(v, d)) * orc_ue8m0(s[d / 32]);
}

/* q[h][d] of one row.  MXFP4: values [H][D/2] packed, scales [H][D/32].
 * FP8: codes [H][D] (e4m3fn); the row's fp32 scale is applied to each dot
 * product (see row_logit). */
static void dequant_q(int q_format, int H, int D, const uint8_t *qv, const uint8_t *qs,
                      const uint8_t *q8, double *q)
{
    for (int h = 0; h < H; h++)
        for (int d = 0; d < D; d++) {
            if (q_format == ORC_Q_MXFP4)
                q[h * D + d] = orc_e2m1(nibble(qv + (int64_t)h * (D / 2), d)) *
                               orc_ue8m0(qs[(int64_t)h * (D / 32) + d / 32]);
            else
                q[h * D + d] = orc_e4m3fn(q8[(int64_t)h * D + d]);
        }
}

/* sum_h w[h] * relu(dot_h) in fp64, dot_h = s_r * (q_h . k) for FP8 Q. */
static double row_logit(int H, int D, const double *q, const double *k, const double *w,
                        int q_format, double rowscale)
{
    double acc = 0.0;
    for (int h = 0; h < H; h++) {
        double dot = 0.0;
        for (int d = 0; d < D; d++)
            dot += q[h * D + d] * k[d];
        if (q_format == ORC_Q_FP8)
            dot *= rowscale;
        double relu = dot > 0.0 ? dot : 0.0;   /* ReLU(NaN) = 0 */
        acc += w[h] * relu;
    }
    return acc;
}

/* The logit the selection sees: the fp64 sum rounded once, to fp32 (round to
 * nearest even) or, in the bf16 variant, to the nearest bf16.  A NaN sum (a NaN or
 * infinite weight) becomes -inf: it ranks below every number and ties with -inf
 * toward the lower token. */
static float final_logit(double acc, int score_format)
{
    if (isnan(acc))
        return -INFINITY;
    if (score_format == ORC_SCORE_BF16)
        return (float)orc_round_bf16(acc);
    return (float)acc;
}

/* Row r's query q[h][d], its weights w[h] (fp32, or bf16 codes widened exactly) and
 * its fp8 row scale (1 for MXFP4); layouts as described at orc_indexer_rows. */
static double row_query(int H, int D, int q_format, int score_format, const uint8_t *q_values,
                        const uint8_t *q_scales, const uint8_t *q_fp8, const float *q_rowscale,
                        const void *weights, int32_t r, double *q, double *w)
{
    dequant_q(q_format, H, D,
              q_values ? q_values + (int64_t)r * H * (D / 2) : NULL,
              q_scales ? q_scales + (int64_t)r * H * (D / 32) : NULL,
              q_fp8 ? q_fp8 + (int64_t)r * H * D : NULL, q);
    for (int h = 0; h < H; h++)
        w[h] = score_format == ORC_SCORE_BF16
                   ? orc_bf16(((const uint16_t *)weights)[(int64_t)r * H + h])
                   : (double)((const float *)weights)[(int64_t)r * H + h];
    return (q_format == ORC_Q_FP8) ? (double)q_rowscale[r] : 1.0;
}

/* ---- top-k selection -------------------------------------------------------- */

typedef struct {
    float logit;
    int32_t t;
} orc_pair;

/* Larger logit first; equal fp32 values (with -0 == +0) by lower token. */
static int cmp_pair(const void *a, const void *b)
{
    const orc_pair *x = (const orc_pair *)a, *y = (const orc_pair *)b;
    if (x->logit > y->logit)
        return -1;
    if (x->logit < y->logit)
        return 1;
    return (x->t > y->t) - (x->t < y->t);
}

/* out[0, count) holds the chosen ids: sort them ascending and fill out[count, width)
 * with -1. */
static void emit_ascending(int32_t *out, int32_t count, int32_t width)
{
    qsort(out, count, sizeof(int32_t), cmp_i32);
    for (int32_t i = count; i < width; i++)
        out[i] = -1;
}

/* out[0, count) = the chosen tokens ascending, out[count, topk) = -1. */
int32_t orc_select_topk(const int32_t *tokens, const float *logits, int32_t n, int32_t topk,
                        int32_t *out)
{
    orc_pair *p = (orc_pair *)malloc(sizeof(orc_pair) * (n > 0 ? n : 1));
    for (int32_t i = 0; i < n; i++) {
        p[i].logit = logits[i];
        p[i].t = tokens[i];
    }
    qsort(p, n, sizeof(orc_pair), cmp_pair);
    int32_t count = n < topk ? n : topk;
    for (int32_t i = 0; i < count; i++)
        out[i] = p[i].t;
    emit_ascending(out, count, topk);
    free(p);
    return count;
}

/* ---- the candidate-source layer ---------------------------------------------- */

typedef struct {
    float score;
    int32_t b;
} orc_block;

/* Larger block score first; equal fp32 scores by lower block id. */
static int cmp_block(const void *a, const void *b)
{
    const orc_block *x = (const orc_block *)a, *y = (const orc_block *)b;
    if (x->score > y->score)
        return -1;
    if (x->score < y->score)
        return 1;
    return (x->b > y->b) - (x->b < y->b);
}

/*
 * For each row r = rows[i] (i < n_sel), with ks, ke and the table row as in
 * orc_indexer_rows below:
 *   logit[t] for every t in [ks, ke)  (the same per-token definition)
 *   score[b] = max of logit[t] over the tokens t of block b (b*cbs <= t <
 *              (b+1)*cbs) that lie in [ks, ke); block b is eligible when it
 *              holds at least one such token
 *   out_cand[i*cand_stride + 0 .. nb): the min(nb, #eligible) eligible blocks
 *              with the largest scores (ties toward the lower block id), in
 *              ascending block order, then -1
 *   out_score[i*score_stride + b] (optional): score[b] for b < score_stride,
 *              NaN where block b is not eligible
 * Returns 0.
 */
int orc_source_candidates(int num_heads, int head_dim, int page_size, int cbs, int nb,
                          int q_format, int score_format, const uint8_t *q_values,
                          const uint8_t *q_scales, const uint8_t *q_fp8,
                          const float *q_rowscale, const void *weights,
                          const uint8_t *k_values, int64_t k_values_page_stride,
                          const uint8_t *k_scales, int64_t k_scales_page_stride,
                          const int32_t *block_table, int64_t block_table_stride,
                          const int32_t *row_ks, const int32_t *row_ke,
                          const int32_t *row_table, const int32_t *rows, int32_t n_sel,
                          int32_t *out_cand, int64_t cand_stride, float *out_score,
                          int64_t score_stride)
{
    int H = num_heads, D = head_dim;
    double *q = (double *)malloc(sizeof(double) * H * D);
    double *k = (double *)malloc(sizeof(double) * D);
    double *w = (double *)malloc(sizeof(double) * H);
    for (int32_t i = 0; i < n_sel; i++) {
        int32_t r = rows[i];
        int32_t ks = row_ks ? row_ks[r] : 0, ke = row_ke[r];
        int32_t tbl = row_table ? row_table[r] : r;
        int32_t nblk = ke > 0 ? (ke + cbs - 1) / cbs : 0;
        double rs = row_query(H, D, q_format, score_format, q_values, q_scales, q_fp8,
                              q_rowscale, weights, r, q, w);
        orc_kview kv = {H, D, page_size, k_values, k_values_page_stride,
                        k_scales, k_scales_page_stride,
                        block_table + (int64_t)tbl * block_table_stride};
        orc_block *blk = (orc_block *)malloc(sizeof(orc_block) * (nblk > 0 ? nblk : 1));
        int32_t n_el = 0;
        for (int32_t b = 0; b < nblk; b++) {
            int64_t lo = (int64_t)b * cbs, hi = lo + cbs;
            if (lo < ks)
                lo = ks;
            if (hi > ke)
                hi = ke;
            float best = 0.0f;
            int any = 0;
            for (int64_t t = lo; t < hi; t++) {
                dequant_k(&kv, (int32_t)t, k);
                float lg = final_logit(row_logit(H, D, q, k, w, q_format, rs), score_format);
                if (!any || lg > best)
                    best = lg;
                any = 1;
            }
            if (out_score && b < score_stride)
                out_score[(int64_t)i * score_stride + b] = any ? best : NAN;
            if (any) {
                blk[n_el].score = best;
                blk[n_el].b = b;
                n_el++;
            }
        }
        if (out_score)
            for (int64_t b = nblk; b < score_stride; b++)
                out_score[(int64_t)i * score_stride + b] = NAN;
        qsort(blk, n_el, sizeof(orc_block), cmp_block);
        int32_t count = n_el < nb ? n_el : nb;
        int32_t *out = out_cand + (int64_t)i * cand_stride;
        for (int32_t j = 0; j < count; j++)
            out[j] = blk[j].b;
        emit_ascending(out, count, nb);
        free(blk);
    }
    free(q);
    free(k);
    free(w);
    return 0;
}

/* ---- one call over a list of rows ------------------------------------------- */

/*
 * For each row r = rows[i] (i < n_sel):
 *   ks = row_ks ? row_ks[r] : 0;  ke = row_ke[r];
 *   tbl = row_table ? row_table[r] : r;
 *   T = candidate tokens;  logits for every t in T;  top-k.
 * Outputs for selected row i:
 *   out_indices[i*out_stride + 0 .. topk)    chosen tokens then -1
 *   out_tokens / out_logits[i*tok_stride ..] T and its logits (optional, may be NULL)
 *   out_exact[i*tok_stride ..]               the fp64 sums before the final rounding
 *                                            (optional, may be NULL)
 *   out_count[i] = |T|                        (optional)
 * q_values/q_scales are [R][H][D/2] / [R][H][D/32]; q_fp8 is [R][H][D];
 * q_rowscale [R]; weights [R][H], fp32 (score_format ORC_SCORE_FP32) or bf16
 * codes (ORC_SCORE_BF16); candidate_blocks [R][cand_stride].
 * Returns 0.
 */
int orc_indexer_rows(int num_heads, int head_dim, int page_size, int cbs, int nb, int topk,
                     int q_format, int score_format, const uint8_t *q_values,
                     const uint8_t *q_scales, const uint8_t *q_fp8, const float *q_rowscale,
                     const void *weights,
                     const uint8_t *k_values, int64_t k_values_page_stride,
                     const uint8_t *k_scales, int64_t k_scales_page_stride,
                     const int32_t *block_table, int64_t block_table_stride,
                     const int32_t *row_ks, const int32_t *row_ke, const int32_t *row_table,
                     const int32_t *candidate_blocks, int64_t cand_stride, const int32_t *rows,
                     int32_t n_sel, int32_t *out_indices, int64_t out_stride,
                     int32_t *out_tokens, float *out_logits, double *out_exact,
                     int64_t tok_stride, int32_t *out_count)
{
    int H = num_heads, D = head_dim;
    double *q = (double *)malloc(sizeof(double) * H * D);
    double *k = (double *)malloc(sizeof(double) * D);
    double *w = (double *)malloc(sizeof(double) * H);
    int64_t cap = (int64_t)nb * cbs;
    int32_t *tokens = (int32_t *)malloc(sizeof(int32_t) * (cap > 0 ? cap : 1));
    float *logits = (float *)malloc(sizeof(float) * (cap > 0 ? cap : 1));
    double *exact = (double *)malloc(sizeof(double) * (cap > 0 ? cap : 1));
    for (int32_t i = 0; i < n_sel; i++) {
        int32_t r = rows[i];
        int32_t ks = row_ks ? row_ks[r] : 0, ke = row_ke[r];
        int32_t tbl = row_table ? row_table[r] : r;
        int32_t n = orc_candidate_tokens(candidate_blocks + (int64_t)r * cand_stride, nb, cbs,
                                         ks, ke, tokens);
        double rs = row_query(H, D, q_format, score_format, q_values, q_scales, q_fp8,
                              q_rowscale, weights, r, q, w);
        orc_kview kv = {H, D, page_size, k_values, k_values_page_stride,
                        k_scales, k_scales_page_stride,
                        block_table + (int64_t)tbl * block_table_stride};
        for (int32_t j = 0; j < n; j++) {
            dequant_k(&kv, tokens[j], k);
            exact[j] = row_logit(H, D, q, k, w, q_format, rs);
            logits[j] = final_logit(exact[j], score_format);
        }
        orc_select_topk(tokens, logits, n, topk, out_indices + (int64_t)i * out_stride);
        if (out_tokens)
            memcpy(out_tokens + (int64_t)i * tok_stride, tokens, sizeof(int32_t) * n);
        if (out_logits)
            memcpy(out_logits + (int64_t)i * tok_stride, logits, sizeof(float) * n);
        if (out_exact)
            memcpy(out_exact + (int64_t)i * tok_stride, exact, sizeof(double) * n);
        if (out_count)
            out_count[i] = n;
    }
    free(q);
    free(k);
    free(w);
    free(tokens);
    free(logits);
    free(exact);
    return 0;
}

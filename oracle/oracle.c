/*
 * oracle.c -- plain, slow CPU reference for tree-masked decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no header, helper or constant with the
 * HIP library; every quantity is recomputed here from the pages' definitions.
 *
 * Sources (cited by page title and section):
 *   [TA]  "tree_attention.metal" (mlx-native 0.9.1): header comment,
 *         TreeAttentionParams, tree_attention_impl.
 *   [OPS] "ops/tree_attention.rs" (mlx-native 0.9.2): module doc, mask
 *         constants, tree_attention() buffer doc, tmp_buffer_bytes.
 *   [FQS] "ffai/flash_quantized_sdpa.rs" (metaltile-std 0.1.0): module doc
 *         (Layout, Mask variants), base and float-mask kernel macros.
 *
 * All arithmetic is IEEE double, with plain loops, and the attention is a
 * direct two-pass softmax: pass 1 takes the maximum logit, pass 2 sums
 * exp(logit - max) and the weighted values.  No blocking, no online update.
 * The one exception is orc_attention_partials / orc_lse_combine, which
 * restate the split-KV scheme of [TA] header (each of several workgroups
 * covers part of the keys; a second pass merges their partial results)
 * so that the merge rule can be checked on its own.
 *
 * Readings of the pages taken here (each is listed in the design notes):
 *   R1  A mask cell <= -65504 excludes the key; any larger value is added
 *       to the scaled logit.  ([OPS] mask constants; [TA] mask read and
 *       the "every cell masked" early exit.)
 *   R2  A row with no included key produces zeros.  ([TA] write-results
 *       block uses 0 when S == 0; [FQS] base macro keeps o when l == 0.)
 *   R5  Tree node i sits at KV position kv_seq_len - q_l + i; the prefix
 *       [0, kv_seq_len - q_l) is visible to every node.  ([TA] header:
 *       abs_pos = kv_seq_len - qL + iq1.)
 *   R8  With no mask buffer the implicit causal rule applies: row i sees
 *       key j iff j <= kv_seq_len - q_l + i.  ([TA] header, flash_attn_vec
 *       implicit mask.)
 *   R8W The implicit rule with a sliding-window start: row i sees key j iff
 *       window_start <= j <= kv_seq_len - q_l + i, one window_start for
 *       every row, as the [TA] header states the byte-identity contract
 *       (0.0f for k_pos in [window_start, abs_pos]).  window_start = 0 is R8.
 *   R12 A sink is one extra virtual key per query head with raw logit
 *       sinks[h] (no scale, no mask) and a zero value.  ([FQS] base macro,
 *       accumulator initialisation.)
 *   R13 Packed codes are little-end first: element d lives in bits
 *       [(d % pf)*bits, +bits) of word d / pf, pf = 32 / bits.  ([FQS]
 *       Layout and base macro dequant.)
 *   R-Q Quantized-path mask cells obey R1 as well; when no mask is given
 *       the quantized path applies R8 (for q_l == 1 this attends every
 *       token, as [FQS] does with window_size 0).
 *   R-B A bool mask holds one u32 per (query row, token): 0 drops the key,
 *       any other value keeps it with no bias.  With a mask (float or bool)
 *       the mask alone decides, as in [FQS] Mask variants and the
 *       bool-mask macro.
 *   R-W A window size W > 0 keeps token t only if t + W > kv_seq_len - 1,
 *       i.e. the last W tokens, for every query row and every mask kind
 *       ([FQS] base, bool- and float-mask macros: the causal / sliding
 *       window gate with causal_upper = tokens - 1).  W = 0 keeps all.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* [OPS] mask constants: masked = -MAXHALF, attended = 0. */
#define ORC_MASKED (-65504.0)

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16 -> double, exactly, from the bit fields.               */
/* ------------------------------------------------------------------------ */
double orc_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);             /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 -> double, exactly, from its bit fields: 1 sign bit, 8 exponent
 * bits (bias 127), 7 mantissa bits, the upper half of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);            /* subnormal: m/128 * 2^-126 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Tree topology -> explicit mask.                                          */
/* [TA] header: chains, fixed trees and dynamic trees all become a          */
/* [q_l, kv_seq_len] float mask, 0 = attended, -65504 = masked.  Row i      */
/* (reading R5) sees the prefix, its ancestors and itself.  Cells in        */
/* [kv_seq_len, mask_stride) are never read by attention; they are set to   */
/* the masked value.                                                        */
/* parents[0] must be -1 and 0 <= parents[i] < i for i >= 1.               */
/* Returns 0, or -1 on an invalid argument (nothing written).               */
/* ------------------------------------------------------------------------ */
int orc_tree_mask(const int32_t *parents, uint32_t q_l, uint32_t kv_seq_len,
                  uint32_t mask_stride, float *mask)
{
    if (q_l == 0 || q_l > kv_seq_len || mask_stride < kv_seq_len)
        return -1;
    if (parents[0] != -1)
        return -1;
    for (uint32_t i = 1; i < q_l; ++i)
        if (parents[i] < 0 || (uint32_t)parents[i] >= i)
            return -1;

    uint32_t base = kv_seq_len - q_l;
    for (uint32_t i = 0; i < q_l; ++i) {
        float *row = mask + (size_t)i * mask_stride;
        for (uint32_t j = 0; j < mask_stride; ++j)
            row[j] = (float)ORC_MASKED;
        for (uint32_t j = 0; j < base; ++j)
            row[j] = 0.0f;
        /* walk from the node up to the root */
        int32_t a = (int32_t)i;
        while (a >= 0) {
            row[base + (uint32_t)a] = 0.0f;
            a = parents[a];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* fp path problem description ([OPS] TreeAttentionParams + buffer doc).    */
/* q    [n_heads, q_l, head_dim] f32                                         */
/* k, v [n_kv_heads, kv_capacity, head_dim], f32 or f16 (raw bits)           */
/* mask [q_l, mask_stride] f32, or NULL for the implicit causal rule         */
/* out  [q_l, n_heads, head_dim] (query-outer, head-inner), here in double   */
/* ------------------------------------------------------------------------ */
typedef struct {
    const float *q;
    const void *k;
    const void *v;
    int kv_f16;
    const float *mask;
    uint32_t n_heads, n_kv_heads, head_dim, kv_seq_len, kv_capacity, q_l,
        mask_stride;
    double scale;
    uint32_t window_start; /* R8W; implicit rule only */
} orc_fp_problem;

static double kv_elem(const void *base, int is_f16, size_t idx)
{
    if (is_f16)
        return orc_f16_to_f64(((const uint16_t *)base)[idx]);
    return (double)((const float *)base)[idx];
}

/* Mask cell for (query row i, key j) per R1/R8. */
static double fp_mask_cell(const orc_fp_problem *p, uint32_t i, uint32_t j)
{
    if (p->mask)
        return (double)p->mask[(size_t)i * p->mask_stride + j];
    int64_t last = (int64_t)p->kv_seq_len - (int64_t)p->q_l + (int64_t)i;
    return (j >= p->window_start && (int64_t)j <= last) ? 0.0 : ORC_MASKED;
}

/* Logit of key j for (node i, head h); returns 0 if the key is excluded. */
static int fp_logit(const orc_fp_problem *p, uint32_t i, uint32_t h,
                    uint32_t j, double *logit)
{
    double m = fp_mask_cell(p, i, j);
    if (m <= ORC_MASKED)
        return 0;
    uint32_t D = p->head_dim;
    uint32_t hk = h / (p->n_heads / p->n_kv_heads); /* GQA ([TA] impl) */
    const float *qrow = p->q + ((size_t)h * p->q_l + i) * D;
    size_t krow = ((size_t)hk * p->kv_capacity + j) * D;
    double dot = 0.0;
    for (uint32_t d = 0; d < D; ++d)
        dot += (double)qrow[d] * kv_elem(p->k, p->kv_f16, krow + d);
    *logit = p->scale * dot + m;
    return 1;
}

/* Direct two-pass softmax attention for one (node i, head h) over keys
 * [j0, j1).  Writes the UNNORMALISED output o[D], the sum s and the max mx
 * (mx = -inf and s = 0 when no key is included). */
static void fp_row_unnormalised(const orc_fp_problem *p, uint32_t i,
                                uint32_t h, uint32_t j0, uint32_t j1,
                                double *o, double *s, double *mx)
{
    uint32_t D = p->head_dim;
    uint32_t hk = h / (p->n_heads / p->n_kv_heads);
    double best = -INFINITY;
    double l;
    /* pass 1: maximum included logit */
    for (uint32_t j = j0; j < j1; ++j)
        if (fp_logit(p, i, h, j, &l) && l > best)
            best = l;
    for (uint32_t d = 0; d < D; ++d)
        o[d] = 0.0;
    *s = 0.0;
    *mx = best;
    if (best == -INFINITY)
        return;
    /* pass 2: weights exp(l - max), their sum and the weighted values */
    for (uint32_t j = j0; j < j1; ++j) {
        if (!fp_logit(p, i, h, j, &l))
            continue;
        double w = exp(l - best);
        *s += w;
        size_t vrow = ((size_t)hk * p->kv_capacity + j) * D;
        for (uint32_t d = 0; d < D; ++d)
            o[d] += w * kv_elem(p->v, p->kv_f16, vrow + d);
    }
}

/* ---- simple thread pool over independent output rows -------------------- */
typedef struct {
    void (*fn)(void *ctx, uint32_t row);
    void *ctx;
    uint32_t nrows;
    uint32_t tid, nthreads;
} orc_job;

static void *orc_worker(void *arg)
{
    orc_job *j = (orc_job *)arg;
    for (uint32_t r = j->tid; r < j->nrows; r += j->nthreads)
        j->fn(j->ctx, r);
    return NULL;
}

static void orc_parallel(void (*fn)(void *, uint32_t), void *ctx,
                         uint32_t nrows, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if ((uint32_t)nthreads > nrows)
        nthreads = nrows ? (int)nrows : 1;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    orc_job *jobs = (orc_job *)calloc((size_t)nthreads, sizeof(orc_job));
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].nrows = nrows;
        jobs[t].tid = (uint32_t)t;
        jobs[t].nthreads = (uint32_t)nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, orc_worker, &jobs[t]);
    orc_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

static int fp_problem_ok(const orc_fp_problem *p)
{
    if (p->n_heads == 0 || p->n_kv_heads == 0 || p->head_dim == 0)
        return 0;
    if (p->n_heads % p->n_kv_heads)
        return 0;
    if (p->kv_seq_len == 0 || p->kv_capacity < p->kv_seq_len || p->q_l == 0)
        return 0;
    if (p->mask && p->mask_stride < p->kv_seq_len)
        return 0;
    return 1;
}

/* ---- whole attention ----------------------------------------------------- */
typedef struct {
    const orc_fp_problem *p;
    const uint32_t *sel; /* (i, h) pairs, or NULL = every row */
    double *out;
} fp_full_ctx;

static void fp_full_row(void *vctx, uint32_t r)
{
    fp_full_ctx *c = (fp_full_ctx *)vctx;
    const orc_fp_problem *p = c->p;
    uint32_t i, h;
    if (c->sel) {
        i = c->sel[2 * r];
        h = c->sel[2 * r + 1];
    } else {
        i = r / p->n_heads; /* out row r = i * n_heads + h ([OPS] doc) */
        h = r % p->n_heads;
    }
    uint32_t D = p->head_dim;
    double *o = c->out + (size_t)r * D;
    double s, mx;
    fp_row_unnormalised(p, i, h, 0, p->kv_seq_len, o, &s, &mx);
    for (uint32_t d = 0; d < D; ++d)
        o[d] = (s > 0.0) ? o[d] / s : 0.0; /* R2 */
}

/*
 * orc_attention: out[r * head_dim + d] for r over the selected rows.
 * sel == NULL: every row, r = i * n_heads + h, i.e. the [q_l, n_heads, D]
 * layout of [OPS].  Otherwise sel holds nsel (i, h) pairs.
 * Returns 0, or -1 on an invalid problem.
 */
int orc_attention_ex(const float *q, const void *k, const void *v, int kv_f16,
                     const float *mask, uint32_t n_heads, uint32_t n_kv_heads,
                     uint32_t head_dim, uint32_t kv_seq_len, uint32_t kv_capacity,
                     uint32_t q_l, uint32_t mask_stride, double scale,
                     uint32_t window_start, const uint32_t *sel, uint32_t nsel,
                     double *out, int nthreads)
{
    orc_fp_problem p = {q,          k,          v,        kv_f16,
                        mask,       n_heads,    n_kv_heads, head_dim,
                        kv_seq_len, kv_capacity, q_l,      mask_stride,
                        scale,      window_start};
    if (!fp_problem_ok(&p))
        return -1;
    if (mask && window_start)
        return -1; /* a mask buffer encodes all visibility ([TA] header) */
    if (sel)
        for (uint32_t r = 0; r < nsel; ++r)
            if (sel[2 * r] >= q_l || sel[2 * r + 1] >= n_heads)
                return -1;
    fp_full_ctx c = {&p, sel, out};
    uint32_t nrows = sel ? nsel : n_heads * q_l;
    orc_parallel(fp_full_row, &c, nrows, nthreads);
    return 0;
}

/* orc_attention: orc_attention_ex with window_start = 0. */
int orc_attention(const float *q, const void *k, const void *v, int kv_f16,
                  const float *mask, uint32_t n_heads, uint32_t n_kv_heads,
                  uint32_t head_dim, uint32_t kv_seq_len, uint32_t kv_capacity,
                  uint32_t q_l, uint32_t mask_stride, double scale,
                  const uint32_t *sel, uint32_t nsel, double *out,
                  int nthreads)
{
    return orc_attention_ex(q, k, v, kv_f16, mask, n_heads, n_kv_heads, head_dim,
                            kv_seq_len, kv_capacity, q_l, mask_stride, scale, 0u,
                            sel, nsel, out, nthreads);
}

/* ---- split-KV partials and their log-sum-exp combine --------------------- */
typedef struct {
    const orc_fp_problem *p;
    const uint32_t *bounds;
    uint32_t nparts;
    double *o_un, *s, *m;
} fp_part_ctx;

static void fp_part_row(void *vctx, uint32_t r)
{
    fp_part_ctx *c = (fp_part_ctx *)vctx;
    const orc_fp_problem *p = c->p;
    uint32_t i = r / p->n_heads, h = r % p->n_heads;
    uint32_t D = p->head_dim;
    for (uint32_t w = 0; w < c->nparts; ++w) {
        size_t pr = (size_t)r * c->nparts + w;
        fp_row_unnormalised(p, i, h, c->bounds[w], c->bounds[w + 1],
                            c->o_un + pr * D, &c->s[pr], &c->m[pr]);
    }
}

/*
 * orc_attention_partials: for every row r = i * n_heads + h and every part
 * w of the key partition bounds[0] = 0 <= ... <= bounds[nparts] = kv_seq_len,
 * the unnormalised output o_un[(r*nparts + w)*D + d], the sum s[r*nparts+w]
 * and the max m[r*nparts+w] (natural-log units; -inf when the part has no
 * included key).  These are the per-workgroup results of [TA]'s split-KV
 * (O unnormalised, S, M) expressed in exact arithmetic.
 */
int orc_attention_partials(const float *q, const void *k, const void *v,
                           int kv_f16, const float *mask, uint32_t n_heads,
                           uint32_t n_kv_heads, uint32_t head_dim,
                           uint32_t kv_seq_len, uint32_t kv_capacity,
                           uint32_t q_l, uint32_t mask_stride, double scale,
                           const uint32_t *bounds, uint32_t nparts,
                           double *o_un, double *s, double *m, int nthreads)
{
    orc_fp_problem p = {q,          k,          v,        kv_f16,
                        mask,       n_heads,    n_kv_heads, head_dim,
                        kv_seq_len, kv_capacity, q_l,      mask_stride,
                        scale};
    if (!fp_problem_ok(&p) || nparts == 0)
        return -1;
    if (bounds[0] != 0 || bounds[nparts] != kv_seq_len)
        return -1;
    for (uint32_t w = 0; w < nparts; ++w)
        if (bounds[w] > bounds[w + 1])
            return -1;
    fp_part_ctx c = {&p, bounds, nparts, o_un, s, m};
    orc_parallel(fp_part_row, &c, n_heads * q_l, nthreads);
    return 0;
}

/*
 * orc_lse_combine: the reduce pass.  For each row, with parts w:
 *   M* = max_w M_w,  S* = sum_w S_w e^(M_w - M*),
 *   O  = sum_w O_w e^(M_w - M*) / S*,   O = 0 when S* = 0 (R2).
 * Parts with S_w = 0 contribute nothing.  Layout as orc_attention_partials.
 */
int orc_lse_combine(const double *o_un, const double *s, const double *m,
                    uint32_t nrows, uint32_t head_dim, uint32_t nparts,
                    double *out)
{
    for (uint32_t r = 0; r < nrows; ++r) {
        double mstar = -INFINITY;
        for (uint32_t w = 0; w < nparts; ++w) {
            size_t pr = (size_t)r * nparts + w;
            if (s[pr] > 0.0 && m[pr] > mstar)
                mstar = m[pr];
        }
        double *o = out + (size_t)r * head_dim;
        for (uint32_t d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        if (mstar == -INFINITY)
            continue;
        double sstar = 0.0;
        for (uint32_t w = 0; w < nparts; ++w) {
            size_t pr = (size_t)r * nparts + w;
            if (!(s[pr] > 0.0))
                continue;
            double f = exp(m[pr] - mstar);
            sstar += s[pr] * f;
            for (uint32_t d = 0; d < head_dim; ++d)
                o[d] += o_un[pr * head_dim + d] * f;
        }
        for (uint32_t d = 0; d < head_dim; ++d)
            o[d] /= sstar;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Affine-quantized K/V attention ([FQS]).                                  */
/* The element type T ([FQS] kernels are generic in T) of q, the scales,   */
/* the biases and the float mask: elem 0 = f16, 1 = bf16, 2 = f32.          */
/* q        [B*nQ, q_l, dim] T                                               */
/* k_packed [B*nKV, kv_capacity, dim/pf] u32, pf = 32/bits                   */
/* k_scales, k_biases [B*nKV, kv_capacity, dim/G] T; V the same              */
/* sinks    [nQ] f32 or NULL                                                 */
/* mask     T, cell (q_idx, i, t) at                                         */
/*          q_idx*mask_head_stride + i*mask_stride + t, or NULL (R-Q)        */
/* out      [B*nQ, q_l, dim] in double                                       */
/* ------------------------------------------------------------------------ */
typedef struct {
    const void *q;
    const uint32_t *kp;
    const void *ks, *kb;
    const uint32_t *vp;
    const void *vs, *vb;
    const float *sinks;
    const void *mask;
    int elem;                  /* 0 f16, 1 bf16, 2 f32 */
    const uint32_t *mask_bool; /* R-B; at most one of mask, mask_bool */
    uint32_t window;           /* R-W */
    uint64_t mask_head_stride;
    uint32_t mask_stride;
    uint32_t batch, nq, nkv, dim, kv_seq_len, kv_capacity, q_l, bits, group;
    double scale;
    const uint32_t *sel; /* (q_idx, i) pairs or NULL */
    double *out;
} orc_q_problem;

/* Element idx of a T array, exactly. */
static double q_elem(const orc_q_problem *p, const void *base, size_t idx)
{
    if (p->elem == 1)
        return orc_bf16_to_f64(((const uint16_t *)base)[idx]);
    if (p->elem == 2)
        return (double)((const float *)base)[idx];
    return orc_f16_to_f64(((const uint16_t *)base)[idx]);
}

/* Dequantised element d of token t of kv stream kv ([FQS] base macro):
 * x = scale_g * code + bias_g with code = (word >> shift) & (2^bits - 1). */
static double q_dequant(const uint32_t *packed, const void *scales,
                        const void *biases, const orc_q_problem *p,
                        uint32_t kv, uint32_t t, uint32_t d)
{
    uint32_t pf = 32u / p->bits;
    uint32_t words = p->dim / pf;
    uint32_t ngroups = p->dim / p->group;
    size_t tok = (size_t)kv * p->kv_capacity + t;
    uint32_t word = packed[tok * words + d / pf];
    uint32_t code = (word >> ((d % pf) * p->bits)) & ((1u << p->bits) - 1u);
    double sc = q_elem(p, scales, tok * ngroups + d / p->group);
    double bi = q_elem(p, biases, tok * ngroups + d / p->group);
    return sc * (double)code + bi;
}

static double q_mask_cell(const orc_q_problem *p, uint32_t q_idx, uint32_t i,
                          uint32_t t)
{
    size_t cell = (size_t)q_idx * p->mask_head_stride + (size_t)i * p->mask_stride + t;
    if (p->mask)
        return q_elem(p, p->mask, cell);
    if (p->mask_bool)
        return p->mask_bool[cell] != 0u ? 0.0 : ORC_MASKED; /* R-B */
    int64_t last = (int64_t)p->kv_seq_len - (int64_t)p->q_l + (int64_t)i;
    return ((int64_t)t <= last) ? 0.0 : ORC_MASKED;
}

static int q_logit(const orc_q_problem *p, uint32_t q_idx, uint32_t i,
                   uint32_t t, double *logit)
{
    /* R-W: the window gate comes before the mask */
    if (p->window > 0u && (uint64_t)t + p->window <= (uint64_t)p->kv_seq_len - 1u)
        return 0;
    double m = q_mask_cell(p, q_idx, i, t);
    if (m <= ORC_MASKED)
        return 0;
    uint32_t kv = q_idx / (p->nq / p->nkv); /* [FQS]: q_idx / repeat_count */
    size_t qrow = ((size_t)q_idx * p->q_l + i) * p->dim;
    double dot = 0.0;
    for (uint32_t d = 0; d < p->dim; ++d)
        dot += q_elem(p, p->q, qrow + d) *
               q_dequant(p->kp, p->ks, p->kb, p, kv, t, d);
    *logit = p->scale * dot + m;
    return 1;
}

static void q_row(void *vctx, uint32_t r)
{
    orc_q_problem *p = (orc_q_problem *)vctx;
    uint32_t q_idx, i;
    if (p->sel) {
        q_idx = p->sel[2 * r];
        i = p->sel[2 * r + 1];
    } else {
        q_idx = r / p->q_l;
        i = r % p->q_l;
    }
    uint32_t kv = q_idx / (p->nq / p->nkv);
    double *o = p->out + (size_t)r * p->dim;
    double l;
    /* pass 1: max over included keys and the sink */
    double best = -INFINITY;
    for (uint32_t t = 0; t < p->kv_seq_len; ++t)
        if (q_logit(p, q_idx, i, t, &l) && l > best)
            best = l;
    double sink = 0.0;
    if (p->sinks) {
        sink = (double)p->sinks[q_idx % p->nq]; /* R12 */
        if (sink > best)
            best = sink;
    }
    for (uint32_t d = 0; d < p->dim; ++d)
        o[d] = 0.0;
    if (best == -INFINITY)
        return; /* R2 */
    /* pass 2 */
    double s = p->sinks ? exp(sink - best) : 0.0; /* sink value is zero */
    for (uint32_t t = 0; t < p->kv_seq_len; ++t) {
        if (!q_logit(p, q_idx, i, t, &l))
            continue;
        double w = exp(l - best);
        s += w;
        for (uint32_t d = 0; d < p->dim; ++d)
            o[d] += w * q_dequant(p->vp, p->vs, p->vb, p, kv, t, d);
    }
    for (uint32_t d = 0; d < p->dim; ++d)
        o[d] = (s > 0.0) ? o[d] / s : 0.0;
}

/*
 * orc_quant_attention_ex: out[r * dim + d]; sel == NULL means every row with
 * r = q_idx * q_l + i; otherwise sel holds nsel (q_idx, i) pairs.  mask
 * (f16 bits) and mask_bool (u32) share the cell layout; at most one may be
 * given.  window: R-W.  Returns 0, or -1 on an invalid problem.
 */
int orc_quant_attention_ex(int elem, const void *q, const uint32_t *k_packed,
                           const void *k_scales, const void *k_biases,
                           const uint32_t *v_packed, const void *v_scales,
                           const void *v_biases, const float *sinks,
                           const void *mask, const uint32_t *mask_bool,
                           uint64_t mask_head_stride, uint32_t mask_stride,
                           uint32_t window, uint32_t batch, uint32_t n_q_heads,
                           uint32_t n_kv_heads, uint32_t dim, uint32_t kv_seq_len,
                           uint32_t kv_capacity, uint32_t q_l, uint32_t bits,
                           uint32_t group_size, double scale, const uint32_t *sel,
                           uint32_t nsel, double *out, int nthreads)
{
    if (batch == 0 || n_q_heads == 0 || n_kv_heads == 0 ||
        n_q_heads % n_kv_heads || dim == 0 || kv_seq_len == 0 ||
        kv_capacity < kv_seq_len || q_l == 0)
        return -1;
    if (bits != 4 && bits != 8)
        return -1;
    if (group_size == 0 || dim % group_size || dim % (32u / bits))
        return -1;
    if (mask && mask_bool)
        return -1;
    if (elem < 0 || elem > 2)
        return -1;
    if ((mask || mask_bool) && mask_stride < kv_seq_len)
        return -1;
    if (sel)
        for (uint32_t r = 0; r < nsel; ++r)
            if (sel[2 * r] >= batch * n_q_heads || sel[2 * r + 1] >= q_l)
                return -1;
    orc_q_problem p;
    memset(&p, 0, sizeof p);
    p.q = q;
    p.kp = k_packed;
    p.ks = k_scales;
    p.kb = k_biases;
    p.vp = v_packed;
    p.vs = v_scales;
    p.vb = v_biases;
    p.sinks = sinks;
    p.mask = mask;
    p.elem = elem;
    p.mask_bool = mask_bool;
    p.window = window;
    p.mask_head_stride = mask_head_stride;
    p.mask_stride = mask_stride;
    p.batch = batch;
    p.nq = n_q_heads;
    p.nkv = n_kv_heads;
    p.dim = dim;
    p.kv_seq_len = kv_seq_len;
    p.kv_capacity = kv_capacity;
    p.q_l = q_l;
    p.bits = bits;
    p.group = group_size;
    p.scale = scale;
    p.sel = sel;
    p.out = out;
    uint32_t nrows = sel ? nsel : batch * n_q_heads * q_l;
    orc_parallel(q_row, &p, nrows, nthreads);
    return 0;
}

/* orc_quant_attention: the float-mask (or no-mask) form, no window. */
int orc_quant_attention(const uint16_t *q, const uint32_t *k_packed,
                        const uint16_t *k_scales, const uint16_t *k_biases,
                        const uint32_t *v_packed, const uint16_t *v_scales,
                        const uint16_t *v_biases, const float *sinks,
                        const uint16_t *mask, uint64_t mask_head_stride,
                        uint32_t mask_stride, uint32_t batch, uint32_t n_q_heads,
                        uint32_t n_kv_heads, uint32_t dim, uint32_t kv_seq_len,
                        uint32_t kv_capacity, uint32_t q_l, uint32_t bits,
                        uint32_t group_size, double scale, const uint32_t *sel,
                        uint32_t nsel, double *out, int nthreads)
{
    return orc_quant_attention_ex(0, q, k_packed, k_scales, k_biases, v_packed,
                                  v_scales, v_biases, sinks, mask, NULL,
                                  mask_head_stride, mask_stride, 0u, batch,
                                  n_q_heads, n_kv_heads, dim, kv_seq_len,
                                  kv_capacity, q_l, bits, group_size, scale, sel,
                                  nsel, out, nthreads);
}

/*
 * csa_oracle.c -- plain fp64 CPU oracle for selective decode attention.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
 * benchmark).  Written for readability, not speed: every quantity is formed in
 * fp64 exactly as the method states it, with no blocking, fusion or reordering.
 * OpenMP only distributes independent (batch, KV head) pairs over host cores.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared csa_oracle.c -lm
 * (-ffp-contract=off keeps every product and sum separately rounded in fp64.)
 *
 * See csa_oracle.h for the layout conventions and the sources.
 */
#include "csa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

/* ----------------------------------------------------------------------------
 * Element access and storage rounding
 * ------------------------------------------------------------------------- */

/* Decode element i of a stored array to fp64.  A bfloat16 pattern is the upper
 * half of an IEEE binary32 with the lower 16 bits zero, so widening is exact. */
static double elem(const void* base, int dtype, size_t i)
{
    if (dtype == OR_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* fp64 -> bfloat16 with one round-to-nearest-even step.  bfloat16 keeps 8
 * significant bits; below 2^-126 its spacing is fixed at 2^-133.  The value is
 * scaled so that its last kept bit is the units place, rounded by rint()
 * (ties-to-even under the default rounding mode) and scaled back. */
uint16_t oracle_round_bf16(double x)
{
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0) return sign;
    if (isinf(ax)) return sign | 0x7f80;
    int e;
    frexp(ax, &e); /* ax = f * 2^e with 0.5 <= f < 1 */
    int ulp_exp = e - 8;
    if (ulp_exp < -133) ulp_exp = -133;
    double r = ldexp(rint(ldexp(ax, -ulp_exp)), ulp_exp);
    if (r >= 0x1p128) return sign | 0x7f80; /* rounds past the largest finite value */
    float f = (float)r;                      /* exact: at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return sign | (uint16_t)(bits >> 16);
}

/* Store an fp64 value into element i of an array of the storage dtype. */
static void store(void* base, int dtype, size_t i, double x)
{
    if (dtype == OR_F32)
        ((float*)base)[i] = (float)x; /* C conversion rounds to nearest even */
    else
        ((uint16_t*)base)[i] = oracle_round_bf16(x);
}

int oracle_store_array(int dtype, size_t n, const double* x, void* out)
{
    if ((dtype != OR_F32 && dtype != OR_BF16) || (n && (!x || !out))) return -1;
    for (size_t i = 0; i < n; ++i) store(out, dtype, i, x[i]);
    return 0;
}

/* ----------------------------------------------------------------------------
 * Shape helpers
 * ------------------------------------------------------------------------- */

static int shape_ok(const oracle_shape* s)
{
    if (!s) return 0;
    if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->head_dim < 1) return 0;
    if (s->n_tokens < 1 || s->block_size < 1) return 0;
    if (s->n_q_heads % s->n_kv_heads != 0) return 0;
    if (s->dtype != OR_F32 && s->dtype != OR_BF16) return 0;
    return 1;
}

static int n_blocks(const oracle_shape* s) { return (s->n_tokens + s->block_size - 1) / s->block_size; }

/* Number of tokens in block b: L for every block but a ragged last one. */
static int block_count(const oracle_shape* s, int b)
{
    int c = s->n_tokens - b * s->block_size;
    return c < s->block_size ? c : s->block_size;
}

static double logit_scale(const oracle_shape* s)
{
    return s->scale != 0.0 ? s->scale : 1.0 / sqrt((double)s->head_dim);
}

/* scale * q . x for one stored query row and one stored key row. */
static double dot_scaled(const oracle_shape* s, const void* q, size_t q_off, const void* x,
                         size_t x_off)
{
    double acc = 0.0;
    for (int t = 0; t < s->head_dim; ++t)
        acc += elem(q, s->dtype, q_off + t) * elem(x, s->dtype, x_off + t);
    return logit_scale(s) * acc;
}

/* ln sum_i exp(v_i) over n values, computed around the maximum. */
static double log_sum_exp(const double* v, int n)
{
    double mx = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (v[i] > mx) mx = v[i];
    if (mx == -INFINITY) return -INFINITY;
    double sum = 0.0;
    for (int i = 0; i < n; ++i) sum += exp(v[i] - mx);
    return mx + log(sum);
}

/* Offsets of row 'row' of KV head j in batch b for [B, Hkv, rows, d] arrays. */
static size_t kv_off(const oracle_shape* s, int b, int j, int rows, int row)
{
    return (((size_t)b * s->n_kv_heads + j) * (size_t)rows + row) * (size_t)s->head_dim;
}

static size_t q_off(const oracle_shape* s, int b, int h)
{
    return ((size_t)b * s->n_q_heads + h) * (size_t)s->head_dim;
}

/* ----------------------------------------------------------------------------
 * Summaries (mean-pool per block; the proxy's key and value)
 * ------------------------------------------------------------------------- */

int oracle_kv_summary_build(const oracle_shape* s, const void* K, const void* V, void* Kbar,
                            void* Vbar)
{
    if (!shape_ok(s) || !K || !V || !Kbar || !Vbar) return -1;
    const int nb = n_blocks(s), d = s->head_dim;
    const int pairs = s->batch * s->n_kv_heads;
#pragma omp parallel for schedule(dynamic)
    for (int p = 0; p < pairs; ++p) {
        const int b = p / s->n_kv_heads, j = p % s->n_kv_heads;
        for (int blk = 0; blk < nb; ++blk) {
            const int c = block_count(s, blk);
            for (int t = 0; t < d; ++t) {
                double sk = 0.0, sv = 0.0;
                for (int i = 0; i < c; ++i) { /* tokens in order */
                    sk += elem(K, s->dtype, kv_off(s, b, j, s->n_tokens, blk * s->block_size + i) + t);
                    sv += elem(V, s->dtype, kv_off(s, b, j, s->n_tokens, blk * s->block_size + i) + t);
                }
                store(Kbar, s->dtype, kv_off(s, b, j, nb, blk) + t, sk / c);
                store(Vbar, s->dtype, kv_off(s, b, j, nb, blk) + t, sv / c);
            }
        }
    }
    return 0;
}

int oracle_kv_box_build(const oracle_shape* s, const void* K, void* Kbox)
{
    if (!shape_ok(s) || !K || !Kbox) return -1;
    const int nb = n_blocks(s), d = s->head_dim;
    const int pairs = s->batch * s->n_kv_heads;
#pragma omp parallel for schedule(dynamic)
    for (int p = 0; p < pairs; ++p) {
        const int b = p / s->n_kv_heads, j = p % s->n_kv_heads;
        for (int blk = 0; blk < nb; ++blk) {
            const int c = block_count(s, blk);
            for (int t = 0; t < d; ++t) {
                double lo = elem(K, s->dtype, kv_off(s, b, j, s->n_tokens, blk * s->block_size) + t), hi = lo;
                for (int i = 1; i < c; ++i) {
                    const double x = elem(K, s->dtype, kv_off(s, b, j, s->n_tokens, blk * s->block_size + i) + t);
                    if (x < lo) lo = x;
                    if (x > hi) hi = x;
                }
                store(Kbox, s->dtype, kv_off(s, b, j, 2 * nb, 2 * blk) + t, lo);
                store(Kbox, s->dtype, kv_off(s, b, j, 2 * nb, 2 * blk + 1) + t, hi);
            }
        }
    }
    return 0;
}

/* ----------------------------------------------------------------------------
 * Block logits and the group score
 * ------------------------------------------------------------------------- */

/* The largest q . k over the box [lo, hi] of a block: each coordinate of the
 * maximiser sits at whichever end of its range gives the larger product. */
static double box_dot_scaled(const oracle_shape* s, const void* q, size_t qo, const void* box, size_t lo_off,
                             size_t hi_off)
{
    double acc = 0.0;
    for (int t = 0; t < s->head_dim; ++t) {
        const double qt = elem(q, s->dtype, qo + t);
        const double a = qt * elem(box, s->dtype, lo_off + t), c = qt * elem(box, s->dtype, hi_off + t);
        acc += a > c ? a : c;
    }
    return acc * logit_scale(s);
}

int oracle_block_logits(const oracle_shape* s, int mode, const void* q, const void* keys,
                        double* logits)
{
    if (!shape_ok(s) || !q || !keys || !logits || mode < 0 || mode > 2) return -1;
    const int nb = n_blocks(s), G = s->n_q_heads / s->n_kv_heads;
#pragma omp parallel for schedule(dynamic)
    for (int bh = 0; bh < s->batch * s->n_q_heads; ++bh) {
        const int b = bh / s->n_q_heads, h = bh % s->n_q_heads, j = h / G;
        double* row = logits + (size_t)bh * nb;
        double* tok = (double*)malloc(sizeof(double) * (size_t)s->block_size);
        for (int blk = 0; blk < nb; ++blk) {
            const int c = block_count(s, blk);
            if (mode == 0) {
                /* first-order (mean-pool) estimate of ln m_b: ln c_b + scale q . kbar_b */
                row[blk] = dot_scaled(s, q, q_off(s, b, h), keys, kv_off(s, b, j, nb, blk)) + log((double)c);
            } else if (mode == 2) {
                /* the largest logit any point of the block's key box could give */
                row[blk] = box_dot_scaled(s, q, q_off(s, b, h), keys, kv_off(s, b, j, 2 * nb, 2 * blk),
                                          kv_off(s, b, j, 2 * nb, 2 * blk + 1));
            } else {
                /* exact ln m_b = ln sum_{i in b} exp(s_i) */
                for (int i = 0; i < c; ++i)
                    tok[i] = dot_scaled(s, q, q_off(s, b, h), keys,
                                        kv_off(s, b, j, s->n_tokens, blk * s->block_size + i));
                row[blk] = log_sum_exp(tok, c);
            }
        }
        free(tok);
    }
    return 0;
}

int oracle_group_score(const oracle_shape* s, const double* logits, double* score)
{
    if (!shape_ok(s) || !logits || !score) return -1;
    const int nb = n_blocks(s), G = s->n_q_heads / s->n_kv_heads;
#pragma omp parallel for schedule(dynamic)
    for (int p = 0; p < s->batch * s->n_kv_heads; ++p) {
        const int b = p / s->n_kv_heads, j = p % s->n_kv_heads;
        double* out = score + (size_t)p * nb;
        const double* first = logits + ((size_t)b * s->n_q_heads + (size_t)j * G) * nb;
        if (G == 1) {
            for (int blk = 0; blk < nb; ++blk) out[blk] = first[blk];
            continue;
        }
        double* lse_h = (double*)malloc(sizeof(double) * G);
        double* terms = (double*)malloc(sizeof(double) * G);
        for (int g = 0; g < G; ++g) lse_h[g] = log_sum_exp(first + (size_t)g * nb, nb);
        for (int blk = 0; blk < nb; ++blk) {
            /* ln P_b^(g) = logit_gb - ln Z^(g); score = ln sum_g P_b^(g) */
            for (int g = 0; g < G; ++g) terms[g] = first[(size_t)g * nb + blk] - lse_h[g];
            out[blk] = log_sum_exp(terms, G);
        }
        free(terms);
        free(lse_h);
    }
    return 0;
}

/* ----------------------------------------------------------------------------
 * Top-k with ties to the lower index
 * ------------------------------------------------------------------------- */

typedef struct {
    double score;
    int index;
} scored_block;

/* Total order: higher score first; equal scores (including +0 and -0) by lower index. */
static int by_score_then_index(const void* pa, const void* pb)
{
    const scored_block* a = (const scored_block*)pa;
    const scored_block* b = (const scored_block*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->index > b->index) - (a->index < b->index);
}

static int by_int(const void* pa, const void* pb)
{
    int a = *(const int32_t*)pa, b = *(const int32_t*)pb;
    return (a > b) - (a < b);
}

int oracle_topk(int rows, int nb, int k, const double* score, int32_t* sel, double* margin)
{
    if (rows < 0 || nb < 1 || k < 0 || !score || (k > 0 && !sel)) return -1;
    const int kk = k < nb ? k : nb;
#pragma omp parallel for schedule(dynamic)
    for (int r = 0; r < rows; ++r) {
        scored_block* v = (scored_block*)malloc(sizeof(scored_block) * (size_t)nb);
        for (int b = 0; b < nb; ++b) {
            v[b].score = score[(size_t)r * nb + b];
            v[b].index = b;
        }
        qsort(v, (size_t)nb, sizeof *v, by_score_then_index);
        for (int i = 0; i < kk; ++i) sel[(size_t)r * kk + i] = v[i].index;
        if (kk > 0) qsort(sel + (size_t)r * kk, (size_t)kk, sizeof(int32_t), by_int);
        if (margin) margin[r] = (kk > 0 && kk < nb) ? v[kk - 1].score - v[kk].score : INFINITY;
        free(v);
    }
    return 0;
}

/* ----------------------------------------------------------------------------
 * Attention over a list of virtual tokens
 * ------------------------------------------------------------------------- */

/* One virtual token: its logit and where its value row lives. */
typedef struct {
    double logit;
    const void* vbase;
    size_t voff;
} vtoken;

/* out = sum_e exp(l_e - M) val_e / sum_e exp(l_e - M); lse = M + ln sum_e exp(l_e - M). */
static void softmax_average(const oracle_shape* s, const vtoken* e, int ne, double* out,
                            double* lse)
{
    double mx = -INFINITY;
    for (int i = 0; i < ne; ++i)
        if (e[i].logit > mx) mx = e[i].logit;
    double denom = 0.0;
    for (int t = 0; t < s->head_dim; ++t) out[t] = 0.0;
    for (int i = 0; i < ne; ++i) {
        const double w = exp(e[i].logit - mx);
        denom += w;
        for (int t = 0; t < s->head_dim; ++t) out[t] += w * elem(e[i].vbase, s->dtype, e[i].voff + t);
    }
    for (int t = 0; t < s->head_dim; ++t) out[t] /= denom;
    *lse = mx + log(denom);
}

int oracle_attend(const oracle_shape* s, const void* q, const void* K, const void* V,
                  const void* Kbar, const void* Vbar, const int32_t* sel, int k,
                  const int32_t* tok_idx, const float* tok_logw, int m, int proxy_mode,
                  double* out, double* lse)
{
    if (!shape_ok(s) || !q || !K || !V || !out || !lse) return -1;
    const int nb = n_blocks(s), G = s->n_q_heads / s->n_kv_heads, n = s->n_tokens;
    if (k < 0 || k > nb || m < 0 || (proxy_mode != 0 && proxy_mode != 1)) return -1;
    if (k > 0 && !sel) return -1;
    if (m > 0 && (!tok_idx || !tok_logw)) return -1;
    if (proxy_mode == 1 && (!Kbar || !Vbar)) return -1;
    const int max_e = k * s->block_size + m + (proxy_mode ? nb : 0);
    if (max_e == 0) return -1; /* an empty virtual-token set has no softmax */
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int bh = 0; bh < s->batch * s->n_q_heads; ++bh) {
        const int b = bh / s->n_q_heads, h = bh % s->n_q_heads, j = h / G;
        const size_t pair = (size_t)b * s->n_kv_heads + j;
        const int32_t* S = sel ? sel + pair * (size_t)k : NULL;
        vtoken* e = (vtoken*)malloc(sizeof(vtoken) * (size_t)max_e);
        char* kept = (char*)calloc((size_t)nb, 1);
        int ne = 0;
        /* exact tokens of the kept blocks, log-weight 0 */
        for (int i = 0; i < k; ++i) {
            const int blk = S[i];
            if (blk < 0 || blk >= nb || kept[blk]) { bad = 1; continue; }
            kept[blk] = 1;
            for (int r = 0; r < block_count(s, blk); ++r) {
                const size_t off = kv_off(s, b, j, n, blk * s->block_size + r);
                e[ne].logit = dot_scaled(s, q, q_off(s, b, h), K, off);
                e[ne].vbase = V;
                e[ne].voff = off;
                ++ne;
            }
        }
        /* weighted tokens: logit + ln w */
        for (int t = 0; t < m; ++t) {
            const int idx = tok_idx[pair * (size_t)m + t];
            if (idx < 0 || idx >= n) { bad = 1; continue; }
            const size_t off = kv_off(s, b, j, n, idx);
            e[ne].logit = dot_scaled(s, q, q_off(s, b, h), K, off) + (double)tok_logw[pair * (size_t)m + t];
            e[ne].vbase = V;
            e[ne].voff = off;
            ++ne;
        }
        /* one count-aware proxy per unread block: mean key, mean value, + ln count */
        if (proxy_mode == 1) {
            for (int blk = 0; blk < nb; ++blk) {
                if (kept[blk]) continue;
                const size_t off = kv_off(s, b, j, nb, blk);
                e[ne].logit = dot_scaled(s, q, q_off(s, b, h), Kbar, off) + log((double)block_count(s, blk));
                e[ne].vbase = Vbar;
                e[ne].voff = off;
                ++ne;
            }
        }
        if (ne == 0)
            bad = 1;
        else
            softmax_average(s, e, ne, out + (size_t)bh * s->head_dim, lse + bh);
        free(kept);
        free(e);
    }
    return bad ? -1 : 0;
}

int oracle_dense(const oracle_shape* s, const void* q, const void* K, const void* V,
                 double* out, double* lse)
{
    if (!shape_ok(s) || !q || !K || !V || !out || !lse) return -1;
    const int G = s->n_q_heads / s->n_kv_heads, n = s->n_tokens;
#pragma omp parallel for schedule(dynamic)
    for (int bh = 0; bh < s->batch * s->n_q_heads; ++bh) {
        const int b = bh / s->n_q_heads, h = bh % s->n_q_heads, j = h / G;
        vtoken* e = (vtoken*)malloc(sizeof(vtoken) * (size_t)n);
        for (int i = 0; i < n; ++i) {
            const size_t off = kv_off(s, b, j, n, i);
            e[i].logit = dot_scaled(s, q, q_off(s, b, h), K, off);
            e[i].vbase = V;
            e[i].voff = off;
        }
        softmax_average(s, e, n, out + (size_t)bh * s->head_dim, lse + bh);
        free(e);
    }
    return 0;
}

int oracle_block_mass(const oracle_shape* s, const void* q, const void* K, const void* V,
                      double* ln_m, double* centroid)
{
    if (!shape_ok(s) || !q || !K || !V || !ln_m) return -1;
    const int nb = n_blocks(s), G = s->n_q_heads / s->n_kv_heads, n = s->n_tokens;
#pragma omp parallel for schedule(dynamic)
    for (int bh = 0; bh < s->batch * s->n_q_heads; ++bh) {
        const int b = bh / s->n_q_heads, h = bh % s->n_q_heads, j = h / G;
        vtoken* e = (vtoken*)malloc(sizeof(vtoken) * (size_t)s->block_size);
        double* tmp = (double*)malloc(sizeof(double) * (size_t)s->head_dim);
        for (int blk = 0; blk < nb; ++blk) {
            const int c = block_count(s, blk);
            for (int i = 0; i < c; ++i) {
                const size_t off = kv_off(s, b, j, n, blk * s->block_size + i);
                e[i].logit = dot_scaled(s, q, q_off(s, b, h), K, off);
                e[i].vbase = V;
                e[i].voff = off;
            }
            double l;
            softmax_average(s, e, c, tmp, &l);
            ln_m[(size_t)bh * nb + blk] = l;
            if (centroid)
                memcpy(centroid + ((size_t)bh * nb + blk) * s->head_dim, tmp,
                       sizeof(double) * (size_t)s->head_dim);
        }
        free(tmp);
        free(e);
    }
    return 0;
}

/* ----------------------------------------------------------------------------
 * Query-guided clusters ("OpenAttention reads 1% of the KV cache -- Count-aware
 * tail proxy", section "Three helpers that make the proxy accurate": keys are
 * projected onto the top eigenvectors of the queries and clustered by k-means
 * in that space once after prefill; each cluster then has one proxy).
 * ------------------------------------------------------------------------- */

/* Squared distance of projected point x to centroid c in r dimensions, the
 * coordinates taken in order. */
static double sq_dist(const double* x, const double* c, int r)
{
    double acc = 0.0;
    for (int j = 0; j < r; ++j) {
        const double t = x[j] - c[j];
        acc += t * t;
    }
    return acc;
}

/* Nearest centroid of x among C; equal distances go to the lower index. */
static int nearest(const double* x, const double* cent, int C, int r)
{
    int best = 0;
    double bd = sq_dist(x, cent, r);
    for (int c = 1; c < C; ++c) {
        const double dc = sq_dist(x, cent + (size_t)c * r, r);
        if (dc < bd) {
            bd = dc;
            best = c;
        }
    }
    return best;
}

int oracle_cluster_build(const oracle_shape* s, int C, int r, int iters, const void* K, const void* V,
                         const float* U, const int32_t* init_idx, int32_t* assign, int32_t* order,
                         int32_t* offsets, void* Kc, void* Vc, double* cent_out)
{
    if (!shape_ok(s) || C < 1 || r < 1 || iters < 0 || !K || !V || !U || !init_idx || !assign || !order ||
        !offsets || !Kc || !Vc)
        return -1;
    const int n = s->n_tokens, d = s->head_dim, pairs = s->batch * s->n_kv_heads;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int p = 0; p < pairs; ++p) {
        const int b = p / s->n_kv_heads, j = p % s->n_kv_heads;
        const float* Up = U + (size_t)p * d * r; /* [d, r] */
        double* P = (double*)malloc(sizeof(double) * (size_t)n * r);
        double* cent = (double*)malloc(sizeof(double) * (size_t)C * r);
        double* sum = (double*)malloc(sizeof(double) * (size_t)C * r);
        int* cnt = (int*)malloc(sizeof(int) * (size_t)C);
        int32_t* a = assign + (size_t)p * n;
        /* projections P_i = K_i U */
        for (int i = 0; i < n; ++i)
            for (int jj = 0; jj < r; ++jj) {
                double acc = 0.0;
                for (int t = 0; t < d; ++t)
                    acc += elem(K, s->dtype, kv_off(s, b, j, n, i) + t) * (double)Up[(size_t)t * r + jj];
                P[(size_t)i * r + jj] = acc;
            }
        /* initial centroids: the projections of the seed tokens */
        for (int c = 0; c < C; ++c) {
            const int i = init_idx[(size_t)p * C + c];
            if (i < 0 || i >= n) bad = 1;
            for (int jj = 0; jj < r; ++jj) cent[(size_t)c * r + jj] = (i >= 0 && i < n) ? P[(size_t)i * r + jj] : 0.0;
        }
        /* Lloyd's iterations: assign to the nearest centroid, move each centroid
         * to the mean of its points (an empty cluster keeps its centroid) */
        for (int it = 0; it <= iters; ++it) {
            for (int i = 0; i < n; ++i) a[i] = nearest(P + (size_t)i * r, cent, C, r);
            if (it == iters) break; /* the last assignment is to the final centroids */
            for (int c = 0; c < C; ++c) {
                cnt[c] = 0;
                for (int jj = 0; jj < r; ++jj) sum[(size_t)c * r + jj] = 0.0;
            }
            for (int i = 0; i < n; ++i) { /* tokens in order */
                cnt[a[i]] += 1;
                for (int jj = 0; jj < r; ++jj) sum[(size_t)a[i] * r + jj] += P[(size_t)i * r + jj];
            }
            for (int c = 0; c < C; ++c)
                if (cnt[c] > 0)
                    for (int jj = 0; jj < r; ++jj) cent[(size_t)c * r + jj] = sum[(size_t)c * r + jj] / cnt[c];
        }
        /* the gathered layout: tokens by cluster, in token order within one */
        int32_t* off = offsets + (size_t)p * (C + 1);
        for (int c = 0; c < C; ++c) cnt[c] = 0;
        for (int i = 0; i < n; ++i) cnt[a[i]] += 1;
        off[0] = 0;
        for (int c = 0; c < C; ++c) off[c + 1] = off[c] + cnt[c];
        int32_t* ord = order + (size_t)p * n;
        for (int c = 0; c < C; ++c) cnt[c] = 0;
        for (int i = 0; i < n; ++i) ord[off[a[i]] + cnt[a[i]]++] = i;
        /* per cluster the mean key and mean value, summed in token order in fp64,
         * rounded once (zero rows for an empty cluster) */
        for (int c = 0; c < C; ++c) {
            const int m = off[c + 1] - off[c];
            for (int t = 0; t < d; ++t) {
                double sk = 0.0, sv = 0.0;
                for (int o = off[c]; o < off[c + 1]; ++o) {
                    sk += elem(K, s->dtype, kv_off(s, b, j, n, ord[o]) + t);
                    sv += elem(V, s->dtype, kv_off(s, b, j, n, ord[o]) + t);
                }
                store(Kc, s->dtype, kv_off(s, b, j, C, c) + t, m > 0 ? sk / m : 0.0);
                store(Vc, s->dtype, kv_off(s, b, j, C, c) + t, m > 0 ? sv / m : 0.0);
            }
        }
        if (cent_out) memcpy(cent_out + (size_t)p * C * r, cent, sizeof(double) * (size_t)C * r);
        free(cnt);
        free(sum);
        free(cent);
        free(P);
    }
    return bad ? -1 : 0;
}

/* Cluster logits [B, Hq, C]: scale q_h . Kc_c + ln count_c (-inf for an empty
 * cluster), the count-aware proxy's logit of the section "Skipping reviews
 * without losing the verdict", per cluster instead of per block. */
int oracle_cluster_logits(const oracle_shape* s, int C, const void* q, const void* Kc, const int32_t* offsets,
                          double* logits)
{
    if (!shape_ok(s) || C < 1 || !q || !Kc || !offsets || !logits) return -1;
    const int G = s->n_q_heads / s->n_kv_heads;
#pragma omp parallel for schedule(dynamic)
    for (int bh = 0; bh < s->batch * s->n_q_heads; ++bh) {
        const int b = bh / s->n_q_heads, h = bh % s->n_q_heads, j = h / G;
        const int32_t* off = offsets + ((size_t)b * s->n_kv_heads + j) * (C + 1);
        for (int c = 0; c < C; ++c) {
            const int m = off[c + 1] - off[c];
            logits[(size_t)bh * C + c] =
                m > 0 ? dot_scaled(s, q, q_off(s, b, h), Kc, kv_off(s, b, j, C, c)) + log((double)m) : -INFINITY;
        }
    }
    return 0;
}

/* Attention over the virtual tokens of the clustered cache: every token of the
 * k selected clusters (log-weight 0) and, with proxies, one proxy per other
 * non-empty cluster (key Kc, value Vc, log-weight ln count).  The tokens of a
 * cluster are the order[] entries of its range. */
int oracle_cluster_attend(const oracle_shape* s, int C, const void* q, const void* K, const void* V,
                          const void* Kc, const void* Vc, const int32_t* order, const int32_t* offsets,
                          const int32_t* sel, int k, int proxy_mode, double* out, double* lse)
{
    if (!shape_ok(s) || C < 1 || !q || !K || !V || !order || !offsets || !out || !lse) return -1;
    if (k < 0 || k > C || (k > 0 && !sel) || (proxy_mode != 0 && proxy_mode != 1)) return -1;
    if (proxy_mode == 1 && (!Kc || !Vc)) return -1;
    const int G = s->n_q_heads / s->n_kv_heads, n = s->n_tokens;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int bh = 0; bh < s->batch * s->n_q_heads; ++bh) {
        const int b = bh / s->n_q_heads, h = bh % s->n_q_heads, j = h / G;
        const size_t pair = (size_t)b * s->n_kv_heads + j;
        const int32_t* off = offsets + pair * (C + 1);
        const int32_t* ord = order + pair * n;
        vtoken* e = (vtoken*)malloc(sizeof(vtoken) * ((size_t)n + C));
        char* kept = (char*)calloc((size_t)C, 1);
        int ne = 0;
        for (int i = 0; i < k; ++i) {
            const int c = sel[pair * k + i];
            if (c < 0 || c >= C || kept[c]) { bad = 1; continue; }
            kept[c] = 1;
            for (int o = off[c]; o < off[c + 1]; ++o) {
                const size_t ko = kv_off(s, b, j, n, ord[o]);
                e[ne].logit = dot_scaled(s, q, q_off(s, b, h), K, ko);
                e[ne].vbase = V;
                e[ne].voff = ko;
                ++ne;
            }
        }
        if (proxy_mode == 1)
            for (int c = 0; c < C; ++c) {
                const int m = off[c + 1] - off[c];
                if (kept[c] || m == 0) continue;
                const size_t co = kv_off(s, b, j, C, c);
                e[ne].logit = dot_scaled(s, q, q_off(s, b, h), Kc, co) + log((double)m);
                e[ne].vbase = Vc;
                e[ne].voff = co;
                ++ne;
            }
        if (ne == 0)
            bad = 1;
        else
            softmax_average(s, e, ne, out + (size_t)bh * s->head_dim, lse + bh);
        free(kept);
        free(e);
    }
    return bad ? -1 : 0;
}

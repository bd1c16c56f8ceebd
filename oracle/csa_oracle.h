/*
 * csa_oracle.h -- plain fp64 CPU oracle for selective decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code with the HIP
 * library: it has its own element decoding, its own rounding to the storage
 * type, its own log-sum-exp and its own sort.
 *
 * Sources (cited by page title and section / equation):
 *  - "OpenAttention reads 1% of the KV cache -- Count-aware tail proxy",
 *    section "Skipping reviews without losing the verdict": the count-aware
 *    proxy is one virtual token whose value is the mean value of the tokens it
 *    replaces and whose logit is their mean logit plus ln(count).
 *  - "COBS: Cumulant Order Block Sparse Attention", Eq. (1) block masses,
 *    Eqs. (2)-(3) discard-and-renormalise, Eq. (5) additive GQA block score,
 *    Eq. (18) first-order mean-pool score, and the OSA paragraph (exact masses).
 *  - "WildCat: Near-Linear Attention in Theory and Practice", Abstract:
 *    attention over a weighted subset of tokens.
 *
 * Conventions shared with the C-ABI (restated here, not included from there):
 *  - q is [B, Hq, d]; K, V are [B, Hkv, n, d]; Kbar, Vbar are [B, Hkv, nb, d];
 *    all row-major.  nb = ceil(n / L).  Query head h reads KV head h / G,
 *    G = Hq / Hkv.
 *  - dtype 0 = IEEE binary32, 1 = bfloat16 given as raw 16-bit patterns.
 *  - Every result is fp64.
 *
 * All functions return 0 on success and -1 on an invalid argument.
 */
#ifndef CSA_ORACLE_H
#define CSA_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_shape {
    int batch;       /* B   */
    int n_q_heads;   /* Hq  */
    int n_kv_heads;  /* Hkv */
    int head_dim;    /* d   */
    int n_tokens;    /* n   */
    int block_size;  /* L   */
    int dtype;       /* 0 = f32, 1 = bf16 */
    double scale;    /* logit scale; 0 means 1/sqrt(d) */
} oracle_shape;

/* Block summaries: per block the mean key and mean value, summed in fp64,
 * divided by the block's token count and rounded once to the storage dtype. */
int oracle_kv_summary_build(const oracle_shape* s, const void* K, const void* V,
                            void* Kbar, void* Vbar);

/* Box summaries (Quest, as analysed in "COBS: Cumulant Order Block Sparse
 * Attention", section on escaping the first-order ceiling): per block the
 * element-wise minimum and maximum of its keys, an axis-aligned bounding box.
 * Kbox is [B, Hkv, nb, 2, d]: row 2b the minimum, row 2b + 1 the maximum, in
 * the key dtype (a minimum or maximum of stored values is a stored value). */
int oracle_kv_box_build(const oracle_shape* s, const void* K, void* Kbox);

/* Round n fp64 values to the storage dtype (0 = f32, 1 = bf16 bit patterns),
 * to nearest with ties to even, in one step. */
int oracle_store_array(int dtype, size_t n, const double* x, void* out);

/* Per-query-head block logits [B, Hq, nb].
 * mode 0 (summary):    scale * q_h . Kbar_b + ln c_b          (COBS Eq. (18))
 * mode 1 (exact mass): ln m_hb = LSE_{i in b} scale * q_h . K_i (COBS Eq. (1))
 * mode 2 (box):        scale * max over the block's box of q_h . k
 *                      = scale * sum_t max(q_t min_bt, q_t max_bt)
 * keys is Kbar for mode 0, K for mode 1 and Kbox for mode 2. */
int oracle_block_logits(const oracle_shape* s, int mode, const void* q, const void* keys,
                        double* logits);

/* Group block score [B, Hkv, nb] from per-head block logits.
 * G = 1: the logit itself (ranking by log-mass, COBS Eq. (5) with G = 1).
 * G > 1: ln sum_{h in group} exp(logit_hb - LSE_b' logit_hb'), the logarithm
 *        of the sum of per-head normalised masses of COBS Eq. (5). */
int oracle_group_score(const oracle_shape* s, const double* logits, double* score);

/* Top-k per row: order by (score descending, index ascending), keep the first
 * min(k, nb) and write them in ascending index order to sel [rows, min(k, nb)].
 * margin (optional, [rows]) receives score_(k) - score_(k+1) in that order,
 * or +inf when every block is kept. */
int oracle_topk(int rows, int nb, int k, const double* score, int32_t* sel, double* margin);

/* Attention over the virtual-token set of each KV head:
 *   exact tokens of the selected blocks (log-weight 0),
 *   weighted tokens tok_idx / tok_logw [B, Hkv, m] (log-weight as given),
 *   and if proxy_mode == 1, one proxy per unselected block
 *   (key Kbar_b, value Vbar_b, log-weight ln c_b).
 * out [B, Hq, d], lse [B, Hq] (natural log). sel is [B, Hkv, k], k <= nb.
 * Kbar/Vbar may be NULL when proxy_mode == 0; tok_* may be NULL when m == 0. */
int oracle_attend(const oracle_shape* s, const void* q, const void* K, const void* V,
                  const void* Kbar, const void* Vbar, const int32_t* sel, int k,
                  const int32_t* tok_idx, const float* tok_logw, int m, int proxy_mode,
                  double* out, double* lse);

/* Dense softmax attention over all n tokens: out [B, Hq, d], lse [B, Hq]. */
int oracle_dense(const oracle_shape* s, const void* q, const void* K, const void* V,
                 double* out, double* lse);

/* Diagnostics for the identities of COBS Eqs. (1)-(3):
 * ln_m [B, Hq, nb] = ln of the exact block mass, and centroid [B, Hq, nb, d] =
 * the attention-weighted mean value of each block (may be NULL). */
int oracle_block_mass(const oracle_shape* s, const void* q, const void* K, const void* V,
                      double* ln_m, double* centroid);

/* Storage rounding exposed for the pins: fp64 -> bf16 bits (ties to even). */
/* Query-guided clusters ("OpenAttention reads 1% of the KV cache -- Count-aware
 * tail proxy", section "Three helpers that make the proxy accurate").  Per KV
 * head: projections P_i = K_i U (U [B, Hkv, d, r], fp32, the caller's basis:
 * the top-r eigenvectors of the queries' second moment), fp64, dimensions
 * summed in order; centroids start at the projections of the seed tokens
 * init_idx [B, Hkv, C]; `iters` rounds of (assign each token to the nearest
 * centroid by squared distance, ties to the lower index; move each centroid to
 * the mean of its points, summed in token order, an empty cluster keeping its
 * centroid), then a final assignment.  Outputs: assign [B, Hkv, n]; order
 * [B, Hkv, n] the tokens by cluster and token index; offsets [B, Hkv, C + 1]
 * the clusters' ranges in order; Kc, Vc [B, Hkv, C, d] the mean key and value
 * of each cluster (fp64 sums in token order, one rounding to the storage
 * dtype; zero rows for an empty cluster); cent_out [B, Hkv, C, r] (may be
 * NULL) the final centroids.  -1 on a seed index outside [0, n). */
int oracle_cluster_build(const oracle_shape* s, int C, int r, int iters, const void* K, const void* V,
                         const float* U, const int32_t* init_idx, int32_t* assign, int32_t* order,
                         int32_t* offsets, void* Kc, void* Vc, double* cent_out);

/* Cluster logits [B, Hq, C]: scale q_h . Kc_c + ln count_c, -inf for an empty
 * cluster. */
int oracle_cluster_logits(const oracle_shape* s, int C, const void* q, const void* Kc, const int32_t* offsets,
                          double* logits);

/* Attention over every token of the k selected clusters (log-weight 0) and,
 * with proxy_mode 1, one proxy per other non-empty cluster (Kc, Vc, ln count). */
int oracle_cluster_attend(const oracle_shape* s, int C, const void* q, const void* K, const void* V,
                          const void* Kc, const void* Vc, const int32_t* order, const int32_t* offsets,
                          const int32_t* sel, int k, int proxy_mode, double* out, double* lse);

uint16_t oracle_round_bf16(double x);

#ifdef __cplusplus
}
#endif

#endif /* CSA_ORACLE_H */

/*
 * csa.h -- C-ABI of libcsa.so: selective decode attention for MI355X (gfx950).
 *
 * A decode query attends to a small read of its KV cache: the exact tokens of
 * the top-k blocks of its KV head, optional weighted tokens, and one
 * count-aware mean proxy per unread block.  Sources, cited by page title and
 * section / equation:
 *   [OA]   "OpenAttention reads 1% of the KV cache -- Count-aware tail proxy",
 *          section "Skipping reviews without losing the verdict" (the proxy is
 *          one virtual token: mean value of the tokens it replaces, logit =
 *          their mean logit + ln count) and section "Three helpers that make
 *          the proxy accurate" (exact tokens and proxies in one online-softmax
 *          pass).
 *   [COBS] "COBS: Cumulant Order Block Sparse Attention": Eq. (1) block mass
 *          m_b, Eqs. (2)-(3) keep a block set and renormalise, Eq. (5) the
 *          additive GQA block score, Eq. (18) the first-order mean-pool score,
 *          and the OSA paragraph (exact masses from a dense key read).
 *   [WC]   "WildCat: Near-Linear Attention in Theory and Practice", Abstract:
 *          attention over a weighted subset, sum w e^s v / sum w e^s.
 *
 * Layout (all row-major, all device memory owned by the caller):
 *   q            [B, Hq, d]        dtype          (unscaled)
 *   K, V         [B, Hkv, n, d]    dtype
 *   Kbar, Vbar   [B, Hkv, nb, d]   dtype          nb = ceil(n / L)
 *   scores       [B, Hkv, nb]      float
 *   sel          [B, Hkv, k]       int32, strictly ascending block indices
 *   tok_idx      [B, Hkv, m]       int32 in [0, n)
 *   tok_logw     [B, Hkv, m]       float (natural-log weights, finite)
 *   out          [B, Hq, d]        float
 *   lse          [B, Hq]           float (natural log of the softmax denominator)
 * Query head h belongs to KV head h / G with G = Hq / Hkv.  Block b holds
 * tokens [b L, min(n, (b + 1) L)); c_b is its token count.  The logit of a
 * token is s_i = scale * q_h . K_i with scale = 1/sqrt(d) unless given.
 *
 * Conventions:
 *   - Every entry point validates its arguments on the host before launching
 *     anything; on a non-OK return nothing was launched and no output was
 *     touched.  csa_last_error() then describes the problem.
 *   - Launches are asynchronous on the given stream (NULL = the default
 *     stream); nothing synchronises.  A launch failure returns CSA_ERR_HIP.
 *   - Nothing is allocated.  Entry points that need scratch memory take a
 *     workspace (ws, ws_bytes) of at least csa_workspace_size() bytes, 256-byte
 *     aligned.  A workspace serves one call at a time; its contents between
 *     calls are meaningless.
 *   - No floating-point atomics: results are bitwise reproducible for the same
 *     inputs, shapes and device.
 *   - Supported in this version: dtype CSA_F32 or CSA_BF16, d in {64, 128},
 *     G <= 64, n <= 2^30, and one KV head's K (or V) below 4 GiB
 *     (n * d * element bytes < 2^32).  All pointers 16-byte aligned.
 *   - Inputs must be finite.  Indices outside their range are rejected only
 *     where the host can see them (sizes); device-resident index values are
 *     trusted unless csa_set_index_checks() turns their checks on.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa_status {
    CSA_OK = 0,
    CSA_ERR_INVALID_ARG = -1, /* null pointer, bad shape or size, misalignment */
    CSA_ERR_UNSUPPORTED = -2, /* valid but outside this version (d, dtype, G)  */
    CSA_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned    */
    CSA_ERR_HIP = -4          /* a HIP launch or query failed                  */
} csa_status;

typedef enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

typedef enum csa_score_mode {
    CSA_SCORE_SUMMARY = 0,    /* first-order score from the mean key  [COBS] Eq. (18) */
    CSA_SCORE_EXACT_MASS = 1, /* exact block mass from every key ("OSA")             */
    CSA_SCORE_BOX = 2,        /* best logit over the block's min/max key box (Quest) */
    CSA_SCORE_COBS2 = 3,      /* second-order (mean + covariance) estimate of ln m_b */
    CSA_SCORE_PROXY_ERROR = 4, /* estimated weight error of the block's proxy [OA]  */
    CSA_SCORE_COBS2_FP4 = 5    /* COBS2 from FP4 (E2M1) eigenvectors                */
} csa_score_mode;

/* Scaled eigenvectors per block in the second-order descriptor (kv_cov_build). */
#define CSA_COBS_RANK 4

typedef enum csa_proxy_mode {
    CSA_PROXY_NONE = 0,      /* unread blocks are discarded, the rest renormalised   */
    CSA_PROXY_COMPLEMENT = 1 /* one count-aware proxy per unread block       [OA]    */
} csa_proxy_mode;

typedef enum csa_entry {
    CSA_WS_BLOCK_SCORE_SUMMARY = 0,
    CSA_WS_BLOCK_SCORE_EXACT_MASS = 1,
    CSA_WS_SPARSE_DECODE_ATTN = 2,
    CSA_WS_DENSE_DECODE_ATTN = 3,
    CSA_WS_SELECTIVE_DECODE_STEP = 4,
    CSA_WS_BLOCK_SCORE_BOX = 5,
    CSA_WS_BLOCK_SCORE_COBS2 = 6,
    CSA_WS_BLOCK_SCORE_PROXY_ERROR = 7,
    CSA_WS_BLOCK_SCORE_COBS2_FP4 = 8,
    CSA_WS_KV_CLUSTER_BUILD = 9, /* k = n_clusters, m = rank */
    CSA_WS_CLUSTER_SCORE = 10,      /* k = n_clusters, m unused */
    CSA_WS_CLUSTER_DECODE_STEP = 11, /* k = clusters read exactly, m = n_clusters */
    CSA_WS_BLOCK_SCORE_COBS2_SUB = 12 /* block_score_cobs2_sub                       */
} csa_entry;

typedef struct csa_shape {
    int32_t batch;      /* B   >= 1                          */
    int32_t n_q_heads;  /* Hq  >= 1, a multiple of Hkv       */
    int32_t n_kv_heads; /* Hkv >= 1                          */
    int32_t head_dim;   /* d: 64 or 128                      */
    int32_t n_tokens;   /* n   >= 1                          */
    int32_t block_size; /* L   >= 1                          */
    csa_dtype dtype;    /* of q, K, V, Kbar, Vbar            */
    float scale;        /* logit scale; 0 means 1/sqrt(d)    */
} csa_shape;

/*
 * kv_summary_build -- per block, the mean key and the mean value
 * ([OA] "Skipping reviews...": the proxy value is the mean of the values it
 * replaces; [COBS] Eq. (18): the mean-pool summary is the mean key).
 * Kbar_b = round(sum_{i in b} K_i / c_b), summed in fp64 token by token, then
 * rounded once (to nearest, ties to even) to the storage dtype; Vbar alike.
 * Reads K, V [B, Hkv, n, d]; writes Kbar, Vbar [B, Hkv, nb, d].
 * Run once per cache (after prefill); no workspace.
 */
int kv_summary_build(const csa_shape* shape, const void* K, const void* V, void* Kbar, void* Vbar,
                     hipStream_t stream);

/*
 * kv_box_build -- per block, the element-wise minimum and maximum of its keys:
 * the axis-aligned bounding box that Quest caches, as analysed in [COBS]
 * (section on escaping the first-order ceiling).  Reads K [B, Hkv, n, d];
 * writes Kbox [B, Hkv, nb, 2, d] (row 0 the minimum, row 1 the maximum), in
 * the storage dtype: a minimum or maximum of stored values is stored exactly.
 * Run once per cache (after prefill); no workspace.
 */
int kv_box_build(const csa_shape* shape, const void* K, void* Kbox, hipStream_t stream);

/*
 * kv_cov_build -- per block, the second-order descriptor of [COBS] (the
 * cumulant expansion of ln m_b truncated at second order, with the block's key
 * covariance kept as its top CSA_COBS_RANK scaled eigenvectors): row 0 the
 * mean key (the same bits as kv_summary_build's Kbar), rows 1..CSA_COBS_RANK
 * xi_i = sqrt(lambda_i) u_i for the largest eigenvalues lambda_i of
 * Sigma_b = (1/c_b) sum_{i in b} (K_i - mean)(K_i - mean)^T, largest first,
 * each signed so that its largest-magnitude coordinate is positive; fp32
 * eigen-solve, rounded once to the storage dtype.  Reads K [B, Hkv, n, d];
 * writes Kcov [B, Hkv, nb, 1 + CSA_COBS_RANK, d].  Blocks of at most 64 tokens
 * (else CSA_ERR_UNSUPPORTED).  Run once per cache (after prefill); no workspace.
 */
int kv_cov_build(const csa_shape* shape, const void* K, void* Kcov, hipStream_t stream);

/*
 * kv_cov4_build -- the descriptor of kv_cov_build with its eigenvectors stored in
 * the E2M1 FP4 format, one fp32 scale per eigenvector, the mean key kept in
 * bfloat16 ([COBS] section on quantising the stored eigenvectors: at rank 4 and
 * d = 128 the covariance factor takes 272 bytes per block instead of 1024).
 * Per block, CSA_COV4_BLOCK_BYTES(d) bytes: the mean key (d bfloat16, the bits
 * of Kbar), the CSA_COBS_RANK scales s_i = max_t |xi_it| / 6 (binary32), then
 * for each eigenvector d/2 bytes of codes, coordinate 2t in the low and 2t + 1
 * in the high nibble of byte t.  xi_it is the bfloat16 value kv_cov_build
 * stores; its code is xi_it / s_i (binary32 quotient) rounded to the nearest of
 * +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even mantissa, zero as +0.  Reads
 * K [B, Hkv, n, d] (bfloat16 only, else CSA_ERR_UNSUPPORTED); writes Kcov4
 * [B, Hkv, nb, CSA_COV4_BLOCK_BYTES(d)] bytes.  Blocks of at most 64 tokens.
 */
#define CSA_COV4_BLOCK_BYTES(d) (2 * (d) + 4 * CSA_COBS_RANK + CSA_COBS_RANK * (d) / 2)
int kv_cov4_build(const csa_shape* shape, const void* K, void* Kcov4, hipStream_t stream);

/*
 * kv_cov_sub_build -- the query-subspace form of the second-order descriptor
 * ([COBS] section on keeping the covariance only within the query subspace:
 * ranking needs Sigma_b only through q^T Sigma_b q, so the covariance is kept
 * within the span of U, the top s eigenvectors of the queries' second moment).
 * U [Hkv, d, s] float (orthonormal columns, the caller's query statistics per KV
 * head, shared by the batch).  Per block: the mean key (the bits of
 * kv_summary_build's Kbar), then the top CSA_COBS_RANK scaled eigenvectors
 * xi_i = sqrt(mu_i) v_i of B_b = U^T Sigma_b U (s x s), largest first, each
 * signed so that its largest-magnitude coordinate is positive, rounded once to
 * the storage dtype and zero-padded to sps = s rounded up to 8 elements.  Writes
 * Kcs [B, Hkv, nb, CSA_COV_SUB_BLOCK_ELEMS(d, s)] elements of the cache dtype (at
 * d = 128, s = 85: the factors take 4 x 88 stored elements for the page's 340
 * against 512 of the full-space descriptor).  fp32 projection Y = X U of the
 * centred keys, then the Gram-matrix eigen-solve of kv_cov_build on Y.
 * 1 <= s <= d (CSA_ERR_INVALID_ARG otherwise); blocks of at most 64 tokens
 * (else CSA_ERR_UNSUPPORTED).  Run once per cache; no workspace.
 */
#define CSA_COV_SUB_BLOCK_ELEMS(d, s) ((d) + CSA_COBS_RANK * (((s) + 7) / 8 * 8))
int kv_cov_sub_build(const csa_shape* shape, int32_t s_dim, const void* K, const float* U, void* Kcs,
                     hipStream_t stream);

/*
 * block_score_cobs2_sub -- block scores from query-subspace descriptors: the block
 * logit scale q_h . Kbar_b + ln c_b + (1/2) scale^2 sum_i (qt_h . xi_bi)^2 with
 * qt_h = U^T q_h (fp32) the query's coordinates in its KV head's subspace, and the
 * group rule of block_score.  Kcs from kv_cov_sub_build with the same U and s.
 * bfloat16 and G <= 8 (else CSA_ERR_UNSUPPORTED).  Writes scores [B, Hkv, nb].
 * Workspace: csa_workspace_size(shape, CSA_WS_BLOCK_SCORE_COBS2_SUB, 0, 0) bytes.
 */
int block_score_cobs2_sub(const csa_shape* shape, int32_t s_dim, const void* q, const void* Kcs, const float* U,
                          float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * kv_cov_sub4_build, block_score_cobs2_sub4 -- the query-subspace descriptor with its
 * factors in E2M1 FP4, one fp32 scale each, the mean key in bfloat16 ([COBS]
 * section on quantising the stored factors, applied to the subspace factors).
 * Per block CSA_COV_SUB4_BLOCK_BYTES(d, s) bytes: the mean key (d bfloat16, the
 * bits of Kbar), the CSA_COBS_RANK scales s_i = max_t |xi_it| / 6 (binary32), then
 * for each factor spf/2 bytes of codes, spf = s rounded up to 32: coordinate 2t
 * in the low and 2t + 1 in the high nibble of byte t, zero codes past s.  xi_it is
 * the bfloat16 value kv_cov_sub_build stores; its code is xi_it / s_i (binary32)
 * rounded to the nearest of +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}, ties to the even
 * mantissa, zero as +0.  At d = 128, s = 85: 464 bytes per block (the factors
 * 208 of them, against 704 in bfloat16).  bfloat16 caches only (else
 * CSA_ERR_UNSUPPORTED); otherwise as kv_cov_sub_build and block_score_cobs2_sub
 * (same workspace entry).
 */
#define CSA_COV_SUB4_BLOCK_BYTES(d, s) (2 * (d) + 4 * CSA_COBS_RANK + CSA_COBS_RANK * (((s) + 31) / 32 * 32) / 2)
int kv_cov_sub4_build(const csa_shape* shape, int32_t s_dim, const void* K, const float* U, void* Kcs4,
                      hipStream_t stream);
int block_score_cobs2_sub4(const csa_shape* shape, int32_t s_dim, const void* q, const void* Kcs4, const float* U,
                           float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * kv_var_build -- per block, the mean and the variance tokens that the
 * proxy-error ranking of [OA] reads (section "Three helpers that make the
 * proxy accurate": mean and variance tokens cached per group of tokens, the
 * variance being the half row of the 1.5 rows per group; the error it
 * estimates is the one described in section "Skipping reviews without losing
 * the verdict"): row 0 the mean key (the same bits as kv_summary_build's
 * Kbar), row 1 the per-coordinate variance of the block's keys about their
 * exact mean, var_bt = (1/c_b) sum_{i in b} (K_it - mean_bt)^2, summed in fp64
 * token by token and rounded once to the storage dtype.  Reads K [B, Hkv, n, d];
 * writes Kvar [B, Hkv, nb, 2, d].  Run once per cache (after prefill); no
 * workspace.
 */
int kv_var_build(const csa_shape* shape, const void* K, void* Kvar, hipStream_t stream);

/*
 * block_score -- the score by which blocks are ranked, per KV head.
 * Per query head h and block b the block logit is
 *   SUMMARY:    l_hb = scale q_h . Kbar_b + ln c_b         (keys = Kbar)  [COBS] Eq. (18)
 *   EXACT_MASS: l_hb = ln m_hb = ln sum_{i in b} e^{s_i}   (keys = K)     [COBS] Eq. (1)
 *   BOX:        l_hb = scale sum_t max(q_t lo_bt, q_t hi_bt) (keys = Kbox), the
 *               largest logit any point of the block's key box could give
 *   COBS2:      l_hb = scale q_h . Kbar_b + ln c_b + (1/2) scale^2 sum_i (q_h . xi_bi)^2
 *               (keys = Kcov from kv_cov_build; bfloat16, G <= 8 and G nb <= 16384,
 *               else CSA_ERR_UNSUPPORTED)
 *   COBS2_FP4:  the COBS2 logit with xi_bi = s_i x E2M1(code) decoded from keys =
 *               Kcov4 (kv_cov4_build); the same conditions as COBS2
 *   PROXY_ERROR: l_hb = shat_hb + ln sigma_hb, the log of the estimated weight
 *               error of the block's proxy, its mass e^{shat_hb} times the spread
 *               of the logits it hides ([OA]), with shat_hb the SUMMARY logit and
 *               sigma_hb = scale sqrt(sum_t q_ht^2 var_bt) the standard deviation
 *               of the block's logits over its tokens when its key coordinates
 *               are uncorrelated (-inf when the block's keys are all equal: its
 *               proxy is exact).  keys = Kvar from kv_var_build; bfloat16,
 *               G <= 8 and G nb <= 16384, else CSA_ERR_UNSUPPORTED.
 * and the score of block b of KV head j is
 *   G = 1: l_hb (ranking by log-mass, [COBS] Eq. (5) with G = 1);
 *   G > 1: ln sum_{h in group j} exp(l_hb - ln sum_b' e^{l_hb'}),
 *          the logarithm of the additive GQA score of [COBS] Eq. (5);
 *          PROXY_ERROR normalises by the proxy masses instead,
 *          ln sum_h exp(l_hb - ln sum_b' e^{shat_hb'}): each head's error as a
 *          share of its estimated softmax denominator.
 * Writes scores [B, Hkv, nb].  Workspace: csa_workspace_size(shape,
 * CSA_WS_BLOCK_SCORE_SUMMARY, _EXACT_MASS, _BOX, _COBS2, _COBS2_FP4 or _PROXY_ERROR, 0, 0)
 * bytes (0 when G = 1).  One KV head's keys (K, or its summary or descriptor
 * rows) must be below 4 GiB, else CSA_ERR_UNSUPPORTED.
 */
int block_score(const csa_shape* shape, csa_score_mode mode, const void* q, const void* keys,
                float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * topk_select -- per row, the k blocks of largest score; equal scores (+0 and
 * -0 are equal) go to the lower index.  Selection is shared by the query heads
 * of a KV head ([COBS] Eq. (4)-(5): one block set per KV head).
 * scores [rows, nb] -> sel [rows, min(k, nb)] written in ascending index order.
 * k >= nb selects every block; k = 0 writes nothing.  Scores must not be NaN.
 */
int topk_select(int32_t rows, int32_t nb, int32_t k, const float* scores, int32_t* sel,
                hipStream_t stream);

/*
 * sparse_decode_attn -- one online-softmax pass over the virtual tokens of each
 * KV head ([OA] "Three helpers...": exact tokens and proxies in one pass):
 *   - every token of the k selected blocks sel (log-weight 0);
 *   - m weighted tokens tok_idx with log-weights tok_logw ([WC] Abstract);
 *   - with CSA_PROXY_COMPLEMENT, one proxy per block not in sel: key Kbar_b,
 *     value Vbar_b, log-weight ln c_b ([OA] "Skipping reviews...").
 * For each query head: l_e = scale q_h . key_e + logw_e, out_h = sum e^{l_e}
 * val_e / sum e^{l_e}, lse_h = ln sum e^{l_e}.  With CSA_PROXY_NONE and m = 0
 * this is keep-and-renormalise ([COBS] Eqs. (2)-(3)).
 * sel may be NULL when k = 0; tok_idx/tok_logw may be NULL when m = 0;
 * Kbar/Vbar may be NULL with CSA_PROXY_NONE; lse may be NULL.
 * 0 <= k <= nb; an empty virtual-token set (k = 0, m = 0, no proxies) is
 * CSA_ERR_INVALID_ARG.  Workspace: csa_workspace_size(shape,
 * CSA_WS_SPARSE_DECODE_ATTN, k, m) bytes.
 */
int sparse_decode_attn(const csa_shape* shape, const void* q, const void* K, const void* V,
                       const void* Kbar, const void* Vbar, const int32_t* sel, int32_t k,
                       const int32_t* tok_idx, const float* tok_logw, int32_t m,
                       csa_proxy_mode proxy_mode, float* out, float* lse, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * dense_decode_attn -- softmax attention over all n tokens (the reference the
 * sparse path approximates; [COBS] Eq. (1) with every block kept).
 * out [B, Hq, d], lse [B, Hq] (lse may be NULL).  Workspace:
 * csa_workspace_size(shape, CSA_WS_DENSE_DECODE_ATTN, 0, 0) bytes.
 */
int dense_decode_attn(const csa_shape* shape, const void* q, const void* K, const void* V,
                      float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * selective_decode_step -- block_score, topk_select and sparse_decode_attn of
 * one decode step in a single call, same results as calling the three in turn
 * (scores and selection bit for bit, outputs to rounding).
 * In summary mode the first-order block logit scale q_h . Kbar_b + ln c_b
 * ([COBS] Eq. (18)) is also the logit of the block's count-aware proxy ([OA]
 * "Skipping reviews...": mean logit + ln count), so where the shape allows
 * (bfloat16, G <= 8, k <= 32, nb <= 2048, and either B * Hkv >= 32 or a small
 * share per KV head over at most 512 blocks: (proxies + k L + m) G <= 4096
 * virtual rows times query heads) one kernel per KV head reads Kbar once, keeps
 * the logits on chip for both uses, selects the blocks and attends.  With fewer
 * KV heads the kernels are split over workgroups: beyond 512 blocks (and
 * 1 <= k <= 32) the logits, then each 128-block chunk's group scores and k best,
 * then the attention, whose workgroups rank those candidates themselves (and
 * with 5 to 8 heads take the proxies' logits from the split logits rather than
 * reading Kbar again), then the merge of the splits; otherwise the three entry
 * points run in turn.
 * keys = Kbar (SUMMARY) or K (EXACT_MASS) as for block_score (BOX, COBS2,
 * COBS2_FP4 and PROXY_ERROR scores are CSA_ERR_UNSUPPORTED here: they need Kbox, Kcov, Kcov4 or Kvar
 * besides Kbar; use the three entry points); Kbar may be NULL in EXACT_MASS
 * mode without proxies.  scores [B, Hkv, nb] and
 * sel [B, Hkv, min(k, nb)] are written when not NULL.  0 <= k; k = 0 with no
 * proxies and m = 0 is CSA_ERR_INVALID_ARG.  Workspace: csa_workspace_size(
 * shape, CSA_WS_SELECTIVE_DECODE_STEP, k, m) bytes.
 */
int selective_decode_step(const csa_shape* shape, csa_score_mode mode, const void* q, const void* K,
                          const void* V, const void* Kbar, const void* Vbar, int32_t k,
                          const int32_t* tok_idx, const float* tok_logw, int32_t m,
                          csa_proxy_mode proxy_mode, float* scores, int32_t* sel, float* out,
                          float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * selective_decode_step_noalloc -- selective_decode_step for callers that cannot
 * allocate device memory: code running under HIP graph capture, tight serving
 * loops and harnesses that forbid hipMalloc.  Same arguments, results and
 * errors as selective_decode_step, without the workspace: where that route
 * needs one, it uses a static device buffer of the library instead, of
 * CSA_STEP_NOALLOC_SCRATCH_BYTES bytes on each GPU (part of the loaded code
 * object, held until the process ends).  A shape whose workspace
 * (csa_workspace_size(shape, CSA_WS_SELECTIVE_DECODE_STEP, k, m)) is larger is
 * rejected with CSA_ERR_WORKSPACE before anything is launched.  The first call
 * on a GPU looks up the buffer's device address there (hipGetSymbolAddress,
 * which allocates nothing); no call allocates or frees memory.  Every call on
 * one GPU shares that GPU's buffer, so calls that overlap in time on one GPU
 * (different streams, or host threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.  Nothing in the buffer needs
 * to start at zero: every call writes what it reads.
 */
#define CSA_STEP_NOALLOC_SCRATCH_BYTES (64u << 20)
int selective_decode_step_noalloc(const csa_shape* shape, csa_score_mode mode, const void* q, const void* K,
                                  const void* V, const void* Kbar, const void* Vbar, int32_t k,
                                  const int32_t* tok_idx, const float* tok_logw, int32_t m,
                                  csa_proxy_mode proxy_mode, float* scores, int32_t* sel, float* out, float* lse,
                                  hipStream_t stream);

/*
 * Query-guided clusters ([OA] "Three helpers that make the proxy accurate":
 * the cache is clustered once after prefill so that each proxy hides tokens
 * with nearly equal logits -- keys are projected onto the top eigenvectors of
 * the queries and clustered by k-means in that space; the proxies of
 * "Skipping reviews..." then stand for clusters instead of fixed blocks).
 *
 * kv_cluster_build -- per KV head, with C = n_clusters and r = rank:
 *   1. projections P_i = K_i U in fp64 (U [B, Hkv, d, r] float, the caller's
 *      basis, e.g. the top r eigenvectors of the queries' second moment), the
 *      d products of a coordinate summed in order;
 *   2. centroids start at P of the seed tokens seeds [B, Hkv, C] (int32 in
 *      [0, n); a seed outside gives a zero centroid);
 *   3. `iters` rounds of: assign each token to the nearest centroid (squared
 *      distance over the r coordinates summed in order, ties to the lower
 *      index); move each centroid to the mean of its points summed in token
 *      order (an empty cluster keeps its centroid); then a final assignment;
 *   4. outputs: assign [B, Hkv, n] int32; order [B, Hkv, n] int32, the tokens
 *      by cluster and, within one, by index; offsets [B, Hkv, C + 1] int32,
 *      cluster c holding order[offsets[c] .. offsets[c + 1]); Kg, Vg
 *      [B, Hkv, n, d] the cache rows in that order; Kc, Vc [B, Hkv, C, d] the
 *      mean key and value of each cluster (fp64 sums in token order, one
 *      rounding to the storage dtype, zero rows for an empty cluster).
 * Every step is fp64 with products and sums rounded one by one, so the
 * results are the bits of a plain sequential evaluation.  Supported: r in
 * {4, 8, 16, 32}, 1 <= C <= 8192 and C r <= 8192 (else CSA_ERR_UNSUPPORTED),
 * iters >= 0.  Workspace: csa_workspace_size(shape, CSA_WS_KV_CLUSTER_BUILD,
 * C, r) bytes.  With index checks on (csa_set_index_checks) a seed outside
 * [0, n) is CSA_ERR_INVALID_ARG.  Run once per cache (after prefill).
 */
int kv_cluster_build(const csa_shape* shape, int32_t n_clusters, int32_t rank, int32_t iters, const void* K,
                     const void* V, const float* U, const int32_t* seeds, int32_t* assign, int32_t* order,
                     int32_t* offsets, void* Kg, void* Vg, void* Kc, void* Vc, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * cluster_score -- the score of each cluster, per KV head: the cluster logit
 * l_hc = scale q_h . Kc_c + ln count_c (-inf for an empty cluster; the logit of
 * the cluster's count-aware proxy, [OA] "Skipping reviews..."), combined over
 * the query heads of a KV head by the rule of block_score (G = 1: l_hc;
 * G > 1: ln sum_h exp(l_hc - ln sum_c' e^{l_hc'}), [COBS] Eq. (5)).
 * offsets from kv_cluster_build; writes scores [B, Hkv, C].  Workspace:
 * csa_workspace_size(shape, CSA_WS_CLUSTER_SCORE, C, 0) bytes (0 when G = 1).
 * The clusters to read are then topk_select(B Hkv, C, k, scores, sel).
 */
int cluster_score(const csa_shape* shape, int32_t n_clusters, const void* q, const void* Kc,
                  const int32_t* offsets, float* scores, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * cluster_decode_attn -- one online-softmax pass per KV head over every token of
 * the k selected clusters sel [B, Hkv, k] (log-weight 0; rows of Kg, Vg) and,
 * with CSA_PROXY_COMPLEMENT, one proxy per other non-empty cluster (key Kc_c,
 * value Vc_c, log-weight ln count_c) ([OA] "Three helpers...": exact tokens and
 * proxies in one pass).  out, lse as for sparse_decode_attn (lse may be NULL).
 * bfloat16 only (else CSA_ERR_UNSUPPORTED); G <= 8; 0 <= k <= min(C, 256);
 * k = 0 without proxies is CSA_ERR_INVALID_ARG.  A selection entry outside
 * [0, C) is skipped, a repeated one read twice (index checks reject both); a
 * KV head whose virtual-token set is empty (every selected cluster empty, no
 * proxies) gets NaN rows and lse -inf.  No workspace.
 */
int cluster_decode_attn(const csa_shape* shape, int32_t n_clusters, const void* q, const void* Kg, const void* Vg,
                        const void* Kc, const void* Vc, const int32_t* offsets, const int32_t* sel, int32_t k,
                        csa_proxy_mode proxy_mode, float* out, float* lse, hipStream_t stream);

/*
 * cluster_decode_step -- cluster_score, topk_select and cluster_decode_attn of one
 * decode step in one call (same scores and selection bit for bit, outputs to
 * rounding).  The cluster logit is the logit of the cluster's proxy, so the
 * ranking and the proxies share it: with 32 or more KV heads, k <= 32 and the
 * logits of C clusters within 64 KiB of on-chip memory, one kernel per KV head
 * ranks, selects and attends (the mean keys read once); otherwise, where the
 * shape allows (G C <= 16384, and k <= 32 with C <= 2048 for the selection),
 * one kernel per KV head computes the logits on the matrix cores, combines the
 * heads and selects, and a second kernel attends.  The conditions of
 * cluster_decode_attn apply; k >= C reads every cluster exactly.  scores
 * [B, Hkv, C] and sel [B, Hkv, min(k, C)] are written when not NULL.
 * Workspace: csa_workspace_size(shape, CSA_WS_CLUSTER_DECODE_STEP, k, C) bytes
 * (unused on the one-kernel route).
 */
int cluster_decode_step(const csa_shape* shape, int32_t n_clusters, const void* q, const void* Kg, const void* Vg,
                        const void* Kc, const void* Vc, const int32_t* offsets, int32_t k, csa_proxy_mode proxy_mode,
                        float* scores, int32_t* sel, float* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Workspace bytes needed by an entry point for this shape (k, m as the call
 * will pass them).  Returns 0 for an invalid shape (see csa_last_error()). */
size_t csa_workspace_size(const csa_shape* shape, csa_entry entry, int32_t k, int32_t m);

/* Static description of a status code. */
const char* csa_status_str(int status);

/* Detail of the last non-OK return on this host thread ("" if none). */
const char* csa_last_error(void);

/*
 * csa_set_index_checks -- debugging aid for the index arrays that live in
 * device memory and are otherwise trusted: with checks on, sparse_decode_attn
 * (sel, tok_idx), selective_decode_step (tok_idx), kv_cluster_build (seeds) and
 * cluster_decode_attn (sel, against [0, C)) first copy them to the
 * host, which waits for the earlier work on their stream (so such calls
 * synchronise and cannot be captured in a graph), and return
 * CSA_ERR_INVALID_ARG, launching nothing, for a selection row that names a
 * block twice or outside [0, nb), or a weighted token outside [0, n) -- the
 * inputs the fp64 reference rejects.  With checks off
 * (the default) those entries are excluded on the device: such a row or token
 * gets log-weight -inf.  The environment variable CSA_CHECK_INDICES=1 turns
 * the checks on from the first call.  Process-wide; returns the previous
 * setting (0 or 1).
 */
int csa_set_index_checks(int enable);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */

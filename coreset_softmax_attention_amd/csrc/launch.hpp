// launch.hpp -- host-side launchers of the libcsa kernels (internal interface
// between the C-ABI entry points and the kernel files).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

// Validated shape with derived quantities.
struct Dims {
    int B, Hq, Hkv, G, d, n, L, nb;
    int dtype;           // DT_F32 / DT_BF16
    float scale;         // logit scale (natural units)
    float ln_L, ln_last; // ln c_b of a full block and of the last block
    int pairs() const { return B * Hkv; }
};

// ---- summaries -------------------------------------------------------------
hipError_t launch_summary(const Dims& s, const void* K, const void* V, void* Kbar, void* Vbar,
                          hipStream_t st);

// ---- block scores ----------------------------------------------------------
// Per-head block logits (natural log units).  When G == 1 they are the scores
// and dst is scores [B, Hkv, nb]; otherwise dst is [B, Hq, nb] workspace.
hipError_t launch_block_logits_summary(const Dims& s, const void* q, const void* Kbar, float* dst,
                                       hipStream_t st);
hipError_t launch_block_logits_exact(const Dims& s, const void* q, const void* K, float* dst,
                                     hipStream_t st);
hipError_t launch_group_score(const Dims& s, const float* logits, float* scores, hipStream_t st);
// Box logits (Kbox [B, Hkv, nb, 2, d]); same destinations as the other logits.
hipError_t launch_block_logits_box(const Dims& s, const void* q, const void* Kbox, float* dst, hipStream_t st);
hipError_t launch_box(const Dims& s, const void* K, void* Kbox, hipStream_t st);
// Second-order descriptors Kcov [B, Hkv, nb, 1 + kCobsRank, d]: the mean key,
// then the top kCobsRank scaled eigenvectors of the block's key covariance.
constexpr int kCobsRank = 4;
bool cov_build_ok(const Dims& s);  // blocks of at most 64 tokens
hipError_t launch_cov(const Dims& s, const void* K, void* Kcov, hipStream_t st);
// Query-subspace descriptors Kcs [B, Hkv, nb, d + kCobsRank * sps] (sps = s
// rounded up to 8): the mean key, then the top kCobsRank scaled eigenvectors of
// U^T Sigma_b U for the caller's basis U [Hkv, d, s] (fp32).
bool cov_sub_ok(const Dims& s, int s_dim);  // cov_build_ok and 1 <= s <= min(d, 128)
hipError_t launch_cov_sub(const Dims& s, int s_dim, const void* K, const float* U, void* Kcs, hipStream_t st);
// The same with FP4 factors (bfloat16 caches): per block the mean key, kCobsRank fp32
// scales and kCobsRank x spf/2 bytes of E2M1 codes, spf = s rounded up to 32.
hipError_t launch_cov_sub4(const Dims& s, int s_dim, const void* K, const float* U, void* Kcs4, hipStream_t st);
// The same with FP4 eigenvectors (bfloat16 caches): per block the mean key,
// kCobsRank fp32 scales and kCobsRank x d/2 bytes of E2M1 codes.
hipError_t launch_cov4(const Dims& s, const void* K, void* Kcov4, hipStream_t st);
// Second-order block scores from Kcov, or from Kcov4 when fp4 (bfloat16,
// fused_summary_score_ok()).  Kcov, and Kcov4 with fewer than
// kFusedStepMinPairs KV heads, go through the tile-split kernel, whose logits
// land in `logits` ([B, Hq, nb], or the scores themselves when G == 1).
hipError_t launch_score_cobs2(const Dims& s, const void* q, const void* Kcov, float* logits, float* scores,
                              hipStream_t st, bool fp4 = false);
// Second-order scores from query-subspace descriptors (bfloat16, G <= 8): split
// kernels (logits to `logits`, the scores themselves when G == 1) and the
// group-score kernel.
// fp4: the descriptors of launch_cov_sub4.
hipError_t launch_score_cobs2_sub(const Dims& s, int s_dim, const void* q, const void* Kcs, const float* U,
                                  float* logits, float* scores, hipStream_t st, bool fp4 = false);
// Mean and variance tokens Kvar [B, Hkv, nb, 2, d] of the proxy-error scores.
hipError_t launch_var(const Dims& s, const void* K, void* Kvar, hipStream_t st);
// Proxy-error block scores from Kvar (bfloat16, fused_summary_score_ok()); with
// fewer than kFusedStepMinPairs KV heads the log-errors go through `logits`
// ([B, Hq, nb], or the scores themselves when G == 1) and the normaliser
// states through `parts` (score_err_parts_bytes()).
size_t score_err_parts_bytes(const Dims& s);
hipError_t launch_score_err(const Dims& s, const void* q, const void* Kvar, float* logits, float* parts,
                            float* scores, hipStream_t st);
// Summary mode with the logits, log-normalisers and group score in one kernel
// (one workgroup per KV head); available when fused_summary_score_ok().
bool fused_summary_score_ok(const Dims& s);
// box = true: box scores from Kbox rows ([min | max], 2d wide) instead of Kbar.
// offsets (clusters): per-row count terms ln(offsets[r + 1] - offsets[r]) from
// the ranges [B, Hkv, nb + 1] instead of the block sizes.  k > 0 (at most 32,
// nb <= 2048): the top-k of the scores to sel as well; scores may then be null.
hipError_t launch_score_summary_fused(const Dims& s, const void* q, const void* Kbar, float* scores, hipStream_t st,
                                      bool box = false, const int32_t* offsets = nullptr, int32_t* sel = nullptr,
                                      int k = 0);
// The same in two kernels for few KV heads: logits over (KV head, tile chunk)
// workgroups into `logits` ([B, Hq, nb]; may be `scores` when G == 1), then one
// workgroup per KV head for the group scores (to `scores`, may be null) and,
// when k > 0 (split_select_ok), the top-k to `sel`.
bool split_select_ok(const Dims& s, int k);
// Group scores (and the top-k when k > 0) from per-head logits [B, Hq, nb], one
// workgroup per KV head with the logits in LDS; when score_finish_ok().
bool score_finish_ok(const Dims& s);
// parts: per (KV head, tile of 32 rows, head) log-sum-exp states of the logits
// (score_err_parts_bytes()), from which the per-head normalisers come; else
// the normalisers are computed from the logits.
hipError_t launch_score_finish(const Dims& s, const float* logits, float* scores, int32_t* sel, int k, hipStream_t st,
                               const float* parts = nullptr);
// parts (G > 1, may be null; score_err_parts_bytes()): above
// kLseFromLogitsMaxBlocks blocks the tiles' log-sum-exp states pass through it
// and the group-score kernel takes the per-head normalisers from them; up to
// that many it computes them from the logits, as the one-workgroup kernels do.
// k < 0: the logits (and tile states) only, for launch_score_group_chunks.
hipError_t launch_score_summary_split(const Dims& s, const void* q, const void* Kbar, float* logits, float* scores,
                                      int32_t* sel, int k, hipStream_t st, bool box = false,
                                      const int32_t* offsets = nullptr, float* parts = nullptr);
// Group scores of the split logits (G > 1: to scores, with the normalisers from
// the tile states `parts`; G == 1: logits are the scores) and each chunk's top-k
// candidates, cand_score / cand_idx [B, Hkv, ceil(nb / kCandChunk), k]: nb above
// kLseFromLogitsMaxBlocks, 1 <= k <= 32, G <= 8.
hipError_t launch_score_group_chunks(const Dims& s, const float* logits, const float* parts, float* scores, int k,
                                     float* cand_score, int32_t* cand_idx, hipStream_t st);

// ---- top-k -----------------------------------------------------------------
hipError_t launch_topk(int rows, int nb, int k, const float* scores, int32_t* sel, hipStream_t st);

// ---- attention -------------------------------------------------------------
struct AttnPlan {
    int rows;            // virtual rows per KV head (exact + weighted + proxy, with padding)
    int exact_rows;      // rows of the exact segment (k L, or n for dense)
    int pend, wbeg, ebeg;  // end of the proxy rows, first weighted row, first exact row
    int hg;              // query heads per workgroup
    int hchunks;         // ceil(G / hg)
    int splits;          // workgroups per (KV head, head chunk)
    int rows_per_split;  // multiple of the wave tile
    int direct;          // MFMA kernel: rows from the global arrays, no LDS copies (a tile or two per wave)
    size_t ws_bytes;     // partial states when splits > 1
};

struct AttnInputs {
    const void* q;
    const void* K;
    const void* V;
    const void* Kbar;
    const void* Vbar;
    const int32_t* sel;
    int k;
    const int32_t* tok_idx;
    const float* tok_logw;
    int m;
    int proxies;
    int dense;
    float* out;
    float* lse;
    // Direct-mode plans only (AttnPlan::direct): with cand_score set, sel is not
    // read; every wave ranks the ncand candidates [B, Hkv, ncand] of
    // launch_score_group_chunks (ascending block order) for its k blocks, and
    // the first workgroup of each KV head writes them to sel_out when given.
    const float* cand_score = nullptr;
    const int32_t* cand_idx = nullptr;
    int ncand = 0;
    int32_t* sel_out = nullptr;
    // Direct-mode plans with proxies, nb a multiple of 4, 5 <= G <= 8 (else ignored):
    // the logits [B, Hq, nb] (natural log, count terms included) of the summary
    // scores, which the proxy rows then use instead of reading the mean keys.
    const float* plog = nullptr;
};

AttnPlan plan_attention(const Dims& s, int k, int m, int proxies, int dense);

// ---- fused decode step (summary score -> top-k -> attention, one launch) ----
constexpr int kFusedStepMinPairs = 32;  // below this, the split kernels use the GPU better
// With fewer KV heads the one-kernel step still wins while each KV head's
// share is small (its virtual rows times its query heads at most this much):
// one workgroup streams it faster than four split kernels launch one after
// another.  Measured on the 32-head / 8-KV-head layer at one and two sequences:
// 14.2 against 19.3 us at 8K tokens, 16.6 against 19.2 us at 32K; from 64K
// tokens (5376) and at G = 7 over 32K tokens (7168) the split kernels win.
constexpr long kFusedStepSmallWork = 4096;

// Up to this many blocks per KV head the per-head normalisers of the summary,
// box and cluster scores are computed from the logits in LDS, the same way in
// the one-workgroup kernels and in the group-score kernel of the split route.
// Beyond it the split route takes them from the tiles' log-sum-exp states,
// which its logit kernel forms in parallel (at 2048 blocks the pass over the
// logits cost the group-score kernel 2.5 us of its chain), and the one-kernel
// step with fewer than kFusedStepMinPairs KV heads is not taken: every shape
// keeps one arithmetic for its scores whichever entry point computes them.
constexpr int kLseFromLogitsMaxBlocks = 512;

// Beyond kLseFromLogitsMaxBlocks blocks the split route of the decode step
// ranks in two levels: one wave per chunk of kCandChunk blocks forms their group
// scores and its k best (launch_score_group_chunks), and the attention kernel
// ranks those candidates itself (AttnInputs::cand_*), so that no workgroup runs
// the whole KV head's group scores and top-k as one chain.
constexpr int kCandChunk = 128;

struct StepInputs {
    const void* q;
    const void* K;
    const void* V;
    const void* Kbar;
    const void* Vbar;
    int k;
    const int32_t* tok_idx;
    const float* tok_logw;
    int m;
    int proxies;
    float* scores;  // may be null
    int32_t* sel;   // may be null
    float* out;
    float* lse;     // may be null
};

// ---- query-guided clusters (cluster.hip) -----------------------------------
constexpr int kClusterMaxClusters = 8192;  // clusters per KV head
constexpr int kClusterMaxSel = 256;        // selected clusters per KV head
constexpr size_t kClusterCentroidLds = 65536;  // C r fp64 centroids in one workgroup's LDS

struct ClusterBuild {
    const void* K;
    const void* V;
    const float* U;        // [B, Hkv, d, r]
    const int32_t* seeds;  // [B, Hkv, C]
    int C, r, iters;
    int32_t* assign;   // [B, Hkv, n]
    int32_t* order;    // [B, Hkv, n]
    int32_t* offsets;  // [B, Hkv, C + 1]
    void* Kg;          // [B, Hkv, n, d] in cluster order
    void* Vg;
    void* Kc;          // [B, Hkv, C, d] cluster means
    void* Vc;
    double* proj;      // workspace: [B, Hkv, n, r] projections
    double* cent;      // workspace: [B, Hkv, C, r] centroids
};
bool cluster_build_ok(int C, int r);  // r in {4, 8, 16, 32}, C r doubles fit kClusterCentroidLds
size_t cluster_build_ws_bytes(const Dims& s, int C, int r);
hipError_t launch_cluster_build(const Dims& s, const ClusterBuild& cb, hipStream_t st);
// Cluster logits [B, Hq, C] (the scores themselves when G == 1).
hipError_t launch_cluster_logits(const Dims& s, int C, const void* q, const void* Kc, const int32_t* offsets,
                                 float* logits, hipStream_t st);
struct ClusterAttn {
    const void* q;
    const void* Kg;
    const void* Vg;
    const void* Kc;
    const void* Vc;
    const int32_t* offsets;
    const int32_t* sel;
    int C, k, proxies;
    float* out;
    float* lse;
};
hipError_t launch_cluster_attention(const Dims& s, const ClusterAttn& ca, hipStream_t st);

bool fused_step_ok(const Dims& s, int k, int m, int proxies);

// The decode step over query-guided clusters in one kernel per KV head (Dims
// with nb = the cluster count): cluster logits from the mean keys with count
// terms from the ranges, group scores, the top-k, then attention over the
// proxies (logits from LDS) and the selected clusters' rows of Kg / Vg.
struct ClusterStepInputs {
    const void* q;
    const void* Kg;
    const void* Vg;
    const void* Kc;
    const void* Vc;
    const int32_t* offsets;
    int k;
    int proxies;
    float* scores;  // may be null
    int32_t* sel;   // may be null
    float* out;
    float* lse;     // may be null
};
bool cluster_step_ok(const Dims& s, int k);  // bf16, G <= 8, k <= 32, nb <= 2048, >= 32 KV heads
hipError_t launch_cluster_step(const Dims& s, const ClusterStepInputs& in, hipStream_t st);
hipError_t launch_decode_step(const Dims& s, const StepInputs& in, hipStream_t st);
hipError_t launch_attention(const Dims& s, const AttnPlan& plan, const AttnInputs& in, void* ws,
                            hipStream_t st);

}  // namespace csa

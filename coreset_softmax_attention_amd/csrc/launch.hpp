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
// The same with FP4 eigenvectors (bfloat16 caches): per block the mean key,
// kCobsRank fp32 scales and kCobsRank x d/2 bytes of E2M1 codes.
hipError_t launch_cov4(const Dims& s, const void* K, void* Kcov4, hipStream_t st);
// Second-order block scores from Kcov, or from Kcov4 when fp4 (bfloat16,
// fused_summary_score_ok()).  Kcov, and Kcov4 with fewer than
// kFusedStepMinPairs KV heads, go through the tile-split kernel, whose logits
// land in `logits` ([B, Hq, nb], or the scores themselves when G == 1).
hipError_t launch_score_cobs2(const Dims& s, const void* q, const void* Kcov, float* logits, float* scores,
                              hipStream_t st, bool fp4 = false);
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
hipError_t launch_score_summary_fused(const Dims& s, const void* q, const void* Kbar, float* scores, hipStream_t st,
                                      bool box = false);
// The same in two kernels for few KV heads: logits over (KV head, tile chunk)
// workgroups into `logits` ([B, Hq, nb]; may be `scores` when G == 1), then one
// workgroup per KV head for the group scores (to `scores`, may be null) and,
// when k > 0 (split_select_ok), the top-k to `sel`.
bool split_select_ok(const Dims& s, int k);
// Group scores (and the top-k when k > 0) from per-head logits [B, Hq, nb], one
// workgroup per KV head with the logits in LDS; when score_finish_ok().
bool score_finish_ok(const Dims& s);
hipError_t launch_score_finish(const Dims& s, const float* logits, float* scores, int32_t* sel, int k, hipStream_t st);
hipError_t launch_score_summary_split(const Dims& s, const void* q, const void* Kbar, float* logits, float* scores,
                                      int32_t* sel, int k, hipStream_t st, bool box = false);

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

bool fused_step_ok(const Dims& s, int k, int m, int proxies);
hipError_t launch_decode_step(const Dims& s, const StepInputs& in, hipStream_t st);
hipError_t launch_attention(const Dims& s, const AttnPlan& plan, const AttnInputs& in, void* ws,
                            hipStream_t st);

}  // namespace csa

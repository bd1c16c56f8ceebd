// api.hip -- the C-ABI entry points of libcsa: argument validation on the host,
// workspace sizing, and dispatch to the kernel launchers.  Every check runs
// before any HIP call, so invalid calls launch nothing and touch no output.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/csa.h"
#include "device.hpp"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* where)
{
    return fail(CSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr long long kMaxRows = 1ll << 31;

// Validate a shape and derive the launch dimensions.
int make_dims(const csa_shape* sh, csa::Dims* d)
{
    if (!sh) return fail(CSA_ERR_INVALID_ARG, "shape is NULL");
    if (sh->batch < 1 || sh->n_q_heads < 1 || sh->n_kv_heads < 1 || sh->head_dim < 1 || sh->n_tokens < 1 ||
        sh->block_size < 1)
        return fail(CSA_ERR_INVALID_ARG, "shape has a non-positive size (B=%d Hq=%d Hkv=%d d=%d n=%d L=%d)",
                    sh->batch, sh->n_q_heads, sh->n_kv_heads, sh->head_dim, sh->n_tokens, sh->block_size);
    if (sh->n_q_heads % sh->n_kv_heads != 0)
        return fail(CSA_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", sh->n_q_heads,
                    sh->n_kv_heads);
    if (sh->dtype != CSA_F32 && sh->dtype != CSA_BF16)
        return fail(CSA_ERR_INVALID_ARG, "unknown dtype %d", (int)sh->dtype);
    if (!isfinite(sh->scale)) return fail(CSA_ERR_INVALID_ARG, "scale is not finite");
    if (sh->head_dim != 64 && sh->head_dim != 128)
        return fail(CSA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", sh->head_dim);
    if (sh->n_tokens > (1 << 30)) return fail(CSA_ERR_UNSUPPORTED, "n_tokens %d above 2^30", sh->n_tokens);
    const int G = sh->n_q_heads / sh->n_kv_heads;
    if (G > 64) return fail(CSA_ERR_UNSUPPORTED, "group size %d above 64", G);
    d->B = sh->batch;
    d->Hq = sh->n_q_heads;
    d->Hkv = sh->n_kv_heads;
    d->G = G;
    d->d = sh->head_dim;
    d->n = sh->n_tokens;
    d->L = sh->block_size < sh->n_tokens ? sh->block_size : sh->n_tokens;  // one ragged block if L >= n
    d->nb = (sh->n_tokens + d->L - 1) / d->L;
    d->dtype = sh->dtype == CSA_F32 ? csa::DT_F32 : csa::DT_BF16;
    d->scale = sh->scale != 0.0f ? sh->scale : (float)(1.0 / sqrt((double)sh->head_dim));
    d->ln_L = (float)log((double)d->L);
    d->ln_last = (float)log((double)(sh->n_tokens - (d->nb - 1) * d->L));
    return CSA_OK;
}

int check_ws(size_t need, const void* ws, size_t ws_bytes)
{
    if (need == 0) return CSA_OK;
    if (!ws) return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
    if (ws_bytes < need) return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need, ws_bytes);
    if (!aligned16(ws)) return fail(CSA_ERR_WORKSPACE, "workspace is not 16-byte aligned");
    return CSA_OK;
}

size_t block_score_ws(const csa::Dims& d)
{
    return d.G > 1 ? (size_t)d.B * d.Hq * d.nb * sizeof(float) : 0;
}

int attn_rows_ok(const csa::Dims& d, long long k, long long m, int proxies, int dense)
{
    const long long head_bytes = (long long)d.n * d.d * (d.dtype == csa::DT_F32 ? 4 : 2);
    if (head_bytes >= (1ll << 32))
        return fail(CSA_ERR_UNSUPPORTED, "one KV head's cache is %lld bytes (must be below 4 GiB)", head_bytes);
    const long long rows = (dense ? (long long)d.n : k * d.L) + m + (proxies ? d.nb : 0);
    if (rows >= kMaxRows) return fail(CSA_ERR_UNSUPPORTED, "virtual-token list of %lld rows above 2^31", rows);
    return CSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Proxy-error scores: the log-errors, then the per-tile normaliser states.
size_t error_score_ws(const csa::Dims& d)
{
    return d.G > 1 ? align256(block_score_ws(d)) + csa::score_err_parts_bytes(d) : 0;
}

// Workspace layout of the unfused decode step: scores | sel | block_score ws | attention ws.
struct StepWs {
    size_t scores, sel, score_ws, attn_ws, total;
};

StepWs step_ws(const csa::Dims& d, int k, int m)
{
    StepWs w{};
    const int kk = k < d.nb ? k : d.nb;
    w.scores = align256((size_t)d.pairs() * d.nb * sizeof(float));
    w.sel = align256((size_t)d.pairs() * (kk > 0 ? kk : 1) * sizeof(int32_t));
    w.score_ws = align256(block_score_ws(d));
    const size_t a = csa::plan_attention(d, kk, m, 1, 0).ws_bytes;
    const size_t b = (kk > 0 || m > 0) ? csa::plan_attention(d, kk, m, 0, 0).ws_bytes : 0;
    w.attn_ws = align256(a > b ? a : b);
    w.total = w.scores + w.sel + w.score_ws + w.attn_ws;
    return w;
}

}  // namespace

extern "C" {

int kv_summary_build(const csa_shape* shape, const void* K, const void* V, void* Kbar, void* Vbar, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!K || !V || !Kbar || !Vbar) return fail(CSA_ERR_INVALID_ARG, "kv_summary_build: NULL tensor pointer");
    if (!aligned16(K) || !aligned16(V) || !aligned16(Kbar) || !aligned16(Vbar))
        return fail(CSA_ERR_INVALID_ARG, "kv_summary_build: tensors must be 16-byte aligned");
    const hipError_t e = csa::launch_summary(d, K, V, Kbar, Vbar, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "kv_summary_build");
}

int kv_box_build(const csa_shape* shape, const void* K, void* Kbox, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!K || !Kbox) return fail(CSA_ERR_INVALID_ARG, "kv_box_build: NULL tensor pointer");
    if (!aligned16(K) || !aligned16(Kbox)) return fail(CSA_ERR_INVALID_ARG, "kv_box_build: tensors must be 16-byte aligned");
    const hipError_t e = csa::launch_box(d, K, Kbox, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "kv_box_build");
}

int kv_cov_build(const csa_shape* shape, const void* K, void* Kcov, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!K || !Kcov) return fail(CSA_ERR_INVALID_ARG, "kv_cov_build: NULL tensor pointer");
    if (!aligned16(K) || !aligned16(Kcov)) return fail(CSA_ERR_INVALID_ARG, "kv_cov_build: tensors must be 16-byte aligned");
    if (!csa::cov_build_ok(d))
        return fail(CSA_ERR_UNSUPPORTED, "kv_cov_build: blocks of %d tokens (at most 64 supported)", d.L);
    const hipError_t e = csa::launch_cov(d, K, Kcov, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "kv_cov_build");
}

int kv_cov4_build(const csa_shape* shape, const void* K, void* Kcov4, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!K || !Kcov4) return fail(CSA_ERR_INVALID_ARG, "kv_cov4_build: NULL tensor pointer");
    if (!aligned16(K) || !aligned16(Kcov4))
        return fail(CSA_ERR_INVALID_ARG, "kv_cov4_build: tensors must be 16-byte aligned");
    if (d.dtype != csa::DT_BF16) return fail(CSA_ERR_UNSUPPORTED, "kv_cov4_build: FP4 descriptors need a bfloat16 cache");
    if (!csa::cov_build_ok(d))
        return fail(CSA_ERR_UNSUPPORTED, "kv_cov4_build: blocks of %d tokens (at most 64 supported)", d.L);
    const hipError_t e = csa::launch_cov4(d, K, Kcov4, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "kv_cov4_build");
}

int kv_var_build(const csa_shape* shape, const void* K, void* Kvar, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!K || !Kvar) return fail(CSA_ERR_INVALID_ARG, "kv_var_build: NULL tensor pointer");
    if (!aligned16(K) || !aligned16(Kvar)) return fail(CSA_ERR_INVALID_ARG, "kv_var_build: tensors must be 16-byte aligned");
    const hipError_t e = csa::launch_var(d, K, Kvar, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "kv_var_build");
}

int block_score(const csa_shape* shape, csa_score_mode mode, const void* q, const void* keys, float* scores, void* ws,
                size_t ws_bytes, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (mode != CSA_SCORE_SUMMARY && mode != CSA_SCORE_EXACT_MASS && mode != CSA_SCORE_BOX && mode != CSA_SCORE_COBS2 &&
        mode != CSA_SCORE_PROXY_ERROR && mode != CSA_SCORE_COBS2_FP4)
        return fail(CSA_ERR_INVALID_ARG, "block_score: unknown mode %d", (int)mode);
    {  // the kernels address one KV head's key rows with 32-bit offsets
        const long long row = (long long)d.d * (d.dtype == csa::DT_F32 ? 4 : 2);
        const long long rows_per_block = mode == CSA_SCORE_BOX || mode == CSA_SCORE_PROXY_ERROR ? 2
                                         : mode == CSA_SCORE_COBS2                              ? 5
                                                                                                : 1;
        const long long key_bytes = mode == CSA_SCORE_EXACT_MASS  ? (long long)d.n * row
                                    : mode == CSA_SCORE_COBS2_FP4 ? (long long)d.nb * CSA_COV4_BLOCK_BYTES(d.d)
                                                                  : (long long)d.nb * rows_per_block * row;
        if (key_bytes >= (1ll << 32))
            return fail(CSA_ERR_UNSUPPORTED, "block_score: one KV head's keys are %lld bytes (must be below 4 GiB)",
                        key_bytes);
    }
    if ((mode == CSA_SCORE_COBS2 || mode == CSA_SCORE_COBS2_FP4) && !csa::fused_summary_score_ok(d))
        return fail(CSA_ERR_UNSUPPORTED, "block_score: second-order scores need bfloat16, G <= 8 and G nb <= 16384");
    if (mode == CSA_SCORE_PROXY_ERROR && !csa::fused_summary_score_ok(d))
        return fail(CSA_ERR_UNSUPPORTED, "block_score: proxy-error scores need bfloat16, G <= 8 and G nb <= 16384");
    if (!q || !keys || !scores) return fail(CSA_ERR_INVALID_ARG, "block_score: NULL tensor pointer");
    if (!aligned16(q) || !aligned16(keys) || !aligned4(scores))
        return fail(CSA_ERR_INVALID_ARG, "block_score: misaligned tensor");
    if (mode == CSA_SCORE_PROXY_ERROR) {
        if (int rc = check_ws(error_score_ws(d), ws, ws_bytes)) return rc;
        float* lg = d.G == 1 ? scores : static_cast<float*>(ws);
        float* parts = d.G == 1 ? nullptr
                                : reinterpret_cast<float*>(static_cast<char*>(ws) + align256(block_score_ws(d)));
        const hipError_t e = csa::launch_score_err(d, q, keys, lg, parts, scores, stream);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "block_score");
    }
    if (int rc = check_ws(block_score_ws(d), ws, ws_bytes)) return rc;
    if (mode == CSA_SCORE_COBS2 || mode == CSA_SCORE_COBS2_FP4) {
        const hipError_t e = csa::launch_score_cobs2(d, q, keys, d.G == 1 ? scores : static_cast<float*>(ws), scores,
                                                     stream, mode == CSA_SCORE_COBS2_FP4);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "block_score");
    }
    if ((mode == CSA_SCORE_SUMMARY || mode == CSA_SCORE_BOX) && csa::fused_summary_score_ok(d)) {
        // matrix cores; one workgroup per KV head when there are enough of them, else the split kernels
        const bool box = mode == CSA_SCORE_BOX;
        const hipError_t e =
            d.pairs() >= csa::kFusedStepMinPairs
                ? csa::launch_score_summary_fused(d, q, keys, scores, stream, box)
                : csa::launch_score_summary_split(d, q, keys, d.G == 1 ? scores : static_cast<float*>(ws), scores,
                                                  nullptr, 0, stream, box);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "block_score");
    }
    float* dst = d.G == 1 ? scores : static_cast<float*>(ws);
    hipError_t e = mode == CSA_SCORE_SUMMARY ? csa::launch_block_logits_summary(d, q, keys, dst, stream)
                   : mode == CSA_SCORE_BOX   ? csa::launch_block_logits_box(d, q, keys, dst, stream)
                                             : csa::launch_block_logits_exact(d, q, keys, dst, stream);
    if (e != hipSuccess) return hip_fail(e, "block_score");
    if (d.G > 1) {
        e = csa::score_finish_ok(d) ? csa::launch_score_finish(d, dst, scores, nullptr, 0, stream)
                                    : csa::launch_group_score(d, dst, scores, stream);
        if (e != hipSuccess) return hip_fail(e, "block_score (group score)");
    }
    return CSA_OK;
}

int topk_select(int32_t rows, int32_t nb, int32_t k, const float* scores, int32_t* sel, hipStream_t stream)
{
    if (rows < 0 || nb < 1 || k < 0)
        return fail(CSA_ERR_INVALID_ARG, "topk_select: rows=%d nb=%d k=%d", rows, nb, k);
    if (rows == 0 || k == 0) return CSA_OK;
    if (!scores || !sel) return fail(CSA_ERR_INVALID_ARG, "topk_select: NULL pointer");
    if (!aligned4(scores) || !aligned4(sel)) return fail(CSA_ERR_INVALID_ARG, "topk_select: misaligned pointer");
    const hipError_t e = csa::launch_topk(rows, nb, k, scores, sel, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "topk_select");
}

int sparse_decode_attn(const csa_shape* shape, const void* q, const void* K, const void* V, const void* Kbar,
                       const void* Vbar, const int32_t* sel, int32_t k, const int32_t* tok_idx,
                       const float* tok_logw, int32_t m, csa_proxy_mode proxy_mode, float* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (proxy_mode != CSA_PROXY_NONE && proxy_mode != CSA_PROXY_COMPLEMENT)
        return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: unknown proxy mode %d", (int)proxy_mode);
    const int proxies = proxy_mode == CSA_PROXY_COMPLEMENT;
    if (k < 0 || k > d.nb) return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: k=%d outside [0, %d]", k, d.nb);
    if (m < 0) return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: m=%d is negative", m);
    if (k == 0 && m == 0 && !proxies)
        return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: empty virtual-token set (k = 0, m = 0, no proxies)");
    if (!q || !K || !V || !out) return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: NULL tensor pointer");
    if (k > 0 && !sel) return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: sel is NULL with k=%d", k);
    if (m > 0 && (!tok_idx || !tok_logw))
        return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: weighted tokens missing with m=%d", m);
    if (proxies && (!Kbar || !Vbar)) return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: proxies need Kbar, Vbar");
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || (proxies && (!aligned16(Kbar) || !aligned16(Vbar))) ||
        !aligned4(out) || (lse && !aligned4(lse)) || (sel && !aligned4(sel)) || (tok_idx && !aligned4(tok_idx)) ||
        (tok_logw && !aligned4(tok_logw)))
        return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: misaligned pointer");
    if (int rc = attn_rows_ok(d, k, m, proxies, 0)) return rc;
    const csa::AttnPlan plan = csa::plan_attention(d, k, m, proxies, 0);
    if (int rc = check_ws(plan.ws_bytes, ws, ws_bytes)) return rc;
    csa::AttnInputs in{q, K, V, Kbar, Vbar, sel, k, tok_idx, tok_logw, m, proxies, 0, out, lse};
    const hipError_t e = csa::launch_attention(d, plan, in, ws, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "sparse_decode_attn");
}

int dense_decode_attn(const csa_shape* shape, const void* q, const void* K, const void* V, float* out, float* lse,
                      void* ws, size_t ws_bytes, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!q || !K || !V || !out) return fail(CSA_ERR_INVALID_ARG, "dense_decode_attn: NULL tensor pointer");
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned4(out) || (lse && !aligned4(lse)))
        return fail(CSA_ERR_INVALID_ARG, "dense_decode_attn: misaligned pointer");
    if (int rc = attn_rows_ok(d, 0, 0, 0, 1)) return rc;
    const csa::AttnPlan plan = csa::plan_attention(d, 0, 0, 0, 1);
    if (int rc = check_ws(plan.ws_bytes, ws, ws_bytes)) return rc;
    csa::AttnInputs in{q, K, V, nullptr, nullptr, nullptr, 0, nullptr, nullptr, 0, 0, 1, out, lse};
    const hipError_t e = csa::launch_attention(d, plan, in, ws, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "dense_decode_attn");
}

int selective_decode_step(const csa_shape* shape, csa_score_mode mode, const void* q, const void* K, const void* V,
                          const void* Kbar, const void* Vbar, int32_t k, const int32_t* tok_idx,
                          const float* tok_logw, int32_t m, csa_proxy_mode proxy_mode, float* scores, int32_t* sel,
                          float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (mode == CSA_SCORE_BOX || mode == CSA_SCORE_COBS2 || mode == CSA_SCORE_PROXY_ERROR ||
        mode == CSA_SCORE_COBS2_FP4)
        return fail(CSA_ERR_UNSUPPORTED, "selective_decode_step: box, second-order and proxy-error scores need "
                                         "Kbox, Kcov or Kvar; call block_score, topk_select and sparse_decode_attn");
    if (mode != CSA_SCORE_SUMMARY && mode != CSA_SCORE_EXACT_MASS)
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: unknown mode %d", (int)mode);
    if (proxy_mode != CSA_PROXY_NONE && proxy_mode != CSA_PROXY_COMPLEMENT)
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: unknown proxy mode %d", (int)proxy_mode);
    const int proxies = proxy_mode == CSA_PROXY_COMPLEMENT;
    if (k < 0 || m < 0) return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: k=%d m=%d", k, m);
    const int kk = k < d.nb ? k : d.nb;
    if (kk == 0 && m == 0 && !proxies)
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: empty virtual-token set (k = 0, m = 0, no proxies)");
    if (!q || !K || !V || !out) return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: NULL tensor pointer");
    if ((mode == CSA_SCORE_SUMMARY || proxies) && !Kbar)
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: Kbar is NULL");
    if (proxies && !Vbar) return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: proxies need Vbar");
    if (m > 0 && (!tok_idx || !tok_logw))
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: weighted tokens missing with m=%d", m);
    if (!aligned16(q) || !aligned16(K) || !aligned16(V) || (Kbar && !aligned16(Kbar)) || (Vbar && !aligned16(Vbar)) ||
        !aligned4(out) || (lse && !aligned4(lse)) || (scores && !aligned4(scores)) || (sel && !aligned4(sel)) ||
        (tok_idx && !aligned4(tok_idx)) || (tok_logw && !aligned4(tok_logw)))
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: misaligned pointer");
    if (int rc = attn_rows_ok(d, kk, m, proxies, 0)) return rc;

    if (mode == CSA_SCORE_SUMMARY && csa::fused_step_ok(d, kk, m, proxies)) {
        csa::StepInputs in{q, K, V, Kbar, Vbar, kk, tok_idx, tok_logw, m, proxies, scores, sel, out, lse};
        const hipError_t e = csa::launch_decode_step(d, in, stream);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "selective_decode_step");
    }
    // the three kernels in turn; scores and selection go to the caller's arrays
    // when given, else to the workspace
    const StepWs w = step_ws(d, kk, m);
    if (int rc = check_ws(w.total, ws, ws_bytes)) return rc;
    char* base = static_cast<char*>(ws);
    float* sc = scores ? scores : reinterpret_cast<float*>(base);
    int32_t* sl = sel ? sel : reinterpret_cast<int32_t*>(base + w.scores);
    void* sws = base + w.scores + w.sel;
    void* aws = base + w.scores + w.sel + w.score_ws;
    if (mode == CSA_SCORE_SUMMARY && csa::fused_summary_score_ok(d) && d.pairs() < csa::kFusedStepMinPairs &&
        csa::split_select_ok(d, kk)) {
        // scores and selection from the split kernels (the top-k rides on the group-score kernel)
        const hipError_t e = csa::launch_score_summary_split(d, q, Kbar, d.G == 1 ? sc : static_cast<float*>(sws),
                                                             sc, sl, kk, stream);
        if (e != hipSuccess) return hip_fail(e, "selective_decode_step (score)");
    } else if (mode == CSA_SCORE_EXACT_MASS && d.G > 1 && csa::score_finish_ok(d) && csa::split_select_ok(d, kk)) {
        // exact masses, then group scores and selection in one kernel
        float* lg = static_cast<float*>(sws);
        hipError_t e = csa::launch_block_logits_exact(d, q, K, lg, stream);
        if (e == hipSuccess) e = csa::launch_score_finish(d, lg, sc, sl, kk, stream);
        if (e != hipSuccess) return hip_fail(e, "selective_decode_step (score)");
    } else {
        if (int rc = block_score(shape, mode, q, mode == CSA_SCORE_SUMMARY ? Kbar : K, sc, sws, w.score_ws, stream))
            return rc;
        if (int rc = topk_select(d.pairs(), d.nb, kk, sc, sl, stream)) return rc;
    }
    return sparse_decode_attn(shape, q, K, V, Kbar, Vbar, kk > 0 ? sl : nullptr, kk, tok_idx, tok_logw, m,
                              proxy_mode, out, lse, aws, w.attn_ws, stream);
}

size_t csa_workspace_size(const csa_shape* shape, csa_entry entry, int32_t k, int32_t m)
{
    csa::Dims d;
    if (make_dims(shape, &d) != CSA_OK) return 0;
    switch (entry) {
    case CSA_WS_BLOCK_SCORE_SUMMARY:
    case CSA_WS_BLOCK_SCORE_EXACT_MASS:
    case CSA_WS_BLOCK_SCORE_BOX:
    case CSA_WS_BLOCK_SCORE_COBS2:
    case CSA_WS_BLOCK_SCORE_COBS2_FP4: return block_score_ws(d);
    case CSA_WS_BLOCK_SCORE_PROXY_ERROR: return error_score_ws(d);
    case CSA_WS_SPARSE_DECODE_ATTN: {
        if (k < 0 || k > d.nb || m < 0) {
            fail(CSA_ERR_INVALID_ARG, "csa_workspace_size: k=%d or m=%d out of range", k, m);
            return 0;
        }
        if (attn_rows_ok(d, k, m, 1, 0) != CSA_OK) return 0;
        // proxies change the row count; size for the larger of the two plans
        const size_t a = csa::plan_attention(d, k, m, 1, 0).ws_bytes;
        const size_t b = (k > 0 || m > 0) ? csa::plan_attention(d, k, m, 0, 0).ws_bytes : 0;
        return a > b ? a : b;
    }
    case CSA_WS_DENSE_DECODE_ATTN:
        if (attn_rows_ok(d, 0, 0, 0, 1) != CSA_OK) return 0;
        return csa::plan_attention(d, 0, 0, 0, 1).ws_bytes;
    case CSA_WS_SELECTIVE_DECODE_STEP: {
        if (k < 0 || m < 0) {
            fail(CSA_ERR_INVALID_ARG, "csa_workspace_size: k=%d or m=%d out of range", k, m);
            return 0;
        }
        const int kk = k < d.nb ? k : d.nb;
        if (attn_rows_ok(d, kk, m, 1, 0) != CSA_OK) return 0;
        return step_ws(d, kk, m).total;
    }
    }
    fail(CSA_ERR_INVALID_ARG, "csa_workspace_size: unknown entry %d", (int)entry);
    return 0;
}

const char* csa_status_str(int status)
{
    switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported";
    case CSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char* csa_last_error(void) { return g_last_error; }

}  // extern "C"

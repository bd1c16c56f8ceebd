// api.hip -- the C-ABI entry points of libcsa: argument validation on the host,
// workspace sizing, and dispatch to the kernel launchers.  Every check runs
// before any HIP call, so invalid calls launch nothing and touch no output.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

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

// The integer a caller passed for a C enum.  Copied byte for byte: a value
// outside the enumerators (which validation then rejects) must not be read
// as the enum type itself, whose range C++ limits to its enumerators' bits.
template <typename E>
int raw_enum(const E& e)
{
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

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
    const int dtype = raw_enum(sh->dtype);
    if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
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
    d->dtype = dtype == CSA_F32 ? csa::DT_F32 : csa::DT_BF16;
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
    if (!aligned256(ws)) return fail(CSA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    return CSA_OK;
}

// ---- optional check of device-resident indices --------------------------------

std::atomic<int> g_index_checks{-1};  // -1: not yet read from the environment

bool index_checks_on()
{
    int v = g_index_checks.load();
    if (v < 0) {
        const char* e = getenv("CSA_CHECK_INDICES");
        v = (e && *e && !(e[0] == '0' && e[1] == 0)) ? 1 : 0;
        int expected = -1;
        g_index_checks.compare_exchange_strong(expected, v);
        v = g_index_checks.load();
    }
    return v == 1;
}

// Copies the caller's index arrays to the host (which waits for the stream's
// earlier work) and rejects what the oracle rejects: a selection row that
// names a block twice or outside [0, nb), a weighted token outside [0, n).
int check_device_indices(const char* where, const csa::Dims& d, const int32_t* sel, int k, const int32_t* tok_idx,
                         int m, hipStream_t st)
{
    const size_t rows = (size_t)d.pairs();
    if (k > 0) {
        std::vector<int32_t> h(rows * (size_t)k);
        hipError_t e = hipMemcpyAsync(h.data(), sel, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "index check (sel)");
        std::vector<int32_t> row((size_t)k);
        for (size_t r = 0; r < rows; ++r) {
            for (int i = 0; i < k; ++i) {
                const int32_t b = h[r * k + i];
                if (b < 0 || b >= d.nb)
                    return fail(CSA_ERR_INVALID_ARG, "%s: sel[%zu][%d] = %d outside [0, %d)", where, r, i, b, d.nb);
                row[i] = b;
            }
            std::sort(row.begin(), row.end());
            for (int i = 1; i < k; ++i)
                if (row[i] == row[i - 1])
                    return fail(CSA_ERR_INVALID_ARG, "%s: sel row %zu names block %d twice", where, r, row[i]);
        }
    }
    if (m > 0) {
        std::vector<int32_t> h(rows * (size_t)m);
        hipError_t e = hipMemcpyAsync(h.data(), tok_idx, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e, "index check (tok_idx)");
        for (size_t r = 0; r < rows; ++r)
            for (int i = 0; i < m; ++i) {
                const int32_t t = h[r * m + i];
                if (t < 0 || t >= d.n)
                    return fail(CSA_ERR_INVALID_ARG, "%s: tok_idx[%zu][%d] = %d outside [0, %d)", where, r, i, t, d.n);
            }
    }
    return CSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Block-score workspace (G > 1): per-head logits [B, Hq, nb], then the per-tile
// log-sum-exp states of the split kernels.
size_t block_logits_bytes(const csa::Dims& d) { return (size_t)d.B * d.Hq * d.nb * sizeof(float); }

size_t block_score_ws(const csa::Dims& d)
{
    return d.G > 1 ? align256(block_logits_bytes(d)) + csa::score_err_parts_bytes(d) : 0;
}

float* score_parts(const csa::Dims& d, void* ws)
{
    return d.G > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + align256(block_logits_bytes(d))) : nullptr;
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

// Proxy-error scores: the log-errors, then the per-tile normaliser states.
size_t error_score_ws(const csa::Dims& d) { return block_score_ws(d); }

// Workspace layout of the unfused decode step: scores | sel | block_score ws | attention ws.
struct StepWs {
    size_t scores, sel, score_ws, attn_ws, cand, total;
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
    // chunk candidates (score and index) of the split route beyond kLseFromLogitsMaxBlocks blocks
    w.cand = d.nb > csa::kLseFromLogitsMaxBlocks && kk > 0
                 ? align256((size_t)d.pairs() * ((d.nb + csa::kCandChunk - 1) / csa::kCandChunk) * kk * 8)
                 : 0;
    w.total = w.scores + w.sel + w.score_ws + w.attn_ws + w.cand;
    return w;
}

// ---- query-guided clusters ---------------------------------------------------

// The cluster shape: clusters take the place of blocks.
csa::Dims cluster_dims(const csa::Dims& d, int C)
{
    csa::Dims dc = d;
    dc.nb = C;
    return dc;
}

// Workspace of cluster_decode_step: scores | sel | per-head logits.
struct ClusterStepWs {
    size_t scores, sel, logits, total;
};

ClusterStepWs cluster_step_ws(const csa::Dims& d, int C, int k)
{
    ClusterStepWs w{};
    const csa::Dims dc = cluster_dims(d, C);
    w.scores = align256((size_t)d.pairs() * C * sizeof(float));
    w.sel = align256((size_t)d.pairs() * (k > 0 ? k : 1) * sizeof(int32_t));
    w.logits = align256(block_score_ws(dc));
    w.total = w.scores + w.sel + w.logits;
    return w;
}

// Cluster scores (and, when k > 0, the top-k to sel).  bfloat16 with G <= 8 and
// G C <= 16384: the matrix-core summary-score kernels with count terms from the
// ranges -- one workgroup per KV head (selecting too when k <= 32 and C <= 2048)
// with 32 or more KV heads, else logits split over tiles; otherwise a scalar
// logit kernel and the group score.  logits: block_score_ws() bytes of scratch
// (G > 1): the logits [B, Hq, C], then the tiles' log-sum-exp states.
hipError_t cluster_scores(const csa::Dims& d, int C, const void* q, const void* Kc, const int32_t* offsets,
                          float* scores, int32_t* sel, int k, float* logits, hipStream_t st)
{
    const csa::Dims dc = cluster_dims(d, C);
    hipError_t e;
    bool selected = false;
    if (csa::fused_summary_score_ok(dc)) {
        selected = k > 0 && csa::split_select_ok(dc, k);
        if (d.pairs() >= csa::kFusedStepMinPairs)
            e = csa::launch_score_summary_fused(dc, q, Kc, scores, st, false, offsets, selected ? sel : nullptr,
                                                selected ? k : 0);
        else
            e = csa::launch_score_summary_split(dc, q, Kc, d.G == 1 ? scores : logits, scores,
                                                selected ? sel : nullptr, selected ? k : 0, st, false, offsets,
                                                score_parts(dc, logits));
    } else {
        float* lg = d.G == 1 ? scores : logits;
        e = csa::launch_cluster_logits(d, C, q, Kc, offsets, lg, st);
        if (e == hipSuccess && d.G > 1)
            e = csa::score_finish_ok(dc) ? csa::launch_score_finish(dc, lg, scores, nullptr, 0, st)
                                         : csa::launch_group_score(dc, lg, scores, st);
    }
    if (e == hipSuccess && k > 0 && !selected) e = csa::launch_topk(d.pairs(), C, k, scores, sel, st);
    return e;
}

// ---- the static scratch of selective_decode_step_noalloc ---------------------

constexpr size_t kScratchBytes = (size_t)CSA_STEP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each GPU, set on first use

}  // namespace

// Scratch of the allocation-free decode step: one copy per GPU, held by the
// loaded code object until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress (scratch_of_current_device) and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[CSA_STEP_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of the current GPU's scratch, looked up once per GPU with that
// GPU current.
int scratch_of_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "selective_decode_step_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(CSA_ERR_UNSUPPORTED, "selective_decode_step_noalloc: device %d (at most %d devices)", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "selective_decode_step_noalloc: hipGetSymbolAddress");
        if (!p || !aligned256(p))
            return fail(CSA_ERR_HIP, "selective_decode_step_noalloc: scratch address %p is not 256-byte aligned", p);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA_OK;
}

// The decode step.  get_ws(need, &ws, &ws_bytes) supplies the workspace of the
// three-kernel route once the arguments are valid (need > 0 only there).
template <typename GetWs>
int step_impl(const csa_shape* shape, int mode, const void* q, const void* K, const void* V, const void* Kbar,
              const void* Vbar, int32_t k, const int32_t* tok_idx, const float* tok_logw, int32_t m, int proxy_mode,
              float* scores, int32_t* sel, float* out, float* lse, GetWs get_ws, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (mode == CSA_SCORE_BOX || mode == CSA_SCORE_COBS2 || mode == CSA_SCORE_PROXY_ERROR ||
        mode == CSA_SCORE_COBS2_FP4)
        return fail(CSA_ERR_UNSUPPORTED, "selective_decode_step: box, second-order and proxy-error scores need "
                                         "Kbox, Kcov or Kvar; call block_score, topk_select and sparse_decode_attn");
    if (mode != CSA_SCORE_SUMMARY && mode != CSA_SCORE_EXACT_MASS)
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: unknown mode %d", mode);
    if (proxy_mode != CSA_PROXY_NONE && proxy_mode != CSA_PROXY_COMPLEMENT)
        return fail(CSA_ERR_INVALID_ARG, "selective_decode_step: unknown proxy mode %d", proxy_mode);
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
    if (index_checks_on())
        if (int rc = check_device_indices("selective_decode_step", d, nullptr, 0, tok_idx, m, stream)) return rc;

    if (mode == CSA_SCORE_SUMMARY && csa::fused_step_ok(d, kk, m, proxies)) {
        void* none = nullptr;
        size_t none_bytes = 0;
        if (int rc = get_ws(0, &none, &none_bytes)) return rc;
        csa::StepInputs in{q, K, V, Kbar, Vbar, kk, tok_idx, tok_logw, m, proxies, scores, sel, out, lse};
        const hipError_t e = csa::launch_decode_step(d, in, stream);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "selective_decode_step");
    }
    // the three kernels in turn; scores and selection go to the caller's arrays
    // when given, else to the workspace
    const StepWs w = step_ws(d, kk, m);
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (int rc = get_ws(w.total, &ws, &ws_bytes)) return rc;
    if (int rc = check_ws(w.total, ws, ws_bytes)) return rc;
    char* base = static_cast<char*>(ws);
    float* sc = scores ? scores : reinterpret_cast<float*>(base);
    int32_t* sl = sel ? sel : reinterpret_cast<int32_t*>(base + w.scores);
    void* sws = base + w.scores + w.sel;
    void* aws = base + w.scores + w.sel + w.score_ws;
    if (mode == CSA_SCORE_SUMMARY && csa::fused_summary_score_ok(d) && d.pairs() < csa::kFusedStepMinPairs &&
        csa::split_select_ok(d, kk) && d.nb > csa::kLseFromLogitsMaxBlocks && kk > 0 &&
        csa::plan_attention(d, kk, m, proxies, 0).direct) {
        // split logits with their tiles' log-sum-exp states, group scores and each
        // chunk's top-k candidates, then the attention kernel ranks the candidates
        float* lg = d.G == 1 ? sc : static_cast<float*>(sws);
        float* parts = score_parts(d, sws);
        float* cand_score = reinterpret_cast<float*>(base + w.scores + w.sel + w.score_ws + w.attn_ws);
        const int nchunks = (d.nb + csa::kCandChunk - 1) / csa::kCandChunk;
        int32_t* cand_idx = reinterpret_cast<int32_t*>(cand_score + (size_t)d.pairs() * nchunks * kk);
        const int last = d.nb - (nchunks - 1) * csa::kCandChunk;
        const int ncand = (nchunks - 1) * kk + (last < kk ? last : kk);
        hipError_t e = csa::launch_score_summary_split(d, q, Kbar, lg, sc, nullptr, -1, stream, false, nullptr, parts);
        if (e == hipSuccess) e = csa::launch_score_group_chunks(d, lg, parts, sc, kk, cand_score, cand_idx, stream);
        if (e != hipSuccess) return hip_fail(e, "selective_decode_step (score)");
        const csa::AttnPlan plan = csa::plan_attention(d, kk, m, proxies, 0);
        if (int rc = check_ws(plan.ws_bytes, aws, w.attn_ws)) return rc;
        csa::AttnInputs in{q, K, V, Kbar, Vbar, nullptr, kk, tok_idx, tok_logw, m, proxies, 0, out, lse};
        in.cand_score = cand_score;
        in.cand_idx = cand_idx;
        in.ncand = ncand;
        in.sel_out = sel;
        in.plog = lg;
        e = csa::launch_attention(d, plan, in, aws, stream);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "selective_decode_step");
    }
    if (mode == CSA_SCORE_SUMMARY && csa::fused_summary_score_ok(d) && d.pairs() < csa::kFusedStepMinPairs &&
        csa::split_select_ok(d, kk)) {
        // scores and selection from the split kernels (the top-k rides on the group-score kernel)
        const hipError_t e = csa::launch_score_summary_split(d, q, Kbar, d.G == 1 ? sc : static_cast<float*>(sws),
                                                             sc, sl, kk, stream, false, nullptr, score_parts(d, sws));
        if (e != hipSuccess) return hip_fail(e, "selective_decode_step (score)");
    } else if (mode == CSA_SCORE_EXACT_MASS && d.G > 1 && csa::score_finish_ok(d) && csa::split_select_ok(d, kk)) {
        // exact masses, then group scores and selection in one kernel
        float* lg = static_cast<float*>(sws);
        hipError_t e = csa::launch_block_logits_exact(d, q, K, lg, stream);
        if (e == hipSuccess) e = csa::launch_score_finish(d, lg, sc, sl, kk, stream);
        if (e != hipSuccess) return hip_fail(e, "selective_decode_step (score)");
    } else {
        if (int rc = block_score(shape, static_cast<csa_score_mode>(mode), q, mode == CSA_SCORE_SUMMARY ? Kbar : K, sc,
                                 sws, w.score_ws, stream))
            return rc;
        if (int rc = topk_select(d.pairs(), d.nb, kk, sc, sl, stream)) return rc;
    }
    return sparse_decode_attn(shape, q, K, V, Kbar, Vbar, kk > 0 ? sl : nullptr, kk, tok_idx, tok_logw, m,
                              static_cast<csa_proxy_mode>(proxy_mode), out, lse, aws, w.attn_ws, stream);
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

namespace {

int cov_sub_build_impl(const char* where, bool fp4, const csa_shape* shape, int32_t s_dim, const void* K,
                       const float* U, void* Kcs, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!K || !U || !Kcs) return fail(CSA_ERR_INVALID_ARG, "%s: NULL pointer", where);
    if (!aligned16(K) || !aligned16(Kcs) || !aligned4(U)) return fail(CSA_ERR_INVALID_ARG, "%s: misaligned pointer", where);
    if (s_dim < 1 || s_dim > d.d) return fail(CSA_ERR_INVALID_ARG, "%s: s=%d outside [1, d=%d]", where, s_dim, d.d);
    if (fp4 && d.dtype != csa::DT_BF16)
        return fail(CSA_ERR_UNSUPPORTED, "%s: FP4 descriptors need a bfloat16 cache", where);
    if (!csa::cov_sub_ok(d, s_dim))
        return fail(CSA_ERR_UNSUPPORTED, "%s: blocks of %d tokens (at most 64) or s=%d above 128", where, d.L, s_dim);
    const hipError_t e = fp4 ? csa::launch_cov_sub4(d, s_dim, K, U, Kcs, stream)
                             : csa::launch_cov_sub(d, s_dim, K, U, Kcs, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, where);
}

int score_sub_impl(const char* where, bool fp4, const csa_shape* shape, int32_t s_dim, const void* q, const void* Kcs,
                   const float* U, float* scores, void* ws, size_t ws_bytes, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (!q || !Kcs || !U || !scores) return fail(CSA_ERR_INVALID_ARG, "%s: NULL pointer", where);
    if (!aligned16(q) || !aligned16(Kcs) || !aligned4(U) || !aligned4(scores))
        return fail(CSA_ERR_INVALID_ARG, "%s: misaligned pointer", where);
    if (s_dim < 1 || s_dim > d.d) return fail(CSA_ERR_INVALID_ARG, "%s: s=%d outside [1, d=%d]", where, s_dim, d.d);
    if (d.dtype != csa::DT_BF16 || d.G > 8) return fail(CSA_ERR_UNSUPPORTED, "%s: needs bfloat16 and G <= 8", where);
    {
        const long long bb = fp4 ? (long long)CSA_COV_SUB4_BLOCK_BYTES(d.d, s_dim)
                                 : 2ll * CSA_COV_SUB_BLOCK_ELEMS((long long)d.d, (long long)s_dim);
        if ((long long)d.nb * bb >= (1ll << 32))
            return fail(CSA_ERR_UNSUPPORTED, "%s: one KV head's descriptors must be below 4 GiB", where);
    }
    if (int rc = check_ws(block_score_ws(d), ws, ws_bytes)) return rc;
    const hipError_t e = csa::launch_score_cobs2_sub(d, s_dim, q, Kcs, U, d.G == 1 ? scores : static_cast<float*>(ws),
                                                     scores, stream, fp4);
    return e == hipSuccess ? CSA_OK : hip_fail(e, where);
}

}  // namespace

int kv_cov_sub_build(const csa_shape* shape, int32_t s_dim, const void* K, const float* U, void* Kcs,
                     hipStream_t stream)
{
    return cov_sub_build_impl("kv_cov_sub_build", false, shape, s_dim, K, U, Kcs, stream);
}

int kv_cov_sub4_build(const csa_shape* shape, int32_t s_dim, const void* K, const float* U, void* Kcs4,
                      hipStream_t stream)
{
    return cov_sub_build_impl("kv_cov_sub4_build", true, shape, s_dim, K, U, Kcs4, stream);
}

int block_score_cobs2_sub(const csa_shape* shape, int32_t s_dim, const void* q, const void* Kcs, const float* U,
                          float* scores, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return score_sub_impl("block_score_cobs2_sub", false, shape, s_dim, q, Kcs, U, scores, ws, ws_bytes, stream);
}

int block_score_cobs2_sub4(const csa_shape* shape, int32_t s_dim, const void* q, const void* Kcs4, const float* U,
                           float* scores, void* ws, size_t ws_bytes, hipStream_t stream)
{
    return score_sub_impl("block_score_cobs2_sub4", true, shape, s_dim, q, Kcs4, U, scores, ws, ws_bytes, stream);
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

int block_score(const csa_shape* shape, csa_score_mode mode_arg, const void* q, const void* keys, float* scores,
                void* ws, size_t ws_bytes, hipStream_t stream)
{
    const int mode = raw_enum(mode_arg);
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (mode != CSA_SCORE_SUMMARY && mode != CSA_SCORE_EXACT_MASS && mode != CSA_SCORE_BOX && mode != CSA_SCORE_COBS2 &&
        mode != CSA_SCORE_PROXY_ERROR && mode != CSA_SCORE_COBS2_FP4)
        return fail(CSA_ERR_INVALID_ARG, "block_score: unknown mode %d", mode);
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
        float* parts = score_parts(d, ws);
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
                                                  nullptr, 0, stream, box, nullptr, score_parts(d, ws));
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
                       const float* tok_logw, int32_t m, csa_proxy_mode proxy_arg, float* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream)
{
    const int proxy_mode = raw_enum(proxy_arg);
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (proxy_mode != CSA_PROXY_NONE && proxy_mode != CSA_PROXY_COMPLEMENT)
        return fail(CSA_ERR_INVALID_ARG, "sparse_decode_attn: unknown proxy mode %d", proxy_mode);
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
    if (index_checks_on())
        if (int rc = check_device_indices("sparse_decode_attn", d, sel, k, tok_idx, m, stream)) return rc;
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
    auto caller_ws = [&](size_t, void** p, size_t* n) {
        *p = ws;
        *n = ws_bytes;
        return (int)CSA_OK;
    };
    return step_impl(shape, raw_enum(mode), q, K, V, Kbar, Vbar, k, tok_idx, tok_logw, m, raw_enum(proxy_mode), scores,
                     sel, out, lse, caller_ws, stream);
}

int selective_decode_step_noalloc(const csa_shape* shape, csa_score_mode mode, const void* q, const void* K,
                                  const void* V, const void* Kbar, const void* Vbar, int32_t k,
                                  const int32_t* tok_idx, const float* tok_logw, int32_t m,
                                  csa_proxy_mode proxy_mode, float* scores, int32_t* sel, float* out, float* lse,
                                  hipStream_t stream)
{
    auto static_ws = [&](size_t need, void** p, size_t* n) {
        if (need > kScratchBytes)
            return fail(CSA_ERR_WORKSPACE,
                        "selective_decode_step_noalloc: this shape needs %zu bytes of scratch, above the %zu of the "
                        "static buffer (use selective_decode_step with a workspace)",
                        need, kScratchBytes);
        if (int rc = scratch_of_current_device(p)) return rc;
        *n = kScratchBytes;
        return (int)CSA_OK;
    };
    return step_impl(shape, raw_enum(mode), q, K, V, Kbar, Vbar, k, tok_idx, tok_logw, m, raw_enum(proxy_mode), scores,
                     sel, out, lse, static_ws, stream);
}

int kv_cluster_build(const csa_shape* shape, int32_t n_clusters, int32_t rank, int32_t iters, const void* K,
                     const void* V, const float* U, const int32_t* seeds, int32_t* assign, int32_t* order,
                     int32_t* offsets, void* Kg, void* Vg, void* Kc, void* Vc, void* ws, size_t ws_bytes,
                     hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (iters < 0) return fail(CSA_ERR_INVALID_ARG, "kv_cluster_build: iters=%d is negative", iters);
    if (n_clusters < 1 || rank < 1)
        return fail(CSA_ERR_INVALID_ARG, "kv_cluster_build: n_clusters=%d rank=%d", n_clusters, rank);
    if (!csa::cluster_build_ok(n_clusters, rank))
        return fail(CSA_ERR_UNSUPPORTED,
                    "kv_cluster_build: n_clusters=%d rank=%d (rank in {4, 8, 16, 32}, n_clusters <= %d, "
                    "n_clusters * rank <= %zu)",
                    n_clusters, rank, csa::kClusterMaxClusters, csa::kClusterCentroidLds / sizeof(double));
    if (!K || !V || !U || !seeds || !assign || !order || !offsets || !Kg || !Vg || !Kc || !Vc)
        return fail(CSA_ERR_INVALID_ARG, "kv_cluster_build: NULL pointer");
    if (!aligned16(K) || !aligned16(V) || !aligned16(Kg) || !aligned16(Vg) || !aligned16(Kc) || !aligned16(Vc) ||
        !aligned4(U) || !aligned4(seeds) || !aligned4(assign) || !aligned4(order) || !aligned4(offsets))
        return fail(CSA_ERR_INVALID_ARG, "kv_cluster_build: misaligned pointer");
    if (int rc = check_ws(csa::cluster_build_ws_bytes(d, n_clusters, rank), ws, ws_bytes)) return rc;
    if (index_checks_on())
        if (int rc = check_device_indices("kv_cluster_build (seeds)", d, nullptr, 0, seeds, n_clusters, stream))
            return rc;
    csa::ClusterBuild cb{};
    cb.K = K;
    cb.V = V;
    cb.U = U;
    cb.seeds = seeds;
    cb.C = n_clusters;
    cb.r = rank;
    cb.iters = iters;
    cb.assign = assign;
    cb.order = order;
    cb.offsets = offsets;
    cb.Kg = Kg;
    cb.Vg = Vg;
    cb.Kc = Kc;
    cb.Vc = Vc;
    cb.proj = static_cast<double*>(ws);
    cb.cent = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                        align256((size_t)d.pairs() * d.n * rank * sizeof(double)));
    const hipError_t e = csa::launch_cluster_build(d, cb, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "kv_cluster_build");
}

int cluster_score(const csa_shape* shape, int32_t n_clusters, const void* q, const void* Kc,
                  const int32_t* offsets, float* scores, void* ws, size_t ws_bytes, hipStream_t stream)
{
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (n_clusters < 1) return fail(CSA_ERR_INVALID_ARG, "cluster_score: n_clusters=%d", n_clusters);
    if (!q || !Kc || !offsets || !scores) return fail(CSA_ERR_INVALID_ARG, "cluster_score: NULL pointer");
    if (!aligned16(q) || !aligned16(Kc) || !aligned4(offsets) || !aligned4(scores))
        return fail(CSA_ERR_INVALID_ARG, "cluster_score: misaligned pointer");
    if (n_clusters > csa::kClusterMaxClusters)
        return fail(CSA_ERR_UNSUPPORTED, "cluster_score: n_clusters=%d above %d", n_clusters, csa::kClusterMaxClusters);
    if ((long long)n_clusters * d.d * (d.dtype == csa::DT_F32 ? 4 : 2) >= (1ll << 32))
        return fail(CSA_ERR_UNSUPPORTED, "cluster_score: one KV head's mean keys must be below 4 GiB");
    if (int rc = check_ws(block_score_ws(cluster_dims(d, n_clusters)), ws, ws_bytes)) return rc;
    const hipError_t e = cluster_scores(d, n_clusters, q, Kc, offsets, scores, nullptr, 0, static_cast<float*>(ws),
                                        stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "cluster_score");
}

// Arguments of the cluster attention shared by cluster_decode_attn and
// cluster_decode_step (sel is checked by the caller).
int check_cluster_attn(const char* where, const csa::Dims& d, int n_clusters, int k, int proxy_mode, const void* q,
                       const void* Kg, const void* Vg, const void* Kc, const void* Vc, const int32_t* offsets,
                       const float* out, const float* lse)
{
    if (proxy_mode != CSA_PROXY_NONE && proxy_mode != CSA_PROXY_COMPLEMENT)
        return fail(CSA_ERR_INVALID_ARG, "%s: unknown proxy mode %d", where, proxy_mode);
    const int proxies = proxy_mode == CSA_PROXY_COMPLEMENT;
    if (n_clusters < 1 || n_clusters > csa::kClusterMaxClusters)
        return fail(n_clusters < 1 ? CSA_ERR_INVALID_ARG : CSA_ERR_UNSUPPORTED, "%s: n_clusters=%d (1 .. %d)", where,
                    n_clusters, csa::kClusterMaxClusters);
    if (k < 0 || k > n_clusters) return fail(CSA_ERR_INVALID_ARG, "%s: k=%d outside [0, %d]", where, k, n_clusters);
    if (k > csa::kClusterMaxSel) return fail(CSA_ERR_UNSUPPORTED, "%s: k=%d above %d", where, k, csa::kClusterMaxSel);
    if (k == 0 && !proxies)
        return fail(CSA_ERR_INVALID_ARG, "%s: empty virtual-token set (k = 0, no proxies)", where);
    if (d.dtype != csa::DT_BF16) return fail(CSA_ERR_UNSUPPORTED, "%s: bfloat16 caches only", where);
    if (d.G > 8) return fail(CSA_ERR_UNSUPPORTED, "%s: group size %d above 8", where, d.G);
    if ((long long)d.n * d.d * 2 >= (1ll << 32))
        return fail(CSA_ERR_UNSUPPORTED, "%s: one KV head's cache must be below 4 GiB", where);
    if (!q || !Kg || !Vg || !offsets || !out || (proxies && (!Kc || !Vc)))
        return fail(CSA_ERR_INVALID_ARG, "%s: NULL pointer", where);
    if (!aligned16(q) || !aligned16(Kg) || !aligned16(Vg) || (proxies && (!aligned16(Kc) || !aligned16(Vc))) ||
        !aligned4(offsets) || !aligned4(out) || (lse && !aligned4(lse)))
        return fail(CSA_ERR_INVALID_ARG, "%s: misaligned pointer", where);
    return CSA_OK;
}

int cluster_decode_attn(const csa_shape* shape, int32_t n_clusters, const void* q, const void* Kg, const void* Vg,
                        const void* Kc, const void* Vc, const int32_t* offsets, const int32_t* sel, int32_t k,
                        csa_proxy_mode proxy_arg, float* out, float* lse, hipStream_t stream)
{
    const int proxy_mode = raw_enum(proxy_arg);
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (int rc = check_cluster_attn("cluster_decode_attn", d, n_clusters, k, proxy_mode, q, Kg, Vg, Kc, Vc, offsets,
                                    out, lse))
        return rc;
    const int proxies = proxy_mode == CSA_PROXY_COMPLEMENT;
    if (k > 0 && !sel) return fail(CSA_ERR_INVALID_ARG, "cluster_decode_attn: NULL pointer");
    if (sel && !aligned4(sel)) return fail(CSA_ERR_INVALID_ARG, "cluster_decode_attn: misaligned pointer");
    if (index_checks_on()) {
        csa::Dims dc = d;
        dc.nb = n_clusters;
        if (int rc = check_device_indices("cluster_decode_attn", dc, sel, k, nullptr, 0, stream)) return rc;
    }
    csa::ClusterAttn ca{q, Kg, Vg, proxies ? Kc : Kg, proxies ? Vc : Vg, offsets, sel, n_clusters, k, proxies, out, lse};
    const hipError_t e = csa::launch_cluster_attention(d, ca, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "cluster_decode_attn");
}

int cluster_decode_step(const csa_shape* shape, int32_t n_clusters, const void* q, const void* Kg, const void* Vg,
                        const void* Kc, const void* Vc, const int32_t* offsets, int32_t k, csa_proxy_mode proxy_arg,
                        float* scores, int32_t* sel, float* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream)
{
    const int proxy_mode = raw_enum(proxy_arg);
    csa::Dims d;
    if (int rc = make_dims(shape, &d)) return rc;
    if (k < 0) return fail(CSA_ERR_INVALID_ARG, "cluster_decode_step: k=%d is negative", k);
    const int kk = n_clusters >= 1 && k > n_clusters ? n_clusters : k;
    if (int rc = check_cluster_attn("cluster_decode_step", d, n_clusters, kk, proxy_mode, q, Kg, Vg, Kc, Vc, offsets,
                                    out, lse))
        return rc;
    if (!Kc) return fail(CSA_ERR_INVALID_ARG, "cluster_decode_step: Kc is NULL (it ranks the clusters)");
    if (!aligned16(Kc) || (scores && !aligned4(scores)) || (sel && !aligned4(sel)))
        return fail(CSA_ERR_INVALID_ARG, "cluster_decode_step: misaligned pointer");
    const ClusterStepWs w = cluster_step_ws(d, n_clusters, kk);
    if (int rc = check_ws(w.total, ws, ws_bytes)) return rc;
    const int proxies = proxy_mode == CSA_PROXY_COMPLEMENT;
    const csa::Dims dc = cluster_dims(d, n_clusters);
    if (csa::cluster_step_ok(dc, kk)) {  // one kernel per KV head; the workspace stays unused
        const csa::ClusterStepInputs in{q, Kg, Vg, Kc, proxies ? Vc : Vg, offsets, kk, proxies, scores, sel, out, lse};
        const hipError_t e = csa::launch_cluster_step(dc, in, stream);
        return e == hipSuccess ? CSA_OK : hip_fail(e, "cluster_decode_step");
    }
    char* base = static_cast<char*>(ws);
    float* sc = scores ? scores : reinterpret_cast<float*>(base);
    int32_t* sl = sel ? sel : reinterpret_cast<int32_t*>(base + w.scores);
    float* lg = reinterpret_cast<float*>(base + w.scores + w.sel);
    hipError_t e = cluster_scores(d, n_clusters, q, Kc, offsets, sc, sl, kk, lg, stream);
    if (e != hipSuccess) return hip_fail(e, "cluster_decode_step (scores)");
    csa::ClusterAttn ca{q, Kg, Vg, proxies ? Kc : Kg, proxies ? Vc : Vg, offsets, sl, n_clusters, kk, proxies, out, lse};
    e = csa::launch_cluster_attention(d, ca, stream);
    return e == hipSuccess ? CSA_OK : hip_fail(e, "cluster_decode_step");
}

size_t csa_workspace_size(const csa_shape* shape, csa_entry entry_arg, int32_t k, int32_t m)
{
    const int entry = raw_enum(entry_arg);
    csa::Dims d;
    if (make_dims(shape, &d) != CSA_OK) return 0;
    switch (entry) {
    case CSA_WS_BLOCK_SCORE_SUMMARY:
    case CSA_WS_BLOCK_SCORE_EXACT_MASS:
    case CSA_WS_BLOCK_SCORE_BOX:
    case CSA_WS_BLOCK_SCORE_COBS2:
    case CSA_WS_BLOCK_SCORE_COBS2_FP4:
    case CSA_WS_BLOCK_SCORE_COBS2_SUB: return block_score_ws(d);
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
    case CSA_WS_KV_CLUSTER_BUILD:
        if (!csa::cluster_build_ok(k, m)) {
            fail(CSA_ERR_UNSUPPORTED, "csa_workspace_size: n_clusters=%d rank=%d unsupported", k, m);
            return 0;
        }
        return csa::cluster_build_ws_bytes(d, k, m);
    case CSA_WS_CLUSTER_SCORE: {
        if (k < 1) {
            fail(CSA_ERR_INVALID_ARG, "csa_workspace_size: n_clusters=%d", k);
            return 0;
        }
        return block_score_ws(cluster_dims(d, k));
    }
    case CSA_WS_CLUSTER_DECODE_STEP:
        if (m < 1 || k < 0) {
            fail(CSA_ERR_INVALID_ARG, "csa_workspace_size: n_clusters=%d (passed as m) or k=%d out of range", m, k);
            return 0;
        }
        return cluster_step_ws(d, m, k < m ? k : m).total;
    }
    fail(CSA_ERR_INVALID_ARG, "csa_workspace_size: unknown entry %d", entry);
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

int csa_set_index_checks(int enable)
{
    const int prev = index_checks_on() ? 1 : 0;
    g_index_checks.store(enable ? 1 : 0);
    return prev;
}

}  // extern "C"

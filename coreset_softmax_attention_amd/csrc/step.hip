// step.hip -- the whole selective decode step of one KV head in one workgroup:
// block score (summary mode) -> top-k -> attention over exact tokens, weighted
// tokens and count-aware proxies.
//
// The first-order block logit of "COBS: Cumulant Order Block Sparse Attention",
// Eq. (18) (scale q . mean key + ln c_b) is also exactly the logit of the
// count-aware proxy of "OpenAttention reads 1% of the KV cache -- Count-aware
// tail proxy" (section "Skipping reviews without losing the verdict"): the mean
// logit of the block plus ln(count).  So the mean keys are read once: the
// logits of all blocks and heads stay in LDS, rank the blocks (Eq. (5), log
// domain) and then serve as the proxy logits; the proxy rows of the attention
// load only their mean values.
//
// Phases of a workgroup (KV head (b, j), all G <= 8 query heads of the group):
//   1. waves stream the mean keys in tiles of 32 rows; MFMA logits -> LDS;
//   2. per-head log-normaliser; group scores (written out if asked), one or
//      four blocks per thread; top-k (up to 512 blocks) from a bound on the
//      k-th largest score (the k-th largest of the waves' maxima) and the few
//      blocks that reach it, else by one wave over all scores; selection
//      (written out if asked), bitmap of selected blocks;
//   3. attention tiles: proxy rows (values only, logits from LDS, selected
//      blocks masked), weighted rows, exact rows of the selected blocks (keys
//      and values, MFMA logits), in the engine of attn_engine.hpp.
#include <type_traits>

#include "attn_engine.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kStepWaves = 8;
constexpr int kStepMaxK = 32;
constexpr int kStepMaxBlocks = 2048;     // top-k by one wave: up to 32 scores per lane
constexpr int kStepMaxLdsBytes = 65536;  // dynamic LDS: logits, scores, bitmap

struct StepParams {
    const char* q;
    const char* K;
    const char* V;
    const char* Kbar;
    const char* Vbar;
    const int32_t* tok_idx;
    const float* tok_logw;
    float* scores;  // optional
    int32_t* sel;   // optional
    float* out;
    float* lse;     // optional
    int Hq, Hkv, G, n, L, nb, k, m, proxies;
    int pend, wbeg, ebeg, rows;  // attention row layout: [proxies][weighted][exact]
    int lstride;                 // LDS row stride of the logits (nb rounded up to 32)
    float scale, ln_L, ln_last, scale_log2;
};

template <int D, int HG>
__global__ void __launch_bounds__(kStepWaves * 64) decode_step_kernel(const StepParams p)
{
    constexpr int NW = kStepWaves, TR = kTileRows;
    using E = MfmaEngine<D, HG, NW>;
    constexpr int RB = E::RB, KS = E::KS;
    extern __shared__ float dyn[];
    __shared__ typename E::Smem sm;
    __shared__ float lse_h[8];
    __shared__ int32_t sel_sm[kStepMaxK];
    __shared__ uint32_t cand_sm[128];          // top-k candidates of the one-wave ranking
    __shared__ __attribute__((aligned(16))) uint32_t topk_sm[2 * NW + 128];  // wave maxima, counts, candidates

    const int LS = p.lstride, G = p.G, nb = p.nb;
    float* lsm = dyn;                                              // [G][LS] block logits (natural log)
    float* ssm = dyn + G * LS;                                     // [LS] group scores
    uint32_t* bits = reinterpret_cast<uint32_t*>(ssm + LS);        // [LS / 32] selected blocks
    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int h0 = j * G;

    E eng(sm, p.q + (size_t)(b * p.Hq + h0) * RB, G);
    const int lane = eng.lane, wave = eng.wave, n16 = eng.n16, g16 = eng.g16;
    for (int w = threadIdx.x; w < LS / 32; w += NW * 64) bits[w] = 0;

    // Loads are issued unconditionally: a tile that does not exist reads
    // through an empty buffer (zeros, no memory traffic).  With loops that
    // have no exit between their halves, this lets the compiler's wait before
    // a tile's use cover that tile's loads only.  The buffers are built from
    // wave-uniform base addresses and sizes.
    const char* const kc = p.K + (size_t)pair * p.n * RB;
    const char* const vc = p.V + (size_t)pair * p.n * RB;
    const char* const ks = p.Kbar + (size_t)pair * nb * RB;
    const char* const vs = p.proxies ? p.Vbar + (size_t)pair * nb * RB : p.V;
    const uint32_t cbytes = (uint32_t)p.n * RB, sbytes = (uint32_t)nb * RB;
    auto size = [](bool live, uint32_t bytes) {  // uniform: keeps the buffer in scalar registers
        return (uint32_t)__builtin_amdgcn_readfirstlane((int)(live ? bytes : 0u));
    };
    auto Kc = [&](bool live) { return buffer_rsrc(kc, size(live, cbytes)); };
    auto Vc = [&](bool live) { return buffer_rsrc(vc, size(live, cbytes)); };
    auto Ks = [&](bool live) { return buffer_rsrc(ks, size(live, sbytes)); };
    auto Vs = [&](bool live) { return buffer_rsrc(vs, size(live && p.proxies, sbytes)); };

    // Tile orders are rotated by a per-workgroup offset, so that workgroups
    // running side by side do not walk the same address offsets at the same
    // time (their heads' arrays start at similarly aligned addresses).
    const uint32_t hsh = (uint32_t)blockIdx.x * 0x9E3779B1u;
    const int nK = (nb + TR - 1) / TR;                                  // mean-key tiles
    const int rotK = (int)((hsh >> 4) % (uint32_t)nK);
    const int nP = p.wbeg / TR;                                          // proxy tiles
    const int nC = p.rows > p.wbeg ? (p.rows - p.wbeg + TR - 1) / TR : 0;  // cache tiles
    const int nT = nP + nC;
    const int rotP = nP ? (int)((hsh >> 8) % (uint32_t)nP) : 0;
    const int rotC = nC ? (int)((hsh >> 16) % (uint32_t)nC) : 0;
    auto row0 = [&](int t) { return t < nP ? (t + rotP) % nP * TR : p.wbeg + (t - nP + rotC) % nC * TR; };
    // this wave's tiles are t = wave + j NW: first Pw proxy tiles, then cache tiles
    const int Pw = wave < nP ? (nP - wave + NW - 1) / NW : 0;
    const int Tw = wave < nT ? (nT - wave + NW - 1) / NW : 0;
    auto tile_of = [&](int jj) { return wave + jj * NW; };

    // Proxy tiles hold only mean values (their logits are the block logits of
    // phase 1) and do not depend on the selection: the wave's first two are
    // loaded now and overlap the scoring phases; their selected blocks are
    // masked once the selection is known.
    uint4 VA[E::NVI], VB[E::NVI];
    auto set_proxy_rows = [&](int tb, int jj, bool masked) {
        if (lane < TR) {
            const int r = row0(tile_of(jj)) + lane;
            float lw = r < p.pend ? 0.0f : kNegInf;  // the logit itself comes from LDS
            if (masked && r < p.pend && ((bits[r >> 5] >> (r & 31)) & 1u)) lw = kNegInf;
            eng.set_row(tb, lane, (uint32_t)(r < p.pend ? r : 0), lw);
        }
    };
    auto issue_first_proxies = [&]() {
        if (Pw > 0) set_proxy_rows(0, 0, false);
        eng.issue_values(VA, 0, Vs(Pw > 0));
        if (Pw > 1) set_proxy_rows(1, 1, false);
        eng.issue_values(VB, 1, Vs(Pw > 1));
    };

    // ---- phase 1: block logits of every head -> LDS ---------------------------
    auto logits_to_lds = [&](int base, const uint4 (&ak)[2][KS]) {
        f32x4_t c[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                c[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ak[rb][s]), eng.bq[s],
                                                                c[rb], 0, 0, 0);
        if (n16 < G) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = base + rb * 16 + 4 * g16 + i;
                    if (row < nb) lsm[n16 * LS + row] = fmaf(c[rb][i], p.scale, row == nb - 1 ? p.ln_last : p.ln_L);
                }
        }
    };
    auto load_keys = [&](int base, uint4 (&ak)[2][KS], bool live) {
        const __amdgpu_buffer_rsrc_t r = Ks(live);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const uint32_t off = (uint32_t)(base + rb * 16 + n16) * RB + g16 * 16;  // past nb: zeros
#pragma unroll
            for (int s = 0; s < KS; ++s) ak[rb][s] = buffer_ld16(r, off + s * 64);
        }
    };
    // The mean keys decide the selection: they have the memory system to
    // themselves.  The wave's first two proxy value tiles go out once its keys
    // have arrived, and stream in while the selection is made.
    for (int t = wave; t < nK; t += 2 * NW) {  // two tiles in flight
        uint4 k0[2][KS], k1[2][KS];
        const int b0 = (t + rotK) % nK * TR, b1 = (t + NW + rotK) % nK * TR;
        const bool two = t + NW < nK;
        load_keys(b0, k0, true);
        load_keys(b1, k1, two);
        logits_to_lds(b0, k0);
        if (two) logits_to_lds(b1, k1);
    }
    issue_first_proxies();
    __syncthreads();

    // ---- phase 2: group score and top-k ----------------------------------------
    if (G > 1) {
        if (wave < G) {
            const float lse = head_lse(lsm + wave * LS, nb, lane);
            if (lane == 0) lse_h[wave] = lse;
        }
        __syncthreads();
    }
    // group scores of blocks threadIdx.x + 64 NW j, ranked by the whole
    // workgroup (one wave-wide maximum per wave, then the few candidates that
    // reach the kk-th largest of them); one wave ranks all scores from LDS when
    // that bound does not apply
    const int kk = p.k;  // <= min(32, nb)
    auto emit = [&](int r, int idx) {
        sel_sm[r] = idx;
        if (p.sel) p.sel[(size_t)pair * kk + r] = idx;
        atomicOr(&bits[idx >> 5], 1u << (idx & 31));
    };
    auto one_wave_topk = [&]() {
        auto load = [&](int i) { return ssm[i]; };
        if (nb <= 8 * 64)
            wave_topk<8>(load, nb, kk, lane, cand_sm, emit);
        else
            wave_topk<kStepMaxBlocks / 64>(load, nb, kk, lane, cand_sm, emit);
    };
    auto score_and_select = [&](auto spt) {
        constexpr int SPT = decltype(spt)::value;
        uint32_t key[SPT];
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            const int i = (int)threadIdx.x + NW * 64 * j;
            key[j] = 0;
            if (i < nb) {
                const float v = G == 1 ? lsm[i] : group_score<HG>(lsm + i, LS, lse_h, G);
                ssm[i] = v;
                key[j] = order_key(v);
                if (p.scores) p.scores[(size_t)pair * nb + i] = v;
            }
        }
        if (kk == 0) return;
        if constexpr (SPT == 1) {
            block_topk<NW, 1>(key, nb, kk, topk_sm, one_wave_topk, emit);
        } else {  // more blocks than threads: one wave over all scores
            __syncthreads();
            if (wave == 0) one_wave_topk();
        }
    };
    static_assert(kStepMaxBlocks == NW * 64 * 4, "scores of up to four blocks per thread");
    if (nb <= NW * 64)
        score_and_select(std::integral_constant<int, 1>{});
    else
        score_and_select(std::integral_constant<int, 4>{});
    __syncthreads();

    // ---- phase 3: attention ------------------------------------------------------
    auto resolve_cache = [&](int r, uint32_t& row, float& lw) {
        row = 0;
        lw = kNegInf;
        if (r >= p.rows) return;
        if (r >= p.wbeg && r < p.wbeg + p.m) {
            const int t = r - p.wbeg;
            const int tok = p.tok_idx[(size_t)pair * p.m + t];
            if (tok >= 0 && tok < p.n) {
                row = (uint32_t)tok;
                lw = p.tok_logw[(size_t)pair * p.m + t] * kLog2e;
            }
        } else if (r >= p.ebeg) {
            const int e = r - p.ebeg;
            const int slot = e / p.L;
            const int tok = sel_sm[slot] * p.L + (e - slot * p.L);
            if (tok < p.n) {
                row = (uint32_t)tok;
                lw = 0.0f;
            }
        }
    };
    auto set_cache_rows = [&](int jj, int tb) {
        if (lane < TR) {
            uint32_t row;
            float lw;
            resolve_cache(row0(tile_of(jj)) + lane, row, lw);
            eng.set_row(tb, lane, row, lw);
        }
    };
    auto issue_cache = [&](int jj, typename E::Tile& t, int tb, bool live) {
        if (live) set_cache_rows(jj, tb);
        eng.issue(t, tb, Kc(live), Vc(live), true);
    };
    auto proxy_tile = [&](int jj, const uint4 (&vr)[E::NVI], int tb) {
        float x[8];
        eng.logits_lds(tb, lsm + (n16 < G ? n16 : G - 1) * LS + row0(tile_of(jj)), x);
        eng.softmax(x);
        eng.accumulate_values(vr);
    };
    auto cache_logits = [&](const typename E::Tile& t, int tb) {
        float x[8];
        eng.logits_mfma(t, tb, p.scale_log2, x);
        eng.softmax(x);
    };

    // The selection is known: mask the selected blocks in the prefetched proxy
    // tiles and finish the proxy tiles (two value tiles in flight), then stream
    // the cache tiles (key and value tiles, one and a half in flight).  Up to
    // four heads, the keys of the wave's first cache tile go out now, so that
    // they stream behind the proxy values instead of after them; its values
    // follow once the proxy tiles are done (the whole first tile now would not
    // fit in registers beside them).  With more heads the keys wait too.
    if (Pw > 0) set_proxy_rows(0, 0, true);
    if (Pw > 1) set_proxy_rows(1, 1, true);
    typename E::Tile CA, CB;
    const bool any_cache = Tw > Pw;
    if constexpr (HG <= 4) {
        if (any_cache) set_cache_rows(Pw, 2);
        eng.issue_keys(CA, 2, Kc(any_cache));
    }
    int jj = 0;
    for (; jj + 1 < Pw; jj += 2) {
        proxy_tile(jj, VA, 0);
        if (jj + 2 < Pw) set_proxy_rows(0, jj + 2, true);
        eng.issue_values(VA, 0, Vs(jj + 2 < Pw));
        proxy_tile(jj + 1, VB, 1);
        if (jj + 3 < Pw) set_proxy_rows(1, jj + 3, true);
        eng.issue_values(VB, 1, Vs(jj + 3 < Pw));
    }
    if (jj < Pw) proxy_tile(jj, VA, 0);  // odd count: the last proxy tile is in VA
    if constexpr (HG <= 4) {
        eng.issue_values(CA.vr, 2, Vc(any_cache));
    } else {
        issue_cache(Pw, CA, 2, any_cache);
    }
    // cache tiles (weighted and exact rows): keys and values; the next tile's
    // loads go out once this tile's keys are consumed (one and a half tiles of
    // registers in flight)
    int jc = Pw;
    for (; jc + 1 < Tw; jc += 2) {
        cache_logits(CA, 2);
        issue_cache(jc + 1, CB, 3, true);
        eng.accumulate(CA);
        cache_logits(CB, 3);
        issue_cache(jc + 2, CA, 2, jc + 2 < Tw);
        eng.accumulate(CB);
    }
    if (jc < Tw) {  // odd count: the last cache tile is in CA
        cache_logits(CA, 2);
        eng.accumulate(CA);
    }
    eng.finish(G, p.out + ((size_t)b * p.Hq + h0) * D, p.lse ? p.lse + (size_t)b * p.Hq + h0 : nullptr, nullptr);
}

size_t step_lds_bytes(const Dims& s)
{
    const int ls = (s.nb + kTileRows - 1) / kTileRows * kTileRows;
    return (size_t)(s.G + 1) * ls * sizeof(float) + (size_t)(ls / 32) * sizeof(uint32_t);
}

template <int D>
hipError_t launch_step_d(const StepParams& p, int pairs, size_t shm, hipStream_t st)
{
    const dim3 grid((unsigned)pairs), block(kStepWaves * 64);
    switch (p.G) {
    case 1: decode_step_kernel<D, 1><<<grid, block, shm, st>>>(p); break;
    case 2: decode_step_kernel<D, 2><<<grid, block, shm, st>>>(p); break;
    case 3: decode_step_kernel<D, 3><<<grid, block, shm, st>>>(p); break;
    case 4: decode_step_kernel<D, 4><<<grid, block, shm, st>>>(p); break;
    case 5: decode_step_kernel<D, 5><<<grid, block, shm, st>>>(p); break;
    case 6: decode_step_kernel<D, 6><<<grid, block, shm, st>>>(p); break;
    case 7: decode_step_kernel<D, 7><<<grid, block, shm, st>>>(p); break;
    case 8: decode_step_kernel<D, 8><<<grid, block, shm, st>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool fused_step_ok(const Dims& s, int k, int m, int proxies)
{
    const long rows = (proxies ? (long)(s.nb - k) : 0L) + (long)k * s.L + m;  // virtual rows per KV head
    const bool enough = s.pairs() >= kFusedStepMinPairs || rows * s.G <= kFusedStepSmallWork;
    return s.dtype == DT_BF16 && s.G <= 8 && k <= kStepMaxK && s.nb <= kStepMaxBlocks && enough &&
           step_lds_bytes(s) <= (size_t)kStepMaxLdsBytes;
}

hipError_t launch_decode_step(const Dims& s, const StepInputs& in, hipStream_t st)
{
    const int pad = kTileRows;
    StepParams p{};
    p.q = static_cast<const char*>(in.q);
    p.K = static_cast<const char*>(in.K);
    p.V = static_cast<const char*>(in.V);
    p.Kbar = static_cast<const char*>(in.Kbar);
    p.Vbar = static_cast<const char*>(in.Vbar);
    p.tok_idx = in.tok_idx;
    p.tok_logw = in.tok_logw;
    p.scores = in.scores;
    p.sel = in.sel;
    p.out = in.out;
    p.lse = in.lse;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.n = s.n;
    p.L = s.L;
    p.nb = s.nb;
    p.k = in.k < s.nb ? in.k : s.nb;
    p.m = in.m;
    p.proxies = in.proxies;
    p.pend = in.proxies ? s.nb : 0;
    p.wbeg = (p.pend + pad - 1) / pad * pad;
    p.ebeg = p.wbeg + (in.m + pad - 1) / pad * pad;
    const int exact_rows = p.k * s.L;
    p.rows = exact_rows > 0 ? p.ebeg + exact_rows : (in.m > 0 ? p.wbeg + in.m : p.pend);
    p.lstride = (s.nb + pad - 1) / pad * pad;
    p.scale = s.scale;
    p.ln_L = s.ln_L;
    p.ln_last = s.ln_last;
    p.scale_log2 = s.scale * kLog2e;
    const size_t shm = step_lds_bytes(s);
    if (s.d == 128) return launch_step_d<128>(p, s.pairs(), shm, st);
    if (s.d == 64) return launch_step_d<64>(p, s.pairs(), shm, st);
    return hipErrorInvalidValue;
}

}  // namespace csa

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
//
// CLUSTER: the same step over query-guided clusters ("OpenAttention reads 1%
// of the KV cache -- Count-aware tail proxy", section "Three helpers that make
// the proxy accurate"): the rows of Kbar / Vbar are the clusters' mean keys and
// values, the count term of a row is ln of its cluster's size (from the ranges
// offsets[c] .. offsets[c + 1]; -inf for an empty cluster), and the exact rows
// are the selected clusters' ranges of K / V (the cache in cluster order), whose
// number is known only after the selection: each wave then forms the running
// row counts of the selected clusters and plans its exact tiles.
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
    const int32_t* offsets;  // CLUSTER: cluster ranges [B, Hkv, nb + 1]
    int Hq, Hkv, G, n, L, nb, k, m, proxies;
    int pend;    // proxy rows [0, pend): one per block (0 without proxies)
    int cr;      // cache rows: the m weighted tokens, then the k L exact rows
    int rt, nc;  // cache rows per cache tile, cache tiles
    int lstride;                 // LDS row stride of the logits (nb rounded up to 32)
    float scale, ln_L, ln_last, scale_log2;
};

template <int D, int HG, bool CLUSTER>
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
    // CLUSTER: each wave's copy of the selected clusters' first rows and running row counts
    __shared__ int32_t cl_start[CLUSTER ? NW : 1][kStepMaxK], cl_cum[CLUSTER ? NW : 1][kStepMaxK + 1];

    const int LS = p.lstride, G = p.G, nb = p.nb;
    float* lsm = dyn;                                              // [G][LS] block logits (natural log)
    float* ssm = dyn + G * LS;                                     // [LS] group scores
    uint32_t* bits = reinterpret_cast<uint32_t*>(ssm + LS);        // [LS / 32] selected blocks
    int32_t* off_sm = reinterpret_cast<int32_t*>(bits + LS / 32);  // CLUSTER: [nb + 1] cluster ranges
    // Over blocks, workgroup w (which runs on XCD w mod 8) takes pair
    // (w mod 8) P / 8 + w / 8: each XCD streams a contiguous eighth of the pairs
    // (32-sequence layer 20.29 -> 20.00 us against pair w; over clusters 27.69 ->
    // 27.90 us, so the cluster step keeps pair w).
    const int pair = !CLUSTER && gridDim.x % 8 == 0
                         ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8)
                         : (int)blockIdx.x;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int32_t* off = CLUSTER ? p.offsets + (size_t)pair * (nb + 1) : nullptr;
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

    // Tiles go in address order in every workgroup (tile orders rotated by a
    // per-workgroup offset, against workgroups walking the same address offsets
    // side by side, took 20.21 -> 20.38 us per step at 32 sequences and 27.85
    // -> 28.15 us over clusters).
    const int nK = (nb + TR - 1) / TR;      // mean-key tiles
    const int nP = (p.pend + TR - 1) / TR;  // proxy tiles
    int nC = p.nc;                          // cache tiles of p.rt rows (CLUSTER: set after the selection)
    int nT = nP + nC;
    // first row of tile t: a proxy row, or a cache row (index into the cache rows)
    auto row0 = [&](int t) { return t < nP ? t * TR : (t - nP) * p.rt; };
    // this wave's tiles are t = wave + j NW: first Pw proxy tiles, then cache tiles
    const int Pw = wave < nP ? (nP - wave + NW - 1) / NW : 0;
    int Tw = wave < nT ? (nT - wave + NW - 1) / NW : 0;
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
            // rows past the proxies point past the buffer: zeros, no memory traffic
            eng.set_row(tb, lane, (uint32_t)(r < p.pend ? r : nb), lw);
        }
    };

    // ---- phase 1: block logits of every head -> LDS ---------------------------
    // CLUSTER: the range starts of the rows this lane writes logits for (rows
    // base + 16 rb + 4 g16 + i, and the next one), loaded with the tile's keys
    auto load_ranges = [&](int base, int (&o)[2][5]) {
        if constexpr (CLUSTER) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 5; ++i) {
                    const int row = base + rb * 16 + 4 * g16 + i;
                    o[rb][i] = row <= nb ? off[row] : 0;
                }
        }
    };
    auto logits_to_lds = [&](int base, const uint4 (&kr)[E::NI], const int (&o)[2][5]) {
        f32x4_t c[2];
        eng.qk_tile(kr, c);
        if (n16 < G) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = base + rb * 16 + 4 * g16 + i;
                    float lnc = row == nb - 1 ? p.ln_last : p.ln_L;
                    if constexpr (CLUSTER) {
                        const int cnt = o[rb][i + 1] - o[rb][i];
                        lnc = cnt > 0 ? logf((float)cnt) : kNegInf;
                        if (row < nb && n16 == 0) off_sm[row] = o[rb][i];
                        if (row == nb - 1 && n16 == 0) off_sm[nb] = o[rb][i + 1];
                    }
                    if (row < nb) lsm[n16 * LS + row] = fmaf(c[rb][i], p.scale, lnc);
                }
        }
    };
    auto load_keys = [&](int base, uint4 (&kr)[E::NI], bool live) {  // past nb: zeros
        const __amdgpu_buffer_rsrc_t r = Ks(live);
        if constexpr (E::kLdsKeys) {  // whole rows, then through LDS
#pragma unroll
            for (int jj = 0; jj < E::NI; ++jj)
                kr[jj] = buffer_ld16_nt(r, (uint32_t)(base + E::RPV * jj + eng.gv) * RB + eng.cv * 16);
        } else {  // the operand layout
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    kr[KS * rb + s] = buffer_ld16(r, (uint32_t)(base + rb * 16 + n16) * RB + g16 * 16 + s * 64);
        }
    };
    // The mean keys decide the selection: they have the memory system to
    // themselves.  The wave's first two proxy value tiles go out once its keys
    // have arrived, and stream in while the selection is made.
    // two adjacent tiles in flight per wave (tiles w and w + NW instead: 19.89 ->
    // 20.13 us per step at 32 sequences, 21.38 -> 21.67 at 64 query heads)
    for (int t = 2 * wave; t < nK; t += 2 * NW) {
        uint4 k0[E::NI], k1[E::NI];
        int o0[2][5], o1[2][5];
        const int b0 = t * TR, b1 = (t + 1) * TR;
        const bool two = t + 1 < nK;
        load_ranges(b0, o0);  // the few range words ahead of the key tiles, not behind them
        if (two) load_ranges(b1, o1);
        load_keys(b0, k0, true);
        load_keys(b1, k1, two);
        logits_to_lds(b0, k0, o0);
        if (two) logits_to_lds(b1, k1, o1);
    }
    // The first proxy value tile goes out before the barrier, the second after
    // it, and from the waves that compute the head log-normalisers only once
    // the selection is known: a wave whose loads wait for room in the memory
    // queue behind the other waves' must not hold up a barrier or the
    // selection.  Measured at 32 sequences of the 32-head layer: 21.95 us per
    // step, against 22.8 with both tiles before the barrier, 22.1 with the
    // second one right after it from every wave, 24.9 with both after it.
    auto issue_second_proxies = [&]() {
        if (Pw > 1) set_proxy_rows(1, 1, false);
        eng.issue_values(VB, 1, Vs(Pw > 1));
    };
    if (Pw > 0) set_proxy_rows(0, 0, false);
    eng.issue_values(VA, 0, Vs(Pw > 0));
    __syncthreads();
    // the last G waves compute the head log-normalisers (the younger wave of each
    // SIMD up to four heads: the older ones, which win the issue arbitration,
    // issue their proxy values meanwhile; 20.00 -> 19.83 and 20.06 -> 19.98 us
    // per step in two sessions against the first G waves)
    const bool lse_wave = G > 1 && wave >= NW - G;
    if (!lse_wave) issue_second_proxies();

    // ---- phase 2: group score and top-k ----------------------------------------
    if (G > 1) {
        if (lse_wave) {
            const int h = wave - (NW - G);
            const float lse = head_lse(lsm + h * LS, nb, lane);
            if (lane == 0) lse_h[h] = lse;
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

    if (lse_wave) issue_second_proxies();

    if constexpr (CLUSTER) {
        // the selected clusters' ranges: lane r < kk holds cluster sel_sm[r]; running
        // row counts by an inclusive scan over the lanes (each wave its own copy)
        int cnt = 0, st = 0;
        if (lane < kk) {
            const int c = sel_sm[lane];
            st = off_sm[c];
            cnt = off_sm[c + 1] - st;
        }
        int inc = cnt;
#pragma unroll
        for (int d2 = 1; d2 < 32; d2 <<= 1) {
            const int o = __shfl_up(inc, d2);
            if (lane >= d2) inc += o;
        }
        if (lane < kk) {
            cl_start[wave][lane] = st;
            cl_cum[wave][lane] = inc - cnt;
        }
        const int exact = __builtin_amdgcn_readfirstlane(__shfl(inc, kk > 0 ? kk - 1 : 0) * (kk > 0 ? 1 : 0));
        if (lane == 0) cl_cum[wave][kk] = exact;
        wave_lds_fence();
        nC = (exact + TR - 1) / TR;
        nT = nP + nC;
        Tw = wave < nT ? (nT - wave + NW - 1) / NW : 0;
    }

    // ---- phase 3: attention ------------------------------------------------------
    // Cache row c: weighted token c (c < m), else exact row c - m of the
    // selected blocks.  Rows that do not count point past the cache buffers
    // (zeros, no memory traffic) with log-weight -inf.
    auto resolve_cache = [&](int c, bool valid, uint32_t& row, float& lw) {
        row = (uint32_t)p.n;
        lw = kNegInf;
        if (!valid || c >= (CLUSTER ? p.m + cl_cum[wave][kk] : p.cr)) return;
        if (c < p.m) {
            const int tok = p.tok_idx[(size_t)pair * p.m + c];
            if (tok >= 0 && tok < p.n) {
                row = (uint32_t)tok;
                lw = p.tok_logw[(size_t)pair * p.m + c] * kLog2e;
            }
        } else if constexpr (CLUSTER) {  // exact row e: the last selected cluster starting at or before it
            const int e = c - p.m;
            int slot = 0;
            for (int s2 = 1; s2 < kk; ++s2)
                if (cl_cum[wave][s2] <= e) slot = s2;
            row = (uint32_t)(cl_start[wave][slot] + (e - cl_cum[wave][slot]));
            lw = 0.0f;
        } else {
            const int e = c - p.m;
            const int slot = e / p.L;
            const int tok = sel_sm[slot] * p.L + (e - slot * p.L);
            if (tok < p.n) {
                row = (uint32_t)tok;
                lw = 0.0f;
            }
        }
    };
    // a cache tile holds p.rt <= 32 rows
    auto set_cache_rows = [&](int jj, int tb) {
        if (lane < TR) {
            uint32_t row;
            float lw;
            resolve_cache(row0(tile_of(jj)) + lane, lane < p.rt, row, lw);
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
    // the cache tiles (key and value tiles, one and a half in flight).  The
    // keys of the wave's first cache tile go out now, so that they stream
    // behind the proxy values instead of after them; its values follow once the
    // proxy tiles are done (the whole first tile now would not fit in registers
    // beside them).  With P V on the matrix cores this holds up to eight heads
    // (64-head layer over the headline cache: 22.41 -> 21.79 us, against the
    // keys waiting for the proxy tiles from five heads on).
    static_assert(HG <= 8, "the fused step takes up to eight heads per KV head");
    if (Pw > 0) set_proxy_rows(0, 0, true);
    if (Pw > 1) set_proxy_rows(1, 1, true);
    typename E::Tile CA, CB;
    const bool any_cache = Tw > Pw;
    if (any_cache) set_cache_rows(Pw, 2);
    eng.issue_keys(CA, 2, Kc(any_cache));
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
    eng.issue_values(CA.vr, 2, Vc(any_cache));
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

size_t step_lds_bytes(const Dims& s, bool cluster = false)
{
    const int ls = (s.nb + kTileRows - 1) / kTileRows * kTileRows;
    return (size_t)(s.G + 1) * ls * sizeof(float) + (size_t)(ls / 32) * sizeof(uint32_t) +
           (cluster ? (size_t)(ls + 1) * sizeof(int32_t) : 0);
}

template <int D, bool CLUSTER>
hipError_t launch_step_d(const StepParams& p, int pairs, size_t shm, hipStream_t st)
{
    const dim3 grid((unsigned)pairs), block(kStepWaves * 64);
    switch (p.G) {
    case 1: decode_step_kernel<D, 1, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 2: decode_step_kernel<D, 2, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 3: decode_step_kernel<D, 3, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 4: decode_step_kernel<D, 4, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 5: decode_step_kernel<D, 5, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 6: decode_step_kernel<D, 6, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 7: decode_step_kernel<D, 7, CLUSTER><<<grid, block, shm, st>>>(p); break;
    case 8: decode_step_kernel<D, 8, CLUSTER><<<grid, block, shm, st>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool fused_step_ok(const Dims& s, int k, int m, int proxies)
{
    const long rows = (proxies ? (long)(s.nb - k) : 0L) + (long)k * s.L + m;  // virtual rows per KV head
    const bool enough = s.pairs() >= kFusedStepMinPairs ||
                        (rows * s.G <= kFusedStepSmallWork && s.nb <= kLseFromLogitsMaxBlocks);
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
    // cache rows in tiles of 32 (fewer tiles of more rows beat an even split
    // of the rows over the waves: each further tile of a wave is one more
    // memory round trip after the selection)
    p.cr = in.m + p.k * s.L;
    p.rt = pad;
    p.nc = (p.cr + pad - 1) / pad;
    p.lstride = (s.nb + pad - 1) / pad * pad;
    p.scale = s.scale;
    p.ln_L = s.ln_L;
    p.ln_last = s.ln_last;
    p.scale_log2 = s.scale * kLog2e;
    const size_t shm = step_lds_bytes(s);
    if (s.d == 128) return launch_step_d<128, false>(p, s.pairs(), shm, st);
    if (s.d == 64) return launch_step_d<64, false>(p, s.pairs(), shm, st);
    return hipErrorInvalidValue;
}

bool cluster_step_ok(const Dims& s, int k)
{
    return s.dtype == DT_BF16 && s.G <= 8 && k >= 0 && k <= kStepMaxK && s.nb <= kStepMaxBlocks &&
           s.pairs() >= kFusedStepMinPairs && step_lds_bytes(s, true) <= (size_t)kStepMaxLdsBytes;
}

hipError_t launch_cluster_step(const Dims& s, const ClusterStepInputs& in, hipStream_t st)
{
    StepParams p{};
    p.q = static_cast<const char*>(in.q);
    p.K = static_cast<const char*>(in.Kg);
    p.V = static_cast<const char*>(in.Vg);
    p.Kbar = static_cast<const char*>(in.Kc);
    p.Vbar = static_cast<const char*>(in.Vc);
    p.offsets = in.offsets;
    p.scores = in.scores;
    p.sel = in.sel;
    p.out = in.out;
    p.lse = in.lse;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.n = s.n;
    p.L = 1;
    p.nb = s.nb;
    p.k = in.k < s.nb ? in.k : s.nb;
    p.m = 0;
    p.proxies = in.proxies;
    p.pend = in.proxies ? s.nb : 0;
    p.cr = 0;
    p.rt = kTileRows;
    p.nc = 0;  // the exact tiles are planned after the selection
    p.lstride = (s.nb + kTileRows - 1) / kTileRows * kTileRows;
    p.scale = s.scale;
    p.scale_log2 = s.scale * kLog2e;
    const size_t shm = step_lds_bytes(s, true);
    if (s.d == 128) return launch_step_d<128, true>(p, s.pairs(), shm, st);
    if (s.d == 64) return launch_step_d<64, true>(p, s.pairs(), shm, st);
    return hipErrorInvalidValue;
}

}  // namespace csa

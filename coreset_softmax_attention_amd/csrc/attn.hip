// attn.hip -- one online-softmax pass over the virtual tokens of a KV head.
//
// The virtual-token list of KV head (b, j) is the concatenation of
//   [proxy]    one row per block of the summary arrays, key Kbar_b, value
//              Vbar_b, log-weight ln c_b; the rows of selected blocks are
//              masked.  This is the count-aware proxy of "OpenAttention reads
//              1% of the KV cache -- Count-aware tail proxy", section
//              "Skipping reviews without losing the verdict";
//   [weighted] m gathered tokens with their log-weights (weighted-coreset
//              attention, "WildCat: Near-Linear Attention in Theory and
//              Practice", Abstract);
//   [exact]    every token of the selected blocks, log-weight 0
//              (dense mode: all n tokens in order).
// Proxy rows come first because their addresses do not depend on the
// selection: their loads start while the selection is still being read.
// Reading all summary rows contiguously and masking the few selected ones
// costs k extra rows but keeps the proxy reads fully coalesced.
//
// Work split: a workgroup owns a contiguous range of virtual rows of one KV
// head for up to 8 query heads of its group (split-K).  Logits use the base-2
// exponent: x = log2(e) (scale q.k + logw).  Partial softmax states (running
// max, sum, unnormalised output) are merged across lanes (shuffles), waves
// (LDS) and splits (merge kernel), always in a fixed order, so results are
// bitwise reproducible.
//
// bfloat16 path (attn_mfma_kernel): each wave takes tiles of 32 virtual rows.
// The rows of a tile are resolved once (index, source array, log-weight) into
// a per-wave LDS table.  q K^T for the tile is two 16x16x32 bf16 MFMA chains
// (rows x heads, the group's heads padded to 16 columns); the online softmax
// runs once per (row, head) on the MFMA output lanes; the probabilities go
// through LDS to the lanes that hold the tile's value rows (16-byte chunks,
// whole rows per lane group, coalesced), which accumulate P V in fp32.
// binary32 path (attn_valu_kernel): rows as 16-byte chunks over LPR lanes,
// dot products reduced with DPP, one online-softmax state per lane group.
#include "attn_engine.hpp"
#include "device.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kNW = 4;                // waves per workgroup
constexpr int kMaxSplitRows = 8192;   // rows per workgroup (bitmap capacity)
constexpr int kMaxSelLds = 512;       // selections kept in LDS by the bfloat16 kernel
constexpr int kMaxTokLds = 1024;      // weighted tokens of a workgroup kept in LDS
constexpr int kTargetWorkgroups = 2048;
// bfloat16 path, chosen by measurement over (waves, workgroups) on the headline
// shape: eight waves (two per SIMD), one workgroup per CU at least
constexpr int kMfmaWaves = 8;          // waves per workgroup
constexpr int kMfmaMinWgs = 256;       // workgroups to cover every CU once
constexpr int kMfmaTilesPerWave = 16;  // tiles a wave streams before the rows are split
constexpr int kDirectMaxK = 32;        // selection held one block per lane in direct mode

constexpr int unroll_for(int hg) { return hg <= 4 ? 8 : 4; }

struct AttnParams {
    const char* q;
    const char* K;
    const char* V;
    const char* Kbar;
    const char* Vbar;
    const int32_t* sel;
    const int32_t* tok_idx;
    const float* tok_logw;
    float* out;
    float* lse;
    float* part;
    const float* cand_score;   // direct mode: candidates to rank instead of sel (may be null)
    const int32_t* cand_idx;
    int32_t* sel_out;          // with candidates: the ranked selection (may be null)
    const float* plog;         // direct mode: the proxy rows' logits [B, Hq, nb], natural log (may be null)
    int ncand;
    int k, m, proxies, dense;
    int Hq, Hkv, G, n, L, nb;
    int rows, exact_rows, splits, rows_per_split;
    int pend, wbeg, ebeg;      // end of the proxy rows, first weighted row, first exact row
    int direct;                // rows resolved from the global arrays, selection in registers (no LDS copies)
    float scale_log2;          // scale * log2(e)
    float log2_L, log2_last;   // log2 c_b of a full and of the last block
};

template <int DT, int D, int HG, int U>
__global__ void __launch_bounds__(kNW * 64) attn_valu_kernel(const AttnParams p)
{
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    constexpr int T = RPW * U;  // rows per wave tile

    __shared__ uint32_t sel_bits[kMaxSplitRows / 32];
    __shared__ float sm_m[kNW][HG], sm_l[kNW][HG];
    __shared__ float sm_acc[kNW][HG][D];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const int pair = blockIdx.x / p.splits, split = blockIdx.x - pair * p.splits;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int g0 = blockIdx.y * HG;        // first head of this chunk within the group
    const int nh = min(HG, p.G - g0);      // active heads in the chunk
    const int h0 = j * p.G + g0;           // global index of the chunk's first query head

    const int r0 = split * p.rows_per_split;
    const int r1 = min(p.rows, r0 + p.rows_per_split);

    // Bitmap of selected blocks among the proxy rows [pb_lo, pb_hi) of this range.
    const int pb_lo = r0;
    const int pb_hi = min(r1, p.pend);
    if (pb_hi > pb_lo) {
        const int words = (pb_hi - pb_lo + 31) >> 5;
        for (int w = threadIdx.x; w < words; w += kNW * 64) sel_bits[w] = 0;
        __syncthreads();
        const int32_t* S = p.sel + (size_t)pair * p.k;
        for (int i = threadIdx.x; i < p.k; i += kNW * 64) {
            const int blk = S[i];
            if (blk >= pb_lo && blk < pb_hi) atomicOr(&sel_bits[(blk - pb_lo) >> 5], 1u << ((blk - pb_lo) & 31));
        }
        __syncthreads();
    }

    float qf[HG][EPL];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
        if (g < nh) {
            const uint4 r = ld16(p.q + ((size_t)(b * p.Hq + h0 + g) * D) * Elem<DT>::bytes + li * 16);
            unpack<DT>(r, qf[g]);
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) qf[g][e] = 0.0f;
        }
    }

    float m_[HG], l_[HG], acc[HG][EPL];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
        m_[g] = kNegInf;
        l_[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }

    const size_t kv_pair = (size_t)pair * p.n;
    const size_t sm_pair = (size_t)pair * p.nb;

    for (int base = r0 + wave * T; base < r1; base += kNW * T) {
        const char* kp[U];
        const char* vp[U];
        float lw[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * RPW + gi;
            bool valid = r < r1;
            const char* kb = p.K;
            const char* vb = p.V;
            size_t row = kv_pair;
            float w = 0.0f;
            if (r < p.pend) {
                const int blk = r;
                kb = p.Kbar;
                vb = p.Vbar;
                row = sm_pair + blk;
                w = blk == p.nb - 1 ? p.log2_last : p.log2_L;
                if (valid) valid = !((sel_bits[(blk - pb_lo) >> 5] >> ((blk - pb_lo) & 31)) & 1u);
            } else if (r >= p.wbeg && r < p.wbeg + p.m) {
                const int t = r - p.wbeg;
                const int tok = p.tok_idx[(size_t)pair * p.m + t];
                valid = valid && tok >= 0 && tok < p.n;
                row = kv_pair + (valid ? tok : 0);
                w = p.tok_logw[(size_t)pair * p.m + t] * kLog2e;
            } else if (r >= p.ebeg && r < p.rows) {
                const int e = r - p.ebeg;
                int tok;
                if (p.dense) {
                    tok = e;
                } else {
                    const int slot = e / p.L;
                    tok = p.sel[(size_t)pair * p.k + slot] * p.L + (e - slot * p.L);
                }
                valid = valid && tok >= 0 && tok < p.n;
                row = kv_pair + (valid ? tok : 0);
            } else {
                valid = false;
            }
            kp[u] = kb + row * RB + li * 16;
            vp[u] = vb + row * RB + li * 16;
            lw[u] = w;
            ok[u] = valid;
        }
        uint4 kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) kr[u] = ld16(kp[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) vr[u] = ld16(vp[u]);

        float x[U][HG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[EPL];
            unpack<DT>(kr[u], kf);
#pragma unroll
            for (int g = 0; g < HG; ++g) {
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) s = fmaf(qf[g][e], kf[e], s);
                s = group_sum<LPR>(s);
                x[u][g] = ok[u] ? fmaf(s, p.scale_log2, lw[u]) : kNegInf;
            }
        }
#pragma unroll
        for (int g = 0; g < HG; ++g) {
            float mx = m_[g];
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, x[u][g]);
            const float a = rescale(m_[g], mx);
            l_[g] *= a;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= a;
            m_[g] = mx;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                x[u][g] = x[u][g] == kNegInf ? 0.0f : exp2_(x[u][g] - mx);
                l_[g] += x[u][g];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[EPL];
            unpack<DT>(vr[u], vf);
#pragma unroll
            for (int g = 0; g < HG; ++g)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(x[u][g], vf[e], acc[g][e]);
        }
    }

    // merge the lane groups of the wave (lanes li, li + LPR, ... hold the same chunk)
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < HG; ++g) {
            const float mo = __shfl_xor(m_[g], off);
            const float lo = __shfl_xor(l_[g], off);
            const float mn = fmaxf(m_[g], mo);
            const float a = rescale(m_[g], mn), ao = rescale(mo, mn);
            l_[g] = l_[g] * a + lo * ao;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * a + __shfl_xor(acc[g][e], off) * ao;
            m_[g] = mn;
        }
    }
    if (gi == 0) {
#pragma unroll
        for (int g = 0; g < HG; ++g) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_acc[wave][g][li * EPL + e] = acc[g][e];
            if (li == 0) {
                sm_m[wave][g] = m_[g];
                sm_l[wave][g] = l_[g];
            }
        }
    }
    __syncthreads();

    // merge the waves and write the result (one split) or the partial state
    for (int idx = threadIdx.x; idx < HG * D; idx += kNW * 64) {
        const int g = idx / D, e = idx - g * D;
        if (g >= nh) continue;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kNW; ++w) M = fmaxf(M, sm_m[w][g]);
        float Ls = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) {
            const float a = rescale(sm_m[w][g], M);
            Ls += sm_l[w][g] * a;
            A += sm_acc[w][g][e] * a;
        }
        if (p.splits == 1) {
            const int h = h0 + g;
            p.out[((size_t)b * p.Hq + h) * D + e] = A / Ls;
            if (e == 0 && p.lse) p.lse[(size_t)b * p.Hq + h] = (M + log2f(Ls)) * kLn2;
        } else {
            float* st = p.part + (((size_t)pair * p.splits + split) * p.G + (g0 + g)) * (D + 2);
            if (e == 0) {
                st[0] = M;
                st[1] = Ls;
            }
            st[2 + e] = A;
        }
    }
}

// ---------------------------------------------------------------------------
// bfloat16 path: q K^T on the matrix cores
// ---------------------------------------------------------------------------




// Where resolve_row finds the selection and the weighted tokens: the
// workgroup's copies in LDS once they are filled, the global arrays before.
struct RowSources {
    const int32_t* sel;      // selection of this KV head (k entries)
    const int32_t* tok_idx;  // weighted tokens, indexed from tok_base
    const float* tok_logw;
    int tok_base;            // index of tok_idx[0] in the KV head's list
};

// Whether block r is among the k selected blocks held one per lane (lane s <
// k: selv = sel[s]) by the wave.
__device__ __forceinline__ bool in_selection(int r, int selv, int k)
{
    bool hit = false;
    for (int s = 0; s < k; ++s) hit |= __builtin_amdgcn_readlane(selv, s) == r;
    return hit;
}

// Virtual row r of KV head `pair` -> (row index in its source array, log2-
// weight); -inf marks a row outside [.., r1), a padding row, a token outside
// the cache, or (when `mask`) a proxy of a selected block (from the bitmap, or
// in direct mode from the selection in the wave's registers).  Invalid rows
// keep row 0, a valid address.
__device__ __forceinline__ void resolve_row(const AttnParams& p, const RowSources& src, int r, int r1, int pb_lo,
                                            const uint32_t* sel_bits, bool mask, int selv, uint32_t& row, float& lw)
{
    row = 0;
    lw = kNegInf;
    if (r >= r1) return;
    if (r < p.pend) {
        row = (uint32_t)r;
        const bool selected = mask && (p.direct ? in_selection(r, selv, p.k)
                                                : ((sel_bits[(r - pb_lo) >> 5] >> ((r - pb_lo) & 31)) & 1u) != 0);
        if (!selected) lw = r == p.nb - 1 ? p.log2_last : p.log2_L;
    } else if (r >= p.wbeg && r < p.wbeg + p.m) {
        const int t = r - p.wbeg - src.tok_base;
        const int tok = src.tok_idx[t];
        if (tok >= 0 && tok < p.n) {
            row = (uint32_t)tok;
            lw = src.tok_logw[t] * kLog2e;
        }
    } else if (r >= p.ebeg) {
        const int e = r - p.ebeg;
        int tok;
        if (p.dense) {
            tok = e;
        } else {
            const int slot = e / p.L;
            tok = src.sel[slot] * p.L + (e - slot * p.L);
        }
        if (tok >= 0 && tok < p.n) {
            row = (uint32_t)tok;
            lw = 0.0f;
        }
    }
}

template <int D, int HG, int NW>
__global__ void __launch_bounds__(NW * 64) attn_mfma_kernel(const AttnParams p)
{
    using E = MfmaEngine<D, HG, NW>;
    constexpr int TR = kTileRows, RB = E::RB;
    __shared__ uint32_t sel_bits[kMaxSplitRows / 32];
    __shared__ int32_t sel_sm[kMaxSelLds];
    __shared__ int32_t tok_sm[kMaxTokLds];
    __shared__ float logw_sm[kMaxTokLds];
    __shared__ typename E::Smem sm;
    static_assert(kMaxTokLds >= NW * 128 && kMaxSelLds >= NW * kDirectMaxK, "ranked mode's per-wave LDS");

    // workgroup w (on XCD w mod 8) takes item (w mod 8) N / 8 + w / 8: each XCD
    // streams a contiguous eighth of the (pair, split) items (sparse_decode_attn
    // over the 32-sequence layer 20.98 -> 20.70 us, the 128K weighted-coreset step
    // 25.90 -> 25.65 us)
    const int wg = gridDim.x % 8 == 0 ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8)
                                      : (int)blockIdx.x;
    const int pair = wg / p.splits, split = wg - pair * p.splits;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int g0 = blockIdx.y * HG;
    const int nh = min(HG, p.G - g0);
    const int h0 = j * p.G + g0;
    const int r0 = split * p.rows_per_split;
    const int r1 = min(p.rows, r0 + p.rows_per_split);
    // selected-block bitmap over the proxy rows [pb_lo, pb_hi) of this range; it is
    // filled after the first tile's loads are in flight
    const int pb_lo = r0;
    const int pb_hi = min(r1, p.pend);
    const bool direct = p.direct != 0;
    const int bitmap_words = !direct && pb_hi > pb_lo ? (pb_hi - pb_lo + 31) >> 5 : 0;
    for (int w = threadIdx.x; w < bitmap_words; w += NW * 64) sel_bits[w] = 0;

    E eng(sm, p.q + (size_t)(b * p.Hq + h0) * RB, nh);
    const int lane = eng.lane, wave = eng.wave;

    // The selection and this workgroup's weighted tokens are copied to LDS
    // (when they fit) after the first tile is issued; until then, and when
    // they do not fit, rows are resolved from the global arrays.
    const int w_lo = max(r0, p.wbeg), w_hi = min(r1, p.wbeg + p.m);  // weighted rows of this range
    const bool sel_in_lds = !direct && !p.dense && p.k > 0 && p.k <= kMaxSelLds;
    const bool tok_in_lds = !direct && w_hi > w_lo && w_hi - w_lo <= kMaxTokLds;
    // Ranked mode (direct only): each wave ranks the KV head's candidates itself.
    const bool ranked = direct && p.cand_score != nullptr;
    RowSources src{ranked ? nullptr : p.sel + (size_t)pair * p.k, p.tok_idx + (size_t)pair * p.m,
                   p.tok_logw + (size_t)pair * p.m, 0};
    // Direct mode (a tile or two per wave, k <= 32): no LDS copies and no barrier
    // before the tiles; the selection sits one block per lane in every wave.
    int selv = direct && !ranked && !p.dense && lane < p.k ? src.sel[lane] : -1;

    auto set_rows = [&](int base, int tb, bool masked) {
        if (lane < TR) {
            uint32_t row;
            float lw;
            resolve_row(p, src, base + lane, r1, pb_lo, sel_bits, masked, selv, row, lw);
            eng.set_row(tb, lane, row, lw);
        }
    };
    // Tile loads are issued unconditionally: a tile past the wave's list reads
    // through empty buffers (zeros, no memory traffic).  Together with loops
    // that have no exit between their halves, this lets the compiler's wait
    // before a tile's use cover that tile's loads only.
    // Segments are padded to whole tiles, so every tile reads either the cache
    // (weighted and exact rows) or the summaries (proxy rows).  The buffers are
    // built from wave-uniform base addresses and sizes.
    const char* const kc = p.K + (size_t)pair * p.n * RB;
    const char* const vc = p.V + (size_t)pair * p.n * RB;
    const char* const ks = p.proxies ? p.Kbar + (size_t)pair * p.nb * RB : p.K;
    const char* const vs = p.proxies ? p.Vbar + (size_t)pair * p.nb * RB : p.V;
    const uint32_t cbytes = (uint32_t)p.n * RB, sbytes = p.proxies ? (uint32_t)p.nb * RB : 0u;
    auto rsrc = [&](int base, bool live, bool keys) {
        const bool summ = base < p.wbeg;  // uniform over the wave
        const uint32_t bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)(live ? (summ ? sbytes : cbytes) : 0u));
        return buffer_rsrc(summ ? (keys ? ks : vs) : (keys ? kc : vc), bytes);
    };
    // Proxy tiles whose logits are given (the split scores' logits of the KV
    // head's query heads): the lane's logits of head n16 ride in the tile's key
    // registers instead of the mean keys.  A row past the blocks reads the next
    // head's logits or nothing; it is masked.
    // (five to eight heads: with fewer, the extra path would push the kernel's
    // registers into scratch)
    const bool given = HG > 4 && direct && p.plog != nullptr;
    const float* const lg = given ? p.plog + ((size_t)b * p.Hq + h0) * p.nb : nullptr;
    const int lg_head = min(eng.n16, nh - 1);
    auto given_tile = [&](int base) { return given && base < p.wbeg; };  // uniform over the wave
    auto load_given = [&](int base, typename E::Tile& t, bool live) {
        const __amdgpu_buffer_rsrc_t r =
            buffer_rsrc(lg, (uint32_t)__builtin_amdgcn_readfirstlane((int)(live ? nh * p.nb * 4 : 0)));
        const uint32_t off = (uint32_t)(lg_head * p.nb + base + 4 * eng.g16) * 4;
        t.kr[0] = buffer_ld16(r, off);
        t.kr[1] = buffer_ld16(r, off + 64);
        // the tile's other key registers are unused here; zeros let the compiler
        // keep one register set for tiles of given and of loaded keys (five to
        // eight heads: 241 -> 198 registers)
#pragma unroll
        for (int jj = 2; jj < E::NI; ++jj) t.kr[jj] = make_uint4(0u, 0u, 0u, 0u);
    };
    auto issue = [&](int base, typename E::Tile& t, int tb, bool masked, bool live) {
        if (live) set_rows(base, tb, masked);
        if (given_tile(base)) {
            load_given(base, t, live);
            eng.issue(t, tb, rsrc(base, live, true), rsrc(base, live, false), false);
        } else {
            eng.issue(t, tb, rsrc(base, live, true), rsrc(base, live, false), true);
        }
    };
    auto issue_keys = [&](int base, typename E::Tile& t, int tb, bool live) {
        if (live) set_rows(base, tb, true);
        if (given_tile(base))
            load_given(base, t, live);
        else
            eng.issue_keys(t, tb, rsrc(base, live, true));
    };
    auto issue_values = [&](int base, typename E::Tile& t, int tb, bool live) {
        eng.issue_values(t.vr, tb, rsrc(base, live, false));
    };
    auto compute = [&](const typename E::Tile& t, int tb, int base) {
        float x[8];
        if (given_tile(base))
            eng.logits_given(tb, __builtin_bit_cast(float4, t.kr[0]), __builtin_bit_cast(float4, t.kr[1]), x);
        else
            eng.logits_mfma(t, tb, p.scale_log2, x);
        eng.softmax(x);
    };

    // Two tiles form the software pipeline: tile t's q K^T and softmax run before
    // tile t+1's loads are issued (so t's key registers are free again), and t's
    // P V runs while t+1 is in flight.
    // Tile order: this range's proxy tiles, then its cache tiles, in address
    // order (lists rotated by a per-workgroup offset, against workgroups side
    // by side walking the same address offsets, took sparse_decode_attn over
    // the 32-sequence layer 20.91 -> 21.20 us).
    const int pe = min(r1, p.wbeg), c0 = max(r0, p.wbeg);
    const int nP = pe > r0 ? (pe - r0 + TR - 1) / TR : 0;
    const int nC = r1 > c0 ? (r1 - c0 + TR - 1) / TR : 0;
    const int nT = nP + nC;
    auto row0 = [&](int t) { return t < nP ? r0 + t * TR : c0 + (t - nP) * TR; };

    typename E::Tile A, B;
    // this wave's tiles: jt = 0 .. Tw - 1 at t = wave + jt NW
    const int Tw = wave < nT ? (nT - wave + NW - 1) / NW : 0;
    auto base_of = [&](int jt) { return jt < Tw ? row0(wave + jt * NW) : 0; };
    const int first = Tw > 0 ? row0(wave) : r1;
    // In ranked mode a first tile of exact rows waits for the ranking; any other
    // goes out before it.
    const bool first_waits = ranked && Tw > 0 && first >= p.ebeg;
    if (!first_waits) issue(first, A, 0, false, Tw > 0);
    if (ranked) {
        // the candidates lie in ascending block order, so ranking by position
        // breaks ties towards the lower block; the wave's scratch and its copy of
        // the selection use the LDS of the non-direct modes
        uint32_t* scratch = reinterpret_cast<uint32_t*>(tok_sm) + wave * 128;
        int32_t* mine = sel_sm + wave * kDirectMaxK;
        const size_t cbase = (size_t)pair * ((p.nb + kCandChunk - 1) / kCandChunk) * p.k;
        const float* cs = p.cand_score + cbase;
        const int32_t* ci = p.cand_idx + cbase;
        auto emit = [&](int r, int i) { mine[r] = ci[i]; };
        if (p.ncand <= 128)
            wave_topk<2>([&](int i) { return cs[i]; }, p.ncand, p.k, lane, scratch, emit);
        else
            wave_topk<8>([&](int i) { return cs[i]; }, p.ncand, p.k, lane, scratch, emit);
        wave_lds_fence();
        selv = lane < p.k ? mine[lane] : -1;
        src.sel = mine;
        if (p.sel_out && split == 0 && wave == 0 && lane < p.k) p.sel_out[(size_t)pair * p.k + lane] = selv;
        if (first_waits) issue(first, A, 0, false, true);
    }
    if (direct && p.k > 0 && !p.dense) {  // mask the selected blocks among the first tile's proxy rows
        const int r = first + lane;
        if (lane < TR && r < pb_hi && in_selection(r, selv, p.k)) sm.tab_lw[0][wave][lane] = kNegInf;
        wave_lds_fence();
    }
    if (bitmap_words > 0 || sel_in_lds || tok_in_lds) {
        __syncthreads();  // bitmap cleared
        if (bitmap_words > 0 || sel_in_lds) {
            const int32_t* S = p.sel + (size_t)pair * p.k;
            for (int i = threadIdx.x; i < p.k; i += NW * 64) {
                const int blk = S[i];
                if (sel_in_lds) sel_sm[i] = blk;
                if (blk >= pb_lo && blk < pb_hi) atomicOr(&sel_bits[(blk - pb_lo) >> 5], 1u << ((blk - pb_lo) & 31));
            }
        }
        if (tok_in_lds) {
            for (int i = threadIdx.x; i < w_hi - w_lo; i += NW * 64) {
                tok_sm[i] = src.tok_idx[w_lo - p.wbeg + i];
                logw_sm[i] = src.tok_logw[w_lo - p.wbeg + i];
            }
        }
        __syncthreads();  // bitmap and copies complete
        if (sel_in_lds) src.sel = sel_sm;
        if (tok_in_lds) {
            src.tok_idx = tok_sm;
            src.tok_logw = logw_sm;
            src.tok_base = w_lo - p.wbeg;
        }
        // mask the selected blocks among the first tile's proxy rows
        const int r = first + lane;
        if (bitmap_words > 0 && lane < TR && r < pb_hi && ((sel_bits[(r - pb_lo) >> 5] >> ((r - pb_lo) & 31)) & 1u))
            sm.tab_lw[0][wave][lane] = kNegInf;
        wave_lds_fence();
    }
    int jt = 0;
    if constexpr (HG <= 4) {
        // a tile's keys go out before the logits of the tile ahead of it, its
        // values right after them
        issue_keys(base_of(1), B, 1, 1 < Tw);
        for (; jt + 1 < Tw; jt += 2) {
            compute(A, 0, base_of(jt));
            issue_values(base_of(jt + 1), B, 1, true);
            eng.accumulate(A);
            issue_keys(base_of(jt + 2), A, 0, jt + 2 < Tw);
            compute(B, 1, base_of(jt + 1));
            issue_values(base_of(jt + 2), A, 0, jt + 2 < Tw);
            eng.accumulate(B);
            issue_keys(base_of(jt + 3), B, 1, jt + 3 < Tw);
        }
    } else {
        // tile jt+1's loads go out once tile jt's keys are consumed
        for (; jt + 1 < Tw; jt += 2) {
            compute(A, 0, base_of(jt));
            issue(base_of(jt + 1), B, 1, true, true);
            eng.accumulate(A);
            compute(B, 1, base_of(jt + 1));
            issue(base_of(jt + 2), A, 0, true, jt + 2 < Tw);
            eng.accumulate(B);
        }
    }
    if (jt < Tw) {  // odd tile count: the last tile is in A
        compute(A, 0, base_of(jt));
        eng.accumulate(A);
    }
    float* part = p.splits == 1 ? nullptr : p.part + (((size_t)pair * p.splits + split) * p.G + g0) * (D + 2);
    eng.finish(nh, p.out + ((size_t)b * p.Hq + h0) * D, p.lse ? p.lse + (size_t)b * p.Hq + h0 : nullptr, part);
}

// Merge the per-split states of one query head, in split order: one workgroup
// per (KV head, head), one thread per output element.  The states of a chunk of
// splits are loaded together, so the merge costs a few memory round trips
// rather than one per split.
template <int D>
__global__ void __launch_bounds__(D) attn_merge_kernel(const float* part, int splits, int G, int Hq, int Hkv,
                                                       float* out, float* lse)
{
    constexpr int CH = 16;
    // each XCD merges a contiguous eighth of the (pair, head) items
    const int wg = gridDim.x % 8 == 0 ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8)
                                      : (int)blockIdx.x;
    const int pair = wg / G, g = wg - pair * G;
    const int b = pair / Hkv, j = pair - b * Hkv;
    const int e = threadIdx.x;
    const size_t stride = (size_t)G * (D + 2);
    const float* st = part + ((size_t)pair * splits * G + g) * (D + 2);
    float M = kNegInf;
    float Ls = 0.0f, A = 0.0f;
    if (splits <= CH) {
        // every state's loads go out together (one memory round trip); the
        // maximum, then the rescaled sums, in split order as below
        float m[CH], l[CH], a[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = c < splits;
            const float* sc = st + (in ? c : 0) * stride;
            m[c] = in ? sc[0] : kNegInf;
            l[c] = sc[1];
            a[c] = sc[2 + e];
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) M = fmaxf(M, m[c]);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (c < splits) {
                const float w = rescale(m[c], M);
                Ls += l[c] * w;
                A += a[c] * w;
            }
        }
        const int h = j * G + g;
        out[((size_t)b * Hq + h) * D + e] = A / Ls;
        if (e == 0 && lse) lse[(size_t)b * Hq + h] = (M + log2f(Ls)) * kLn2;
        return;
    }
    for (int s0 = 0; s0 < splits; s0 += CH) {
        float m[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) m[c] = s0 + c < splits ? st[(s0 + c) * stride] : kNegInf;
#pragma unroll
        for (int c = 0; c < CH; ++c) M = fmaxf(M, m[c]);
    }
    for (int s0 = 0; s0 < splits; s0 += CH) {
        float m[CH], l[CH], a[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bool in = s0 + c < splits;
            const float* sc = st + (in ? s0 + c : 0) * stride;
            m[c] = in ? sc[0] : kNegInf;
            l[c] = sc[1];
            a[c] = sc[2 + e];
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            if (s0 + c < splits) {
                const float w = rescale(m[c], M);
                Ls += l[c] * w;
                A += a[c] * w;
            }
        }
    }
    const int h = j * G + g;
    out[((size_t)b * Hq + h) * D + e] = A / Ls;
    if (e == 0 && lse) lse[(size_t)b * Hq + h] = (M + log2f(Ls)) * kLn2;
}

hipError_t launch_merge(const AttnParams& p, int D, int pairs, hipStream_t st)
{
    const dim3 grid((unsigned)(pairs * p.G));
    if (D == 128)
        attn_merge_kernel<128><<<grid, dim3(128), 0, st>>>(p.part, p.splits, p.G, p.Hq, p.Hkv, p.out, p.lse);
    else
        attn_merge_kernel<64><<<grid, dim3(64), 0, st>>>(p.part, p.splits, p.G, p.Hq, p.Hkv, p.out, p.lse);
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const AttnParams& p, int hg, int pairs, int hchunks, hipStream_t st)
{
    const dim3 grid((unsigned)(pairs * p.splits), (unsigned)hchunks, 1);
    const dim3 block(kNW * 64);
    switch (hg) {
    case 1: attn_valu_kernel<DT_F32, D, 1, unroll_for(1)><<<grid, block, 0, st>>>(p); break;
    case 2: attn_valu_kernel<DT_F32, D, 2, unroll_for(2)><<<grid, block, 0, st>>>(p); break;
    case 3: attn_valu_kernel<DT_F32, D, 3, unroll_for(3)><<<grid, block, 0, st>>>(p); break;
    case 4: attn_valu_kernel<DT_F32, D, 4, unroll_for(4)><<<grid, block, 0, st>>>(p); break;
    case 5: attn_valu_kernel<DT_F32, D, 5, unroll_for(5)><<<grid, block, 0, st>>>(p); break;
    case 6: attn_valu_kernel<DT_F32, D, 6, unroll_for(6)><<<grid, block, 0, st>>>(p); break;
    case 7: attn_valu_kernel<DT_F32, D, 7, unroll_for(7)><<<grid, block, 0, st>>>(p); break;
    case 8: attn_valu_kernel<DT_F32, D, 8, unroll_for(8)><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_merge(p, D, pairs, st);
}

template <int D>
hipError_t launch_bf16(const AttnParams& p, int hg, int pairs, int hchunks, hipStream_t st)
{
    const dim3 grid((unsigned)(pairs * p.splits), (unsigned)hchunks, 1);
    const dim3 block(kMfmaWaves * 64);
    switch (hg) {
    case 1: attn_mfma_kernel<D, 1, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 2: attn_mfma_kernel<D, 2, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 3: attn_mfma_kernel<D, 3, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 4: attn_mfma_kernel<D, 4, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 5: attn_mfma_kernel<D, 5, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 6: attn_mfma_kernel<D, 6, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 7: attn_mfma_kernel<D, 7, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    case 8: attn_mfma_kernel<D, 8, kMfmaWaves><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_merge(p, D, pairs, st);
}

}  // namespace

AttnPlan plan_attention(const Dims& s, int k, int m, int proxies, int dense)
{
    AttnPlan pl{};
    pl.exact_rows = dense ? s.n : k * s.L;
    pl.pend = proxies ? s.nb : 0;
    if (s.dtype == DT_BF16) {  // tiles never straddle two segments
        const int pad = kTileRows;
        pl.wbeg = (pl.pend + pad - 1) / pad * pad;
        pl.ebeg = pl.wbeg + (m + pad - 1) / pad * pad;
    } else {
        pl.wbeg = pl.pend;
        pl.ebeg = pl.pend + m;
    }
    pl.rows = pl.ebeg + pl.exact_rows;
    if (pl.exact_rows == 0) pl.rows = m > 0 ? pl.wbeg + m : pl.pend;
    pl.hg = s.G <= 8 ? s.G : 8;
    pl.hchunks = (s.G + pl.hg - 1) / pl.hg;
    if (pl.rows <= 0) {  // empty virtual-token set: nothing to plan (callers reject it)
        pl.splits = 1;
        pl.rows_per_split = 0;
        pl.ws_bytes = 0;
        return pl;
    }
    const int items = s.pairs() * pl.hchunks;
    int tile, splits, max_splits;
    if (s.dtype == DT_F32) {
        tile = 64 / (s.d * 4 / 16) * unroll_for(pl.hg);  // rows per wave iteration
        max_splits = (pl.rows + tile - 1) / tile;
        splits = (kTargetWorkgroups + items - 1) / items;
    } else {
        // one workgroup per (KV head, head chunk) unless that leaves CUs idle or a
        // wave would stream more than kMfmaTilesPerWave tiles; never less than a
        // tile per wave
        tile = kTileRows;
        const int tiles = (pl.rows + tile - 1) / tile;
        max_splits = (tiles + kMfmaWaves - 1) / kMfmaWaves;
        const int for_cus = (kMfmaMinWgs + items - 1) / items;
        const int for_len = (tiles + kMfmaWaves * kMfmaTilesPerWave - 1) / (kMfmaWaves * kMfmaTilesPerWave);
        splits = for_cus > for_len ? for_cus : for_len;
    }
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    int per = (pl.rows + splits - 1) / splits;
    per = (per + tile - 1) / tile * tile;
    const int cap = kMaxSplitRows / tile * tile;
    if (per > cap) per = cap;
    pl.rows_per_split = per;
    pl.splits = (pl.rows + per - 1) / per;
    pl.ws_bytes = pl.splits > 1 ? (size_t)s.pairs() * pl.splits * s.G * (s.d + 2) * sizeof(float) : 0;
    // a tile or two per wave: copying the selection and the weighted tokens to
    // LDS first would cost a barrier and a memory round trip that the few tiles
    // cannot amortise
    pl.direct = s.dtype == DT_BF16 && !dense && k <= kDirectMaxK && pl.rows_per_split <= 2 * kMfmaWaves * kTileRows;
    return pl;
}

hipError_t launch_attention(const Dims& s, const AttnPlan& pl, const AttnInputs& in, void* ws, hipStream_t st)
{
    AttnParams p{};
    p.q = static_cast<const char*>(in.q);
    p.K = static_cast<const char*>(in.K);
    p.V = static_cast<const char*>(in.V);
    p.Kbar = static_cast<const char*>(in.Kbar);
    p.Vbar = static_cast<const char*>(in.Vbar);
    p.sel = in.sel;
    p.tok_idx = in.tok_idx;
    p.tok_logw = in.tok_logw;
    if (pl.direct && in.cand_score) {
        p.cand_score = in.cand_score;
        p.cand_idx = in.cand_idx;
        p.ncand = in.ncand;
        p.sel_out = in.sel_out;
    }
    if (pl.direct && in.proxies && s.nb % 4 == 0 && pl.hg > 4 && s.G <= 8) p.plog = in.plog;
    p.out = in.out;
    p.lse = in.lse;
    p.part = static_cast<float*>(ws);
    p.k = in.k;
    p.m = in.m;
    p.proxies = in.proxies;
    p.dense = in.dense;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.n = s.n;
    p.L = s.L;
    p.nb = s.nb;
    p.rows = pl.rows;
    p.exact_rows = pl.exact_rows;
    p.pend = pl.pend;
    p.wbeg = pl.wbeg;
    p.ebeg = pl.ebeg;
    p.direct = pl.direct;
    p.splits = pl.splits;
    p.rows_per_split = pl.rows_per_split;
    p.scale_log2 = s.scale * kLog2e;
    p.log2_L = s.ln_L * kLog2e;
    p.log2_last = s.ln_last * kLog2e;
    const int pairs = s.pairs();
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_bf16<128>(p, pl.hg, pairs, pl.hchunks, st);
        if (s.d == 64) return launch_bf16<64>(p, pl.hg, pairs, pl.hchunks, st);
    } else {
        if (s.d == 128) return launch_f32<128>(p, pl.hg, pairs, pl.hchunks, st);
        if (s.d == 64) return launch_f32<64>(p, pl.hg, pairs, pl.hchunks, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa

// score.hip -- block scores used to choose the blocks read exactly.
//
// Per query head h and block b ("COBS: Cumulant Order Block Sparse
// Attention"):
//   summary mode, Eq. (18) with phi_b = mean key, a_b = ln c_b:
//       l_hb = scale q_h . Kbar_b + ln c_b
//   exact-mass mode, Eq. (1) (the OSA diagnostic reads every key):
//       l_hb = ln m_hb = ln sum_{i in b} exp(scale q_h . K_i)
// and per KV head, Eq. (5): G = 1 ranks by l_hb itself; G > 1 ranks by
//       ln sum_{h in group} exp(l_hb - ln sum_b' exp(l_hb'))
// i.e. the logarithm of the sum of per-head normalised masses, which keeps
// the ranking of Eq. (5) and cannot underflow.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kNW = 4;

constexpr int score_unroll(int hg) { return hg <= 4 ? 8 : 4; }

struct LogitParams {
    const char* q;
    const char* keys;   // Kbar [pairs, nb, d] or K [pairs, n, d]
    float* dst;         // [B, Hq, nb] (G > 1) or scores [B, Hkv, nb] (G == 1)
    int Hq, Hkv, G, n, L, nb;
    int items_per_wg;   // summary: rows per workgroup; exact: blocks per workgroup
    int chunks;         // workgroups per KV head
    float scale;        // natural units (summary logits)
    float ln_L, ln_last;
    float scale_log2;   // base-2 units (exact-mass log-sum-exp)
};

// Load the query fragments of the chunk's heads (zeros for inactive slots).
template <int DT, int EPL, int HG>
__device__ __forceinline__ void load_q(const LogitParams& p, int b, int h0, int nh, int li, float (&qf)[HG][EPL],
                                       int D)
{
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
}

// Summary-mode logits: one virtual row per block summary.
template <int DT, int D, int HG, int U>
__global__ void __launch_bounds__(kNW * 64) logits_summary_kernel(const LogitParams p)
{
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    constexpr int T = RPW * U;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const int pair = blockIdx.x / p.chunks, chunk = blockIdx.x - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int g0 = blockIdx.y * HG, nh = min(HG, p.G - g0), h0 = j * p.G + g0;
    float qf[HG][EPL];
    load_q<DT, EPL, HG>(p, b, h0, nh, li, qf, D);

    const int r0 = chunk * p.items_per_wg, r1 = min(p.nb, r0 + p.items_per_wg);
    const char* base_ptr = p.keys + (size_t)pair * p.nb * RB + li * 16;
    for (int base = r0 + wave * T; base < r1; base += kNW * T) {
        uint4 kr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = min(base + u * RPW + gi, r1 - 1);
            kr[u] = ld16(base_ptr + (size_t)r * RB);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * RPW + gi;
            float kf[EPL];
            unpack<DT>(kr[u], kf);
            float mine = 0.0f;
#pragma unroll
            for (int g = 0; g < HG; ++g) {
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) s = fmaf(qf[g][e], kf[e], s);
                s = group_sum<LPR>(s);
                if (li == g) mine = s;
            }
            // lane li of the row writes head li (natural-log units)
            if (r < r1 && li < nh) {
                const float v = fmaf(mine, p.scale, r == p.nb - 1 ? p.ln_last : p.ln_L);
                const size_t at = p.G == 1 ? (size_t)pair * p.nb + r : ((size_t)b * p.Hq + h0 + li) * p.nb + r;
                p.dst[at] = v;
            }
        }
    }
}

// Box logits: scale * sum_t max(q_t lo_bt, q_t hi_bt), the largest logit any
// point of block b's key box [lo_b, hi_b] could give (Kbox rows 2b and 2b + 1).
template <int DT, int D, int HG, int U>
__global__ void __launch_bounds__(kNW * 64) logits_box_kernel(const LogitParams p)
{
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    constexpr int T = RPW * U;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const int pair = blockIdx.x / p.chunks, chunk = blockIdx.x - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int g0 = blockIdx.y * HG, nh = min(HG, p.G - g0), h0 = j * p.G + g0;
    float qf[HG][EPL];
    load_q<DT, EPL, HG>(p, b, h0, nh, li, qf, D);

    const int r0 = chunk * p.items_per_wg, r1 = min(p.nb, r0 + p.items_per_wg);
    const char* base_ptr = p.keys + (size_t)pair * 2 * p.nb * RB + li * 16;
    for (int base = r0 + wave * T; base < r1; base += kNW * T) {
        uint4 lr[U], hr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = min(base + u * RPW + gi, r1 - 1);
            lr[u] = ld16(base_ptr + (size_t)(2 * r) * RB);
            hr[u] = ld16(base_ptr + (size_t)(2 * r + 1) * RB);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * RPW + gi;
            float lf[EPL], hf[EPL];
            unpack<DT>(lr[u], lf);
            unpack<DT>(hr[u], hf);
            float mine = 0.0f;
#pragma unroll
            for (int g = 0; g < HG; ++g) {
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) s += fmaxf(qf[g][e] * lf[e], qf[g][e] * hf[e]);
                s = group_sum<LPR>(s);
                if (li == g) mine = s;
            }
            if (r < r1 && li < nh) {
                const size_t at = p.G == 1 ? (size_t)pair * p.nb + r : ((size_t)b * p.Hq + h0 + li) * p.nb + r;
                p.dst[at] = mine * p.scale;
            }
        }
    }
}

// Exact-mass logits: each wave reduces whole blocks (log-sum-exp of the
// block's token logits).
template <int DT, int D, int HG, int U>
__global__ void __launch_bounds__(kNW * 64) logits_exact_kernel(const LogitParams p)
{
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    constexpr int T = RPW * U;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const int pair = blockIdx.x / p.chunks, chunk = blockIdx.x - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int g0 = blockIdx.y * HG, nh = min(HG, p.G - g0), h0 = j * p.G + g0;
    float qf[HG][EPL];
    load_q<DT, EPL, HG>(p, b, h0, nh, li, qf, D);

    const char* base_ptr = p.keys + (size_t)pair * p.n * RB + li * 16;
    const int blk0 = chunk * p.items_per_wg, blk1 = min(p.nb, blk0 + p.items_per_wg);
    for (int blk = blk0 + wave; blk < blk1; blk += kNW) {
        const int t0 = blk * p.L, t1 = min(p.n, t0 + p.L);
        float m_[HG], l_[HG];
#pragma unroll
        for (int g = 0; g < HG; ++g) {
            m_[g] = kNegInf;
            l_[g] = 0.0f;
        }
        for (int base = t0; base < t1; base += T) {
            uint4 kr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int t = min(base + u * RPW + gi, t1 - 1);
                kr[u] = ld16_nt(base_ptr + (size_t)t * RB);
            }
            float x[U][HG];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool ok = base + u * RPW + gi < t1;
                float kf[EPL];
                unpack<DT>(kr[u], kf);
#pragma unroll
                for (int g = 0; g < HG; ++g) {
                    float s = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) s = fmaf(qf[g][e], kf[e], s);
                    s = group_sum<LPR>(s);
                    x[u][g] = ok ? s * p.scale_log2 : kNegInf;
                }
            }
#pragma unroll
            for (int g = 0; g < HG; ++g) {
                float mx = m_[g];
#pragma unroll
                for (int u = 0; u < U; ++u) mx = fmaxf(mx, x[u][g]);
                float acc = l_[g] * rescale(m_[g], mx);
#pragma unroll
                for (int u = 0; u < U; ++u) acc += x[u][g] == kNegInf ? 0.0f : exp2_(x[u][g] - mx);
                l_[g] = acc;
                m_[g] = mx;
            }
        }
        // merge the lane groups of the wave
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int g = 0; g < HG; ++g) {
                const float mo = __shfl_xor(m_[g], off), lo = __shfl_xor(l_[g], off);
                const float mn = fmaxf(m_[g], mo);
                l_[g] = l_[g] * rescale(m_[g], mn) + lo * rescale(mo, mn);
                m_[g] = mn;
            }
        }
        float mine = 0.0f;
#pragma unroll
        for (int g = 0; g < HG; ++g)
            if (lane == g) mine = (m_[g] + log2f(l_[g])) * kLn2;
        if (lane < nh) {
            const size_t at = p.G == 1 ? (size_t)pair * p.nb + blk : ((size_t)b * p.Hq + h0 + lane) * p.nb + blk;
            p.dst[at] = mine;
        }
    }
}

// Exact-mass logits on the matrix cores (bfloat16, G <= 16, L a multiple of
// 32): ln m_{h,b} = log-sum-exp over the block's tokens of scale * q_h . K_i.
// A wave streams the 32-token key tiles of its blocks (two tiles in flight;
// whole rows with the non-temporal hint, 102.8 against 110.0 us per GQA
// exact-mass step with the keys loaded in the operand layout),
// q K^T of a tile is two 16x16x32 MFMA chains (tokens x heads), and each
// output lane keeps an online (max, sum) for its head over its rows; at the
// end of a block the four row groups of a head are merged with lane swaps.
constexpr int kExactWaves = 4;

template <int D>
__global__ void __launch_bounds__(kExactWaves * 64) logits_exact_mfma_kernel(const LogitParams p)
{
    constexpr int RB = D * 2, KS = D / 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, g16 = lane >> 4;
    // workgroup w (on XCD w mod 8) takes item (w mod 8) N / 8 + w / 8: each XCD
    // scans a contiguous eighth of the keys (exact-mass step over 32 KV heads of 8
    // sequences 348.4 -> 340.3 us; no change over 8 KV heads)
    const int wg = gridDim.x % 8 == 0 ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8)
                                      : (int)blockIdx.x;
    const int pair = wg / p.chunks, chunk = wg - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    // this wave's blocks: a contiguous share of the chunk's
    const int blk0 = chunk * p.items_per_wg, blk1 = min(p.nb, blk0 + p.items_per_wg);
    const int per_wave = (blk1 - blk0 + kExactWaves - 1) / kExactWaves;
    const int wb0 = blk0 + wave * per_wave, wb1 = min(blk1, wb0 + per_wave);
    if (wb0 >= wb1) return;  // whole wave; no barrier in this kernel
    const int tpb = p.L / 32;  // tiles per block
    const int t0 = wb0 * tpb, t1 = wb1 * tpb;

    bf16x8_t bq[KS];
    load_q_operand<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bq);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.keys + (size_t)pair * p.n * RB, (uint32_t)p.n * RB);

    // Every tile load is issued unconditionally (a tile past the wave's share
    // reads through an empty buffer: zeros, no memory traffic) and the loop
    // has no exit between its two halves, so that the compiler's wait before a
    // tile's MFMAs covers that tile's loads only, not the next tile's too.
    const __amdgpu_buffer_rsrc_t none = buffer_rsrc(p.keys, 0u);
    // Key rows are loaded whole (LPV lanes per row, RPV rows per instruction)
    // with the non-temporal hint, then moved into the MFMA operand layout
    // through a per-wave LDS slot of 16 rows padded to LPV + 1 chunks.
    constexpr int LPV = RB / 16, RPV = 64 / LPV, NI = 32 / RPV;
    static_assert(RPV * NI / 2 == 16, "half a tile's loads cover one 16-row MFMA block");
    __shared__ uint4 slot_all[kExactWaves][16 * (LPV + 1)];
    uint4* const slot = slot_all[wave];
    const int gv = lane / LPV, cv = lane % LPV;
    auto load = [&](int t, uint4 (&ak)[NI]) {
        const __amdgpu_buffer_rsrc_t r = t < t1 ? kr : none;
#pragma unroll
        for (int jj = 0; jj < NI; ++jj)
            ak[jj] = buffer_ld16_nt(r, (uint32_t)(t * 32 + RPV * jj + gv) * RB + cv * 16);  // past n: zeros
    };
    float m_run = kNegInf, l_run = 0.0f;  // this lane's head n16, its rows of the current block
    auto consume = [&](int t, const uint4 (&ak)[NI]) {
        f32x4_t c[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int jj = 0; jj < NI / 2; ++jj) slot[(RPV * jj + gv) * (LPV + 1) + cv] = ak[rb * (NI / 2) + jj];
            wave_lds_fence();
            uint4 a[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) a[s] = slot[n16 * (LPV + 1) + 4 * s + g16];
            wave_lds_fence();  // the slot is rewritten next
#pragma unroll
            for (int s = 0; s < KS; ++s)
                c[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[s]), bq[s], c[rb], 0, 0, 0);
        }
        float x[8];
        float mx = m_run;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = t * 32 + rb * 16 + 4 * g16 + i;
                x[rb * 4 + i] = row < p.n ? c[rb][i] * p.scale_log2 : kNegInf;
                mx = fmaxf(mx, x[rb * 4 + i]);
            }
        float acc = l_run * rescale(m_run, mx);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += x[e] == kNegInf ? 0.0f : exp2_(x[e] - mx);
        m_run = mx;
        l_run = acc;
        if ((t + 1) % tpb == 0) {  // block complete: merge the four row groups of each head
#pragma unroll
            for (int level = 0; level < 2; ++level) {
                const LanePair pm = level == 0 ? swap16(__float_as_uint(m_run)) : swap32(__float_as_uint(m_run));
                const LanePair pl = level == 0 ? swap16(__float_as_uint(l_run)) : swap32(__float_as_uint(l_run));
                const float ma = __uint_as_float(pm.a), mb = __uint_as_float(pm.b);
                const float mn = fmaxf(ma, mb);
                l_run = __uint_as_float(pl.a) * rescale(ma, mn) + __uint_as_float(pl.b) * rescale(mb, mn);
                m_run = mn;
            }
            const int blk = t / tpb;
            if (g16 == 0 && n16 < p.G) {
                const size_t at = p.G == 1 ? (size_t)pair * p.nb + blk : ((size_t)b * p.Hq + j * p.G + n16) * p.nb + blk;
                p.dst[at] = (m_run + log2f(l_run)) * kLn2;
            }
            m_run = kNegInf;
            l_run = 0.0f;
        }
    };
    uint4 A[NI], B[NI];
    load(t0, A);
    load(t0 + 1, B);
    int t = t0;
    for (; t + 1 < t1; t += 2) {
        consume(t, A);
        load(t + 2, A);
        consume(t + 1, B);
        load(t + 3, B);
    }
    if (t < t1) consume(t, A);
}

// Group score per KV head from the per-head logits [B, Hq, nb] (G > 1).
__global__ void __launch_bounds__(256) group_score_kernel(const float* logits, float* scores, int Hq, int Hkv,
                                                         int G, int nb)
{
    extern __shared__ float sm[];  // [G] per-head log normaliser, then [8] scratch
    float* lse_h = sm;
    float* red = sm + G;
    const int pair = blockIdx.x, b = pair / Hkv, j = pair - b * Hkv;
    const float* first = logits + ((size_t)b * Hq + (size_t)j * G) * nb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int g = 0; g < G; ++g) {
        const float* row = first + (size_t)g * nb;
        float mx = kNegInf;
        for (int i = threadIdx.x; i < nb; i += 256) mx = fmaxf(mx, row[i]);
        for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if (lane == 0) red[wave] = mx;
        __syncthreads();
        mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        __syncthreads();
        float s = 0.0f;
        for (int i = threadIdx.x; i < nb; i += 256) s += exp2_((row[i] - mx) * kLog2e);
        for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
        if (lane == 0) red[4 + wave] = s;
        __syncthreads();
        if (threadIdx.x == 0) lse_h[g] = mx + logf((red[4] + red[5]) + (red[6] + red[7]));
        __syncthreads();
    }
    for (int i = threadIdx.x; i < nb; i += 256) {
        float mx = kNegInf;
        for (int g = 0; g < G; ++g) mx = fmaxf(mx, first[(size_t)g * nb + i] - lse_h[g]);
        float s = 0.0f;
        for (int g = 0; g < G; ++g) s += exp2_((first[(size_t)g * nb + i] - lse_h[g] - mx) * kLog2e);
        scores[(size_t)pair * nb + i] = mx + logf(s);
    }
}


// ---------------------------------------------------------------------------
// Summary mode on the matrix cores.  A tile of 32 blocks of one KV head: the
// mean keys are the A operand of v_mfma_f32_16x16x32_bf16 (two 16-row chains),
// the G query heads the B operand (padded to 16 columns); the logit of head h
// and block b is scale * (q_h . Kbar_b) + ln c_b.
//   * fused: one workgroup per KV head keeps all its logits in LDS, then the
//     per-head log-normalisers and the group scores (many KV heads);
//   * split: the tiles of a KV head spread over several workgroups that write
//     the logits to a workspace, then one workgroup per KV head finishes the
//     group scores and, for the decode step, the top-k (few KV heads).
// Both produce the same bits.
// ---------------------------------------------------------------------------

constexpr int kFusedWaves = 8;
constexpr int kFusedMaxLogits = 16384;  // G * nb floats in LDS
static_assert(kFusedMaxLogits / 2 / 32 <= 4 * 64, "the group-score kernel merges up to 256 tile states per head");
constexpr int kSplitWaves = 4;          // waves (one tile each) per workgroup of the split logits kernel
constexpr int kFinishMaxK = 32;
constexpr int kFinishMaxBlocks = 2048;  // top-k by one wave: up to 32 scores per lane
static_assert(kCandChunk % 64 == 0 && kCandChunk <= 128, "candidate chunks of one or two blocks per lane");

struct FusedScoreParams {
    const char* q;
    const char* Kbar;
    float* scores;
    float* logits;  // split: [B, Hq, nb] (the scores when G == 1)
    int32_t* sel;   // finish: selection [B, Hkv, k] when k > 0
    float* parts;   // split kernels: per (KV head, tile, head) log2 (max, sum) of the logits (may be null)
    const int32_t* offsets;  // clusters: ranges [B, Hkv, nb + 1] give the count terms (else blocks)
    const float* U;          // query-subspace descriptors: the basis [Hkv, d, s]
    int s_dim, sps;          // its dimension s and the stored factor length (s rounded up to 8)
    int Hq, Hkv, G, nb, k, chunks;
    float scale, ln_L, ln_last;
};

// ln of the token count of row r: a block's (ln L, or the last block's), or a
// cluster's from its range (-inf when empty).  off: this KV head's ranges or null.
__device__ __forceinline__ float count_term(const FusedScoreParams& p, const int32_t* off, int r)
{
    if (off) {
        const int c = off[r + 1] - off[r];
        return c > 0 ? logf((float)c) : kNegInf;
    }
    return r == p.nb - 1 ? p.ln_last : p.ln_L;
}

// Merge the online log-sum-exp states of the four lane groups holding one head:
// lanes n16, n16 + 16, n16 + 32, n16 + 48.
__device__ __forceinline__ void merge_lse_groups(float& m2, float& s2)
{
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const LanePair pm = r == 0 ? swap16(__float_as_uint(m2)) : swap32(__float_as_uint(m2));
        const LanePair ps = r == 0 ? swap16(__float_as_uint(s2)) : swap32(__float_as_uint(s2));
        const float ma = __uint_as_float(pm.a), mb = __uint_as_float(pm.b);
        const float mn = fmaxf(ma, mb);
        s2 = __uint_as_float(ps.a) * rescale(ma, mn) + __uint_as_float(ps.b) * rescale(mb, mn);
        m2 = mn;
    }
}

// The mean keys of the tile of blocks [base, base + 32), loaded whole (LPV
// lanes per row, RPV rows per load) with the non-temporal hint: kr[j] holds
// chunk lane % LPV of row RPV j + lane / LPV.  Rows past nb read as zeros.
template <int D>
struct KeyTile {
    static constexpr int RB = D * 2, LPV = RB / 16, RPV = 64 / LPV, NI = 32 / RPV;
    static_assert(RPV * NI / 2 == 16, "half a tile's loads cover one 16-row MFMA block");
    uint4 kr[NI];
};

// A wave's LDS slot for the layout change of a key tile: 16 rows padded to
// LPV + 1 chunks (the lanes of a whole-row write and of an operand read hit
// different banks).
template <int D>
constexpr int kKeySlot = 16 * (D * 2 / 16 + 1);

template <int D>
__device__ __forceinline__ void load_key_tile(__amdgpu_buffer_rsrc_t kr, int base, int lane, KeyTile<D>& t)
{
    using T = KeyTile<D>;
    const int gv = lane / T::LPV, cv = lane % T::LPV;
#pragma unroll
    for (int jj = 0; jj < T::NI; ++jj)
        t.kr[jj] = buffer_ld16_nt(kr, (uint32_t)(base + T::RPV * jj + gv) * T::RB + cv * 16);
}

// The tile's 16-row block rb in the A-operand layout (lane (n16, g16): row n16,
// 16-byte chunks 4 s + g16), through the wave's slot.
template <int D>
__device__ __forceinline__ void key_tile_operand(const KeyTile<D>& t, int rb, int lane, uint4* slot, uint4 (&a)[D / 32])
{
    using T = KeyTile<D>;
    const int gv = lane / T::LPV, cv = lane % T::LPV, n16 = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int jj = 0; jj < T::NI / 2; ++jj) slot[(T::RPV * jj + gv) * (T::LPV + 1) + cv] = t.kr[rb * (T::NI / 2) + jj];
    wave_lds_fence();
#pragma unroll
    for (int s = 0; s < D / 32; ++s) a[s] = slot[n16 * (T::LPV + 1) + 4 * s + g16];
    wave_lds_fence();  // the slot is rewritten next
}

// Logits of a loaded tile for every head of the group: dst[h * stride + b].
// With `track`, each output lane also folds its logits (in log2 units) into an
// online log-sum-exp state (m2, s2) of its head.
template <int D>
__device__ __forceinline__ void key_tile_logits(const FusedScoreParams& p, const KeyTile<D>& t,
                                                const bf16x8_t (&bq)[D / 32], int base, float* dst, int stride,
                                                int lane, const int32_t* off, bool track, float& m2, float& s2,
                                                uint4* slot)
{
    constexpr int KS = D / 32;
    const int n16 = lane & 15, g16 = lane >> 4;
    f32x4_t c[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        uint4 a[KS];
        key_tile_operand<D>(t, rb, lane, slot, a);
#pragma unroll
        for (int s = 0; s < KS; ++s)
            c[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[s]), bq[s], c[rb], 0, 0, 0);
    }
    if (n16 < p.G) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = base + rb * 16 + 4 * g16 + i;
                if (row < p.nb) {
                    const float v = fmaf(c[rb][i], p.scale, count_term(p, off, row));
                    dst[n16 * stride + row] = v;
                    if (track && v > kNegInf) {
                        const float t2 = v * kLog2e;
                        const float mn = fmaxf(m2, t2);
                        s2 = s2 * rescale(m2, mn) + exp2_(t2 - mn);
                        m2 = mn;
                    }
                }
            }
    }
}

template <int D>
__device__ __forceinline__ void key_tile_logits(const FusedScoreParams& p, const KeyTile<D>& t,
                                                const bf16x8_t (&bq)[D / 32], int base, float* dst, int stride,
                                                int lane, const int32_t* off, uint4* slot)
{
    float m2 = kNegInf, s2 = 0.0f;
    key_tile_logits<D>(p, t, bq, base, dst, stride, lane, off, false, m2, s2, slot);
}

// Group scores of one KV head from its logits lsm[h * nb + b] in LDS, by the
// whole workgroup (NW waves): written to lsm[b] (row 0, in place: block b's
// column is read only by the thread that writes it) and to scores when given.
template <int NW>
__device__ __forceinline__ void group_scores_in_lds(float* lsm, float* lse_h, int G, int nb, float* scores,
                                                    bool lse_given = false)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (G > 1 && !lse_given) {
        for (int h = wave; h < G; h += NW) {
            const float lse = head_lse(lsm + h * nb, nb, lane);
            if (lane == 0) lse_h[h] = lse;
        }
        __syncthreads();
    }
    if (nb <= NW * 64) {  // a block per thread at most
        const int i = threadIdx.x;
        if (i < nb) {
            const float v = G == 1 ? lsm[i] : group_score<8>(lsm + i, nb, lse_h, G);
            lsm[i] = v;
            if (scores) scores[i] = v;
        }
        return;
    }
    // four blocks per thread at a time, their reads issued together
    constexpr int U = 4;
    for (int i0 = threadIdx.x; i0 < nb; i0 += U * NW * 64) {
        float v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = min(i0 + u * NW * 64, nb - 1);
            v[u] = G == 1 ? lsm[i] : group_score<8>(lsm + i, nb, lse_h, G);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = i0 + u * NW * 64;
            if (i < nb) {
                lsm[i] = v[u];
                if (scores) scores[i] = v[u];
            }
        }
    }
}

// The query operand of the block-logit product.  Summary rows (D = d): q
// itself.  Box rows (D = 2d, the block's [minimum | maximum] keys): the vector
// [min(q, 0) | max(q, 0)], since per coordinate max(q lo, q hi) is q hi when
// q >= 0 and q lo otherwise, so the best logit over the box is one dot product.
template <int D, bool BOX>
__device__ __forceinline__ void load_score_q(const char* q_first_head, int nh, int lane, bf16x8_t (&bq)[D / 32])
{
    if constexpr (!BOX) {
        load_q_operand<D>(q_first_head, nh, lane, bq);
    } else {
        constexpr int DQ = D / 2;  // head_dim
        const int n16 = lane & 15, g16 = lane >> 4;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
            const int c = 4 * s + g16;  // 16-byte chunk of the 2d-vector
            const bool low_half = c < DQ / 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (n16 < nh) v = ld16(q_first_head + (size_t)n16 * DQ * 2 + (low_half ? c : c - DQ / 8) * 16);
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t neg = ((w[i] & 0x80008000u) >> 15) * 0xffffu;  // bfloat16 lanes with the sign set
                w[i] &= low_half ? neg : ~neg;
            }
            bq[s] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
    }
}

// LDS of the selection of one KV head by NW waves.
template <int NW>
struct SelectSmem {
    uint32_t cand[NW][128];              // per-wave scratch of the one-wave ranking
    uint32_t topk[2 * NW + 128];         // wave maxima, overflow flags, candidate slots
    int32_t cidx[NW * kFinishMaxK];      // two-level: the waves' candidates, ascending block index
};

// The top-k (k <= 32) of the nb <= 2048 scores lsm[0 .. nb) of one KV head, by
// the whole workgroup (NW waves), to out[0 .. k) in ascending index order.
// Up to one score per thread, the waves' maxima bound the search.  Beyond, each
// wave ranks its contiguous share of the blocks (its k best), then one wave
// ranks the NW k candidates: they lie in ascending block order, so ranking by
// position breaks ties towards the lower block like ranking by index, and the
// k best of the union are the k best overall.
template <int NW>
__device__ __forceinline__ void select_in_lds(const float* lsm, int nb, int k, int32_t* out, SelectSmem<NW>& ss)
{
    const int lane = threadIdx.x & 63;
    auto emit = [&](int r, int idx) { out[r] = idx; };
    if (nb <= NW * 64) {
        auto one_wave_topk = [&]() { wave_topk<8>([&](int i) { return lsm[i]; }, nb, k, lane, ss.cand[0], emit); };
        uint32_t key[1] = {(int)threadIdx.x < nb ? order_key(lsm[threadIdx.x]) : 0u};
        block_topk<NW, 1>(key, nb, k, ss.topk, one_wave_topk, emit);
        return;
    }
    static_assert(kFinishMaxBlocks <= NW * 4 * 64 && NW * kFinishMaxK <= 4 * 64, "four scores per lane");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per = (nb + NW - 1) / NW;
    auto share = [&](int w) { return min(per, max(0, nb - w * per)); };
    int base = 0, total = 0;  // this wave's first candidate slot; all candidates
    for (int w = 0; w < NW; ++w) {
        const int c = min(k, share(w));
        if (w < wave) base += c;
        total += c;
    }
    const int lo = wave * per, kw = min(k, share(wave));
    if (kw > 0)
        wave_topk<4>([&](int i) { return lsm[lo + i]; }, share(wave), kw, lane, ss.cand[wave],
                     [&](int r, int i) { ss.cidx[base + r] = lo + i; });
    __syncthreads();
    if (wave == 0)
        wave_topk<4>([&](int i) { return lsm[ss.cidx[i]]; }, total, k, lane, ss.cand[0],
                     [&](int r, int i) { out[r] = ss.cidx[i]; });
}

template <int D, bool BOX>
__global__ void __launch_bounds__(kFusedWaves * 64) score_summary_fused_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, NW = kFusedWaves, QB = BOX ? D : RB;  // QB: bytes per query row
    extern __shared__ float lsm[];  // [G][nb] block logits
    __shared__ float lse_h[8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __shared__ SelectSmem<NW> ss;
    __shared__ uint4 kslot[NW][kKeySlot<D>];
    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int32_t* off = p.offsets ? p.offsets + (size_t)pair * (p.nb + 1) : nullptr;

    bf16x8_t bq[KS];
    load_score_q<D, BOX>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * QB, p.G, lane, bq);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * RB, (uint32_t)p.nb * RB);
    for (int base = wave * 32; base < p.nb; base += 2 * NW * 32) {  // two tiles in flight
        KeyTile<D> t0, t1;
        const int base1 = base + NW * 32;
        load_key_tile<D>(kr, base, lane, t0);
        load_key_tile<D>(kr, base1, lane, t1);  // past nb: zeros, no memory traffic
        key_tile_logits<D>(p, t0, bq, base, lsm, p.nb, lane, off, kslot[wave]);
        if (base1 < p.nb) key_tile_logits<D>(p, t1, bq, base1, lsm, p.nb, lane, off, kslot[wave]);
    }
    __syncthreads();
    group_scores_in_lds<NW>(lsm, lse_h, p.G, p.nb, p.scores ? p.scores + (size_t)pair * p.nb : nullptr);
    if (p.k > 0) {
        __syncthreads();
        select_in_lds<NW>(lsm, p.nb, p.k, p.sel + (size_t)pair * p.k, ss);
    }
}

// Split logits: workgroup (pair, chunk) computes tiles chunk * kSplitWaves + wave.
template <int D, bool BOX>
__global__ void __launch_bounds__(kSplitWaves * 64) score_logits_split_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, QB = BOX ? D : RB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // each XCD takes a contiguous eighth of the (pair, chunk) items, as in the
    // exact-mass scan (128K weighted-coreset step 25.62 -> 25.03 us)
    const int wg = gridDim.x % 8 == 0 ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8)
                                      : (int)blockIdx.x;
    const int pair = wg / p.chunks, chunk = wg - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int base = (chunk * kSplitWaves + wave) * 32;
    if (base >= p.nb) return;  // whole wave; no barrier in this kernel
    __shared__ uint4 kslot[kSplitWaves][kKeySlot<D>];
    bf16x8_t bq[KS];
    load_score_q<D, BOX>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * QB, p.G, lane, bq);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * RB, (uint32_t)p.nb * RB);
    KeyTile<D> t;
    load_key_tile<D>(kr, base, lane, t);
    float m2 = kNegInf, s2 = 0.0f;
    key_tile_logits<D>(p, t, bq, base, p.logits + (size_t)pair * p.G * p.nb, p.nb, lane,
                       p.offsets ? p.offsets + (size_t)pair * (p.nb + 1) : nullptr, p.parts != nullptr, m2, s2,
                       kslot[wave]);
    if (p.parts) {  // this tile's log-sum-exp state per head, for the group-score kernel's normalisers
        merge_lse_groups(m2, s2);
        if (lane < 8) {
            const int tiles = (p.nb + 31) / 32;
            float* dst = p.parts + (((size_t)pair * tiles + base / 32) * 8 + lane) * 2;
            dst[0] = m2;
            dst[1] = s2;
        }
    }
}

// Second-order logits (COBS, cumulant expansion of ln m_b truncated at second
// order): scale q.kbar_b + ln c_b + (1/2) scale^2 sum_i (q.xi_bi)^2 from the
// descriptor rows Kcov [.., nb, 1 + kCobsRank, d].  For a tile of 32 blocks
// [base, base + 32): the mean rows (tile row r -> block base + r) and four
// sub-tiles of 8 blocks x 4 eigenvector rows (tile row r -> block
// base + 8 u + r / 4, eigenvector r % 4), all through the same MFMA; an output
// lane of a sub-tile holds the four eigenvector products of one block, so the
// sum of squares needs no lane exchange.  The two parts meet in a per-wave LDS
// tile tmp[8 heads][32 blocks] and go to dst[h * stride + b].
template <int D>
__device__ __forceinline__ void cobs2_tile_logits(const FusedScoreParams& p, __amdgpu_buffer_rsrc_t kr,
                                                  const bf16x8_t (&bq)[D / 32], int base, float* dst, int stride,
                                                  int lane, float (*tmp)[32], uint4* slot)
{
    constexpr int RB = D * 2, KS = D / 32, NR = 1 + kCobsRank;
    static_assert(kCobsRank == 4, "one output lane holds one block's four eigenvector products");
    // The tile's 32 NR rows are contiguous: they are loaded whole with the
    // non-temporal hint (LPV lanes per row, RPV rows per load), and each group
    // of 8 blocks goes through the wave's LDS slot (kCobsSlot rows: the 32
    // eigenvector rows in sub-tile order, then the 8 mean rows) into the
    // operand layout.
    constexpr int LPV = RB / 16, RPV = 64 / LPV, NG = 8 * NR / RPV;
    static_assert(8 * NR % RPV == 0, "whole loads per group of 8 blocks");
    const int n16 = lane & 15, g16 = lane >> 4, gv = lane / LPV, ck = lane % LPV;
    uint4 rows[4][NG];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int jj = 0; jj < NG; ++jj)  // past nb: zeros
            rows[u][jj] = buffer_ld16_nt(kr, (uint32_t)((base + 8 * u) * NR + RPV * jj + gv) * RB + ck * 16);
    uint4 am[2][KS];
    float sq[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int jj = 0; jj < NG; ++jj) {
            const int lr = RPV * jj + gv, bl = lr / NR, kind = lr - bl * NR;
            const int pos = kind == 0 ? 32 + bl : 4 * bl + kind - 1;
            slot[pos * (LPV + 1) + ck] = rows[u][jj];
        }
        wave_lds_fence();
        uint4 ax[2][KS];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int s = 0; s < KS; ++s) ax[rb][s] = slot[(rb * 16 + n16) * (LPV + 1) + 4 * s + g16];
        // the mean rows of blocks 8 u .. 8 u + 7: lanes n16 = 8 (u % 2) + i of mean block u / 2
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 v = slot[(32 + (n16 & 7)) * (LPV + 1) + 4 * s + g16];
            if ((n16 >> 3) == (u & 1)) am[u >> 1][s] = v;
        }
        wave_lds_fence();  // the slot is rewritten next
        f32x4_t cx[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                cx[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ax[rb][s]), bq[s], cx[rb], 0,
                                                                 0, 0);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            sq[u][rb] = (cx[rb][0] * cx[rb][0] + cx[rb][1] * cx[rb][1]) + (cx[rb][2] * cx[rb][2] + cx[rb][3] * cx[rb][3]);
    }
    f32x4_t cm[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            cm[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, am[rb][s]), bq[s], cm[rb], 0, 0,
                                                             0);
    if (n16 < p.G) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = rb * 16 + 4 * g16 + i;
                tmp[n16][tr] = fmaf(cm[rb][i], p.scale, base + tr == p.nb - 1 ? p.ln_last : p.ln_L);
            }
    }
    wave_lds_fence();
    const float half_s2 = 0.5f * p.scale * p.scale;
    if (n16 < p.G) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) tmp[n16][8 * u + 4 * rb + g16] += half_s2 * sq[u][rb];
    }
    wave_lds_fence();
    for (int e = lane; e < p.G * 32; e += 64) {
        const int h = e >> 5, b = e & 31;
        if (base + b < p.nb) dst[h * stride + base + b] = tmp[h][b];
    }
    wave_lds_fence();  // tmp is reused by the next tile
}

// Query-subspace descriptors, per block [mean: d bfloat16][4 x sps bfloat16]
// (kv_cov_sub_build).  The query's coordinates in the subspace, qt = U^T q, are
// not bfloat16: each enters the MFMA as two bfloat16 terms (hi + lo, within about
// 2^-17 of the fp32 value), two chains into one accumulator.  Otherwise the tile
// of cobs2_tile_logits, the factor rows KSS k-steps of 32 long (chunks past the
// stored length read as zero).
template <int D, int KSS>
__device__ __forceinline__ void cobs2_sub_tile_logits(const FusedScoreParams& p, __amdgpu_buffer_rsrc_t kr,
                                                      const bf16x8_t (&bq)[D / 32], const bf16x8_t (&bh)[KSS],
                                                      const bf16x8_t (&bl)[KSS], int base, float* dst, int stride,
                                                      int lane, float (*tmp)[32], uint4* gslot)
{
    constexpr int RB = D * 2, KS = D / 32;
    static_assert(kCobsRank == 4, "one output lane holds one block's four factor products");
    const int n16 = lane & 15, g16 = lane >> 4;
    const uint32_t BB = (uint32_t)(RB + kCobsRank * p.sps * 2), nch = (uint32_t)(p.sps / 8);
    // The tile's 32 BB bytes are contiguous (BB a multiple of 64).  Group by group
    // of 8 blocks (two groups in flight), they are loaded 16 bytes per lane (a
    // KiB per load, non-temporal; chunks past the group or past nb read as zeros),
    // copied to the wave's LDS slot, and the lanes' operand chunks taken from there.
    constexpr int NJG = ((RB + kCobsRank * 32 * KSS * 2) * 8 / 16 + 63) / 64;  // loads per lane per group, at most
    const int GC = (int)(8 * BB / 16);  // 16-byte chunks of a group of 8 blocks
    const uint32_t oob = (uint32_t)p.nb * BB;  // the buffer's size: a load there reads zeros
    uint4 vg[2][NJG];
    auto load_group = [&](int u, uint4 (&dstv)[NJG]) {
#pragma unroll
        for (int jj = 0; jj < NJG; ++jj) {
            const int cl = 64 * jj + lane;
            dstv[jj] = buffer_ld16_nt(kr, cl < GC ? (uint32_t)base * BB + (uint32_t)(u * GC + cl) * 16 : oob);
        }
    };
    load_group(0, vg[0]);
    load_group(1, vg[1]);
    const char* const g = reinterpret_cast<const char*>(gslot);
    uint4 am[2][KS];
    float sq[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int jj = 0; jj < NJG; ++jj) {
            const int cl = 64 * jj + lane;
            if (cl < GC) gslot[cl] = vg[u & 1][jj];
        }
        wave_lds_fence();
        uint4 ax[2][KSS];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int tr = rb * 16 + n16;
            const char* x = g + (tr / 4) * BB + RB + (uint32_t)(tr % 4) * p.sps * 2;
#pragma unroll
            for (int s = 0; s < KSS; ++s) {
                const uint32_t c = 4 * s + g16;
                ax[rb][s] = c < nch ? *reinterpret_cast<const uint4*>(x + c * 16) : make_uint4(0, 0, 0, 0);
            }
        }
        // the mean rows of blocks 8 u .. 8 u + 7: lanes n16 = 8 (u % 2) + i of mean block u / 2
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 m = *reinterpret_cast<const uint4*>(g + (n16 & 7) * BB + g16 * 16 + s * 64);
            if ((n16 >> 3) == (u & 1)) am[u >> 1][s] = m;
        }
        wave_lds_fence();  // the slot is rewritten next
        if (u + 2 < 4) load_group(u + 2, vg[u & 1]);
        f32x4_t cx[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int s = 0; s < KSS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ax[rb][s]);
                cx[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[s], cx[rb], 0, 0, 0);
                cx[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[s], cx[rb], 0, 0, 0);
            }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            sq[u][rb] = (cx[rb][0] * cx[rb][0] + cx[rb][1] * cx[rb][1]) + (cx[rb][2] * cx[rb][2] + cx[rb][3] * cx[rb][3]);
    }
    f32x4_t cm[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            cm[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, am[rb][s]), bq[s], cm[rb], 0, 0,
                                                             0);
    if (n16 < p.G) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = rb * 16 + 4 * g16 + i;
                tmp[n16][tr] = fmaf(cm[rb][i], p.scale, base + tr == p.nb - 1 ? p.ln_last : p.ln_L);
            }
    }
    wave_lds_fence();
    const float half_s2 = 0.5f * p.scale * p.scale;
    if (n16 < p.G) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) tmp[n16][8 * u + 4 * rb + g16] += half_s2 * sq[u][rb];
    }
    wave_lds_fence();
    for (int e = lane; e < p.G * 32; e += 64) {
        const int h = e >> 5, b = e & 31;
        if (base + b < p.nb) dst[h * stride + base + b] = tmp[h][b];
    }
    wave_lds_fence();  // tmp is reused by the next tile
}

// FP4 query-subspace descriptors, per block [mean: d bfloat16][4 fp32 scales][4 x
// spf/2 bytes of E2M1 codes] (spf = s rounded up to 32): the tile of
// cobs2_fp4_tile_logits with factor rows of spf coordinates (KSS = spf / 32 code
// words per lane) against qt as two bfloat16 terms in the code words' order.
template <int D, int KSS>
__device__ __forceinline__ void cobs2_sub4_tile_logits(const FusedScoreParams& p, __amdgpu_buffer_rsrc_t kr,
                                                       const bf16x8_t (&bq)[D / 32], const bf16x8_t (&bh)[KSS],
                                                       const bf16x8_t (&bl)[KSS], int base, float* dst, int stride,
                                                       int lane, float (*tmp)[32], uint4* gslot)
{
    constexpr int KS = D / 32, SPF = 32 * KSS;
    constexpr uint32_t BB = 2 * D + 16 + 4 * SPF / 2;
    static_assert(kCobsRank == 4, "one output lane holds one block's four factor products");
    // The tile's 32 BB bytes are contiguous: they are loaded 16 bytes per lane (a
    // KiB per load, non-temporal; chunks past the tile or past nb read as zeros)
    // and each group of 8 blocks is copied to the wave's LDS slot, from which the
    // lanes take their mean-row chunks, code words and scales.
    constexpr int GC = 8 * BB / 16, NJ = (4 * GC + 63) / 64;  // chunks per group; loads per lane
    static_assert(8 * BB % 16 == 0, "groups of whole 16-byte chunks");
    const int n16 = lane & 15, g16 = lane >> 4;
    const uint32_t oob = (uint32_t)p.nb * BB;  // the buffer's size: a load there reads zeros
    uint4 v[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
        const int ci = 64 * jj + lane;
        v[jj] = buffer_ld16_nt(kr, ci < 4 * GC ? (uint32_t)base * BB + (uint32_t)ci * 16 : oob);
    }
    const char* const g = reinterpret_cast<const char*>(gslot);
    uint4 am[2][KS];
    uint32_t ac[4][2][KSS];  // the lane's code words: coordinates 8 (KSS g16 + s) .. + 7
    float4 scl[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int jj = u * GC / 64; jj <= ((u + 1) * GC - 1) / 64; ++jj) {
            const int ci = 64 * jj + lane;
            if (ci >= u * GC && ci < (u + 1) * GC) gslot[ci - u * GC] = v[jj];
        }
        wave_lds_fence();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int tr = rb * 16 + n16;
            const char* c = g + (tr / 4) * BB + 2 * D + 16 + (tr % 4) * (SPF / 2) + g16 * 4 * KSS;
#pragma unroll
            for (int s = 0; s < KSS; ++s) ac[u][rb][s] = *reinterpret_cast<const uint32_t*>(c + 4 * s);
            scl[u][rb] = *reinterpret_cast<const float4*>(g + (4 * rb + g16) * BB + 2 * D);
        }
        // the mean rows of blocks 8 u .. 8 u + 7: lanes n16 = 8 (u % 2) + i of mean block u / 2
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 m = *reinterpret_cast<const uint4*>(g + (n16 & 7) * BB + g16 * 16 + s * 64);
            if ((n16 >> 3) == (u & 1)) am[u >> 1][s] = m;
        }
        wave_lds_fence();  // the slot is rewritten next
    }
    f32x4_t cm[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            cm[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, am[rb][s]), bq[s], cm[rb], 0, 0,
                                                             0);
    float sq[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4_t cx[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int s = 0; s < KSS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const uint32_t w = ac[u][rb][s];
                typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
                const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
                const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
                const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
                const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
                const bf16x8_t a = __builtin_bit_cast(
                    bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                                         __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)));
                cx[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh[s], cx[rb], 0, 0, 0);
                cx[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl[s], cx[rb], 0, 0, 0);
            }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float e0 = cx[rb][0] * scl[u][rb].x, e1 = cx[rb][1] * scl[u][rb].y;
            const float e2 = cx[rb][2] * scl[u][rb].z, e3 = cx[rb][3] * scl[u][rb].w;
            sq[u][rb] = (e0 * e0 + e1 * e1) + (e2 * e2 + e3 * e3);
        }
    }
    if (n16 < p.G) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = rb * 16 + 4 * g16 + i;
                tmp[n16][tr] = fmaf(cm[rb][i], p.scale, base + tr == p.nb - 1 ? p.ln_last : p.ln_L);
            }
    }
    wave_lds_fence();
    const float half_s2 = 0.5f * p.scale * p.scale;
    if (n16 < p.G) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) tmp[n16][8 * u + 4 * rb + g16] += half_s2 * sq[u][rb];
    }
    wave_lds_fence();
    for (int e = lane; e < p.G * 32; e += 64) {
        const int h = e >> 5, b = e & 31;
        if (base + b < p.nb) dst[h * stride + base + b] = tmp[h][b];
    }
    wave_lds_fence();  // tmp is reused by the next tile
}

// qt = U^T q for the G heads of KV head j, by the whole workgroup, into
// qt_sm[h][0 .. 32 KSS) (zeros past s), fp32: a thread per (head, coordinate), the
// d products in four interleaved partial sums with every load of a row of q and
// of a column of U issued together.  The caller synchronises before reading it.
template <int D, int KSS>
__device__ __forceinline__ void subspace_query(const FusedScoreParams& p, const char* q_first_head, int j,
                                               float (*qt_sm)[128])
{
    const float* Uj = p.U + (size_t)j * D * p.s_dim;
    const int sd = p.s_dim;
    for (int e = threadIdx.x; e < p.G * 32 * KSS; e += blockDim.x) {
        const int h = e / (32 * KSS), c = e - h * (32 * KSS);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (c < sd) {
            const uint4* q8 = reinterpret_cast<const uint4*>(q_first_head + (size_t)h * D * 2);
            const float* uc = Uj + c;
#pragma unroll
            for (int t8 = 0; t8 < D / 8; ++t8) {
                float qf[8];
                unpack<DT_BF16>(q8[t8], qf);
#pragma unroll
                for (int e8 = 0; e8 < 8; ++e8) acc[e8 & 3] = fmaf(qf[e8], uc[(size_t)(8 * t8 + e8) * sd], acc[e8 & 3]);
            }
        }
        qt_sm[h][c] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
}

// The B operands of qt as hi + lo bfloat16 terms: lane (n16, g16) holds head n16,
// elements 8 c .. 8 c + 7 at k-step s with c = 4 s + g16, or (BY_LANE, the order
// of the FP4 code words a lane loads) c = KSS g16 + s.
template <int KSS, bool BY_LANE = false>
__device__ __forceinline__ void subspace_operands(const float (*qt_sm)[128], int G, int lane, bf16x8_t (&bh)[KSS],
                                                  bf16x8_t (&bl)[KSS])
{
    const int n16 = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int s = 0; s < KSS; ++s) {
        uint32_t hw[4] = {0, 0, 0, 0}, lw[4] = {0, 0, 0, 0};
        const int c = BY_LANE ? KSS * g16 + s : 4 * s + g16;
        if (n16 < G) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = qt_sm[n16][8 * c + e];
                const uint32_t hb = __float_as_uint(x) >> 16;  // the leading 8 significant bits
                const float r = x - __uint_as_float(hb << 16);
                const uint32_t ru = __float_as_uint(r);
                const uint32_t lb = (ru + 0x7fffu + ((ru >> 16) & 1u)) >> 16;
                hw[e >> 1] |= hb << (16 * (e & 1));
                lw[e >> 1] |= lb << (16 * (e & 1));
            }
        }
        bh[s] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        bl[s] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
}

// FP4 descriptors, per block [mean: d bfloat16][4 fp32 scales][4 x d/2 bytes of E2M1
// codes] (kv_cov4_build).  The same tile as cobs2_tile_logits: the mean rows
// against q, and the eigenvector rows, their codes widened to bfloat16 by the
// hardware conversion (exact), against a copy of q whose k-chunks follow the
// code bytes each lane loads (lane g16 of a row loads its d/8 consecutive code
// bytes, i.e. coordinates [4 g16 KS, 4 (g16 + 1) KS) ... so the q operand takes
// 16-byte chunk KS g16 + s at k-step s); each product is then multiplied by
// the eigenvector's fp32 scale before it is squared.
constexpr int fp4_block_bytes(int d) { return 2 * d + 4 * kCobsRank + kCobsRank * d / 2; }

template <int D>
__device__ __forceinline__ void cobs2_fp4_tile_logits(const FusedScoreParams& p, __amdgpu_buffer_rsrc_t kr,
                                                      const bf16x8_t (&bq)[D / 32], const bf16x8_t (&bqp)[D / 32],
                                                      int base, float* dst, int stride, int lane, float (*tmp)[32],
                                                      uint4* gslot)
{
    constexpr int KS = D / 32, BB = fp4_block_bytes(D), CB = D / 8;  // code bytes per lane and row
    static_assert(kCobsRank == 4, "one output lane holds one block's four eigenvector products");
    // The tile's 32 BB bytes are contiguous: loaded 16 bytes per lane (a KiB per
    // load, non-temporal; chunks past the tile or past nb read as zeros), each
    // group of 8 blocks copied to the wave's LDS slot, the lanes' mean chunks,
    // code words and scales taken from there.
    constexpr int GC = 8 * BB / 16, NJ = (4 * GC + 63) / 64;  // chunks per group; loads per lane
    static_assert(8 * BB % 16 == 0, "groups of whole 16-byte chunks");
    const int n16 = lane & 15, g16 = lane >> 4;
    const uint32_t oob = (uint32_t)p.nb * BB;  // the buffer's size: a load there reads zeros
    uint4 v[NJ];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
        const int ci = 64 * jj + lane;
        v[jj] = buffer_ld16_nt(kr, ci < 4 * GC ? (uint32_t)base * BB + (uint32_t)ci * 16 : oob);
    }
    const char* const g = reinterpret_cast<const char*>(gslot);
    uint4 am[2][KS];
    uint32_t ac[4][2][KS];  // four code bytes per k-step
    float4 scl[4][2];       // the four scales of the block an output lane holds
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int jj = u * GC / 64; jj <= ((u + 1) * GC - 1) / 64; ++jj) {
            const int ci = 64 * jj + lane;
            if (ci >= u * GC && ci < (u + 1) * GC) gslot[ci - u * GC] = v[jj];
        }
        wave_lds_fence();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int tr = rb * 16 + n16;
            const char* c = g + (tr / 4) * BB + 2 * D + 16 + (tr % 4) * (D / 2) + g16 * CB;
            if constexpr (KS == 4) {
                const uint4 c4 = *reinterpret_cast<const uint4*>(c);
                ac[u][rb][0] = c4.x;
                ac[u][rb][1] = c4.y;
                ac[u][rb][2] = c4.z;
                ac[u][rb][3] = c4.w;
            } else {
                ac[u][rb][0] = *reinterpret_cast<const uint32_t*>(c);
                ac[u][rb][1] = *reinterpret_cast<const uint32_t*>(c + 4);
            }
            scl[u][rb] = *reinterpret_cast<const float4*>(g + (4 * rb + g16) * BB + 2 * D);
        }
        // the mean rows of blocks 8 u .. 8 u + 7: lanes n16 = 8 (u % 2) + i of mean block u / 2
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 m = *reinterpret_cast<const uint4*>(g + (n16 & 7) * BB + g16 * 16 + s * 64);
            if ((n16 >> 3) == (u & 1)) am[u >> 1][s] = m;
        }
        wave_lds_fence();  // the slot is rewritten next
    }
    f32x4_t cm[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
            cm[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, am[rb][s]), bq[s], cm[rb], 0, 0,
                                                             0);
    float sq[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4_t cx[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const uint32_t w = ac[u][rb][s];
                typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
                const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
                const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
                const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
                const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
                const uint4 a = make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                                           __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3));
                cx[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), bqp[s], cx[rb], 0, 0,
                                                                 0);
            }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const float e0 = cx[rb][0] * scl[u][rb].x, e1 = cx[rb][1] * scl[u][rb].y;
            const float e2 = cx[rb][2] * scl[u][rb].z, e3 = cx[rb][3] * scl[u][rb].w;
            sq[u][rb] = (e0 * e0 + e1 * e1) + (e2 * e2 + e3 * e3);
        }
    }
    if (n16 < p.G) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = rb * 16 + 4 * g16 + i;
                tmp[n16][tr] = fmaf(cm[rb][i], p.scale, base + tr == p.nb - 1 ? p.ln_last : p.ln_L);
            }
    }
    wave_lds_fence();
    const float half_s2 = 0.5f * p.scale * p.scale;
    if (n16 < p.G) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) tmp[n16][8 * u + 4 * rb + g16] += half_s2 * sq[u][rb];
    }
    wave_lds_fence();
    for (int e = lane; e < p.G * 32; e += 64) {
        const int h = e >> 5, b = e & 31;
        if (base + b < p.nb) dst[h * stride + base + b] = tmp[h][b];
    }
    wave_lds_fence();  // tmp is reused by the next tile
}

// The query operand with 16-byte chunk KS g16 + s at k-step s (see above).
template <int D>
__device__ __forceinline__ void load_q_operand_by_lane_chunks(const char* q_first_head, int nh, int lane,
                                                              bf16x8_t (&bq)[D / 32])
{
    constexpr int KS = D / 32;
    const int n16 = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n16 < nh) v = ld16(q_first_head + (size_t)n16 * D * 2 + (KS * g16 + s) * 16);
        bq[s] = __builtin_bit_cast(bf16x8_t, v);
    }
}

template <int D, bool FP4>
__global__ void __launch_bounds__(kFusedWaves * 64) score_cobs2_fused_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, NW = kFusedWaves, NR = 1 + kCobsRank;
    constexpr int BB = FP4 ? fp4_block_bytes(D) : NR * RB;
    extern __shared__ float lsm[];  // [G][nb] block logits
    __shared__ float lse_h[8];
    __shared__ float tmp[NW][8][32];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    bf16x8_t bq[KS], bqp[KS];
    load_q_operand<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bq);
    if constexpr (FP4) load_q_operand_by_lane_chunks<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bqp);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * BB, (uint32_t)p.nb * BB);
    static_assert(FP4, "bfloat16 descriptors go through the split kernel");
    __shared__ uint4 gslot[NW][8 * BB / 16];
    for (int base = wave * 32; base < p.nb; base += NW * 32)
        cobs2_fp4_tile_logits<D>(p, kr, bq, bqp, base, lsm, p.nb, lane, tmp[wave], gslot[wave]);
    __syncthreads();
    group_scores_in_lds<NW>(lsm, lse_h, p.G, p.nb, p.scores + (size_t)pair * p.nb);
}

template <int D, bool FP4>
__global__ void __launch_bounds__(kSplitWaves * 64) score_cobs2_split_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, NR = 1 + kCobsRank;
    constexpr int BB = FP4 ? fp4_block_bytes(D) : NR * RB;
    __shared__ float tmp[kSplitWaves][8][32];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.x / p.chunks, chunk = blockIdx.x - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int base = (chunk * kSplitWaves + wave) * 32;
    if (base >= p.nb) return;  // whole wave; no workgroup barrier in this kernel
    bf16x8_t bq[KS], bqp[KS];
    load_q_operand<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bq);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * BB, (uint32_t)p.nb * BB);
    if constexpr (FP4) {
        __shared__ uint4 gslot[kSplitWaves][8 * BB / 16];
        load_q_operand_by_lane_chunks<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bqp);
        cobs2_fp4_tile_logits<D>(p, kr, bq, bqp, base, p.logits + (size_t)pair * p.G * p.nb, p.nb, lane, tmp[wave],
                                 gslot[wave]);
    } else {
        __shared__ uint4 cslot[kSplitWaves][40 * (RB / 16 + 1)];
        cobs2_tile_logits<D>(p, kr, bq, base, p.logits + (size_t)pair * p.G * p.nb, p.nb, lane, tmp[wave],
                             cslot[wave]);
    }
}

// Query-subspace second-order logits, split form: workgroup (pair, chunk), one tile
// per wave, the subspace query computed by the workgroup first.
template <int D, int KSS, bool FP4>
__global__ void __launch_bounds__(kSplitWaves * 64) score_cobs2_sub_split_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32;
    __shared__ float tmp[kSplitWaves][8][32];
    __shared__ float qt_sm[8][128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.x / p.chunks, chunk = blockIdx.x - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int base = (chunk * kSplitWaves + wave) * 32;
    const char* q0 = p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB;
    subspace_query<D, KSS>(p, q0, j, qt_sm);
    __syncthreads();
    if (base >= p.nb) return;  // whole wave; no barrier after this point
    bf16x8_t bq[KS], bh[KSS], bl[KSS];
    load_q_operand<D>(q0, p.G, lane, bq);
    subspace_operands<KSS, FP4>(qt_sm, p.G, lane, bh, bl);
    const uint32_t BB = FP4 ? (uint32_t)(2 * D + 16 + 64 * KSS) : (uint32_t)(RB + kCobsRank * p.sps * 2);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * BB, (uint32_t)p.nb * BB);
    float* dst = p.logits + (size_t)pair * p.G * p.nb;
    __shared__ uint4 gslot[kSplitWaves][FP4 ? (2 * D + 16 + 64 * KSS) / 2 : (RB + kCobsRank * 32 * KSS * 2) / 2];
    if constexpr (FP4)
        cobs2_sub4_tile_logits<D, KSS>(p, kr, bq, bh, bl, base, dst, p.nb, lane, tmp[wave], gslot[wave]);
    else
        cobs2_sub_tile_logits<D, KSS>(p, kr, bq, bh, bl, base, dst, p.nb, lane, tmp[wave], gslot[wave]);
}

// Query-subspace second-order scores, one workgroup per KV head: the subspace
// query once, the tiles by the eight waves, the group scores in LDS.
template <int D, int KSS, bool FP4>
__global__ void __launch_bounds__(kFusedWaves * 64) score_cobs2_sub_fused_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, NW = kFusedWaves;
    extern __shared__ float lsm[];  // [G][nb] block logits
    __shared__ float lse_h[8];
    __shared__ float tmp[NW][8][32];
    __shared__ float qt_sm[8][128];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    const char* q0 = p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB;
    subspace_query<D, KSS>(p, q0, j, qt_sm);
    __syncthreads();
    bf16x8_t bq[KS], bh[KSS], bl[KSS];
    load_q_operand<D>(q0, p.G, lane, bq);
    subspace_operands<KSS, FP4>(qt_sm, p.G, lane, bh, bl);
    const uint32_t BB = FP4 ? (uint32_t)(2 * D + 16 + 64 * KSS) : (uint32_t)(RB + kCobsRank * p.sps * 2);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * BB, (uint32_t)p.nb * BB);
    __shared__ uint4 gslot[NW][FP4 ? (2 * D + 16 + 64 * KSS) / 2 : (RB + kCobsRank * 32 * KSS * 2) / 2];
    for (int base = wave * 32; base < p.nb; base += NW * 32) {
        if constexpr (FP4)
            cobs2_sub4_tile_logits<D, KSS>(p, kr, bq, bh, bl, base, lsm, p.nb, lane, tmp[wave], gslot[wave]);
        else
            cobs2_sub_tile_logits<D, KSS>(p, kr, bq, bh, bl, base, lsm, p.nb, lane, tmp[wave], gslot[wave]);
    }
    __syncthreads();
    group_scores_in_lds<NW>(lsm, lse_h, p.G, p.nb, p.scores + (size_t)pair * p.nb);
}

// Proxy-error logits ("OpenAttention reads 1% of the KV cache -- Count-aware
// tail proxy", section "Skipping reviews without losing the verdict": a proxy's
// weight error grows with its mass and with the spread of its block's logits,
// here estimated from cached mean and variance tokens).  Rows
// Kvar [.., nb, 2, d]: the mean key and the per-coordinate key variance of each
// block.  For the tile of blocks [base, base + 32), lane (n16, g16) gets head
// n16 of blocks base + 16 rb + 4 g16 + i from three MFMA chains: the summary
// logit shat = scale q.kbar + ln c from the mean rows, and sum_t q_t^2 var_t
// from the variance rows against q^2 split into two bfloat16 halves (q is
// bfloat16, so q^2 has at most 16 significant bits and hi + lo holds it
// exactly; the products are exact in fp32).  The log-error shat + ln sigma,
// sigma = scale sqrt(sum), goes to dst[h * stride + b] (-inf for sigma = 0);
// the lane's online log-sum-exp of shat (log2 units) is kept in (m2, s2).
template <int D>
__device__ __forceinline__ void err_tile_logits(const FusedScoreParams& p, __amdgpu_buffer_rsrc_t kr,
                                                const bf16x8_t (&bq)[D / 32], const bf16x8_t (&bqh)[D / 32],
                                                const bf16x8_t (&bql)[D / 32], int base, float* dst, int stride,
                                                int lane, float& m2, float& s2, uint4* slot)
{
    constexpr int RB = D * 2, KS = D / 32;
    // The tile's 64 rows (mean and variance row of 32 blocks, contiguous) are
    // loaded whole with the non-temporal hint (LPV lanes per row, RPV rows per
    // load), then each 16-block half goes through the wave's LDS slot into the
    // operand layout: slot rows 0..15 the mean rows, 16..31 the variance rows.
    constexpr int LPV = RB / 16, RPV = 64 / LPV, NI = 64 / RPV;
    const int n16 = lane & 15, g16 = lane >> 4, gv = lane / LPV, ck = lane % LPV;
    uint4 rows[NI];
#pragma unroll
    for (int jj = 0; jj < NI; ++jj)  // past nb: zeros
        rows[jj] = buffer_ld16_nt(kr, (uint32_t)(2 * base + RPV * jj + gv) * RB + ck * 16);
    uint4 am[2][KS], av[2][KS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int jj = 0; jj < NI / 2; ++jj) {
            const int lr = RPV * jj + gv;  // row of this half: block lr / 2, mean (even) or variance (odd)
            slot[((lr & 1) * 16 + (lr >> 1)) * (LPV + 1) + ck] = rows[rb * (NI / 2) + jj];
        }
        wave_lds_fence();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            am[rb][s] = slot[n16 * (LPV + 1) + 4 * s + g16];
            av[rb][s] = slot[(16 + n16) * (LPV + 1) + 4 * s + g16];
        }
        wave_lds_fence();  // the slot is rewritten next
    }
    f32x4_t cm[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
    f32x4_t cv[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            cm[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, am[rb][s]), bq[s], cm[rb], 0, 0,
                                                             0);
            cv[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[rb][s]), bqh[s], cv[rb], 0,
                                                             0, 0);
            cv[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[rb][s]), bql[s], cv[rb], 0,
                                                             0, 0);
        }
    if (n16 < p.G) {
        const float s2c = p.scale * p.scale;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = base + rb * 16 + 4 * g16 + i;
                if (b < p.nb) {
                    const float sh = fmaf(cm[rb][i], p.scale, b == p.nb - 1 ? p.ln_last : p.ln_L);
                    const float var = cv[rb][i] * s2c;
                    dst[n16 * stride + b] = var > 0.0f ? sh + 0.5f * logf(var) : kNegInf;
                    const float t = sh * kLog2e;
                    const float mn = fmaxf(m2, t);
                    s2 = s2 * rescale(m2, mn) + exp2_(t - mn);
                    m2 = mn;
                }
            }
    }
}

// q^2 as two bfloat16 operands (hi + lo == q^2 exactly) in the layout of bq.
template <int D>
__device__ __forceinline__ void square_q_operand(const bf16x8_t (&bq)[D / 32], bf16x8_t (&hi)[D / 32],
                                                 bf16x8_t (&lo)[D / 32])
{
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        const uint4 v = __builtin_bit_cast(uint4, bq[s]);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t h2 = 0, l2 = 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float f = __uint_as_float(half ? (w[e] & 0xffff0000u) : (w[e] << 16));
                const float sq = f * f;  // exact: 8 significant bits squared
                const uint32_t hb = bf16_from_f64((double)sq);
                const uint32_t lb = bf16_from_f64((double)(sq - __uint_as_float(hb << 16)));
                h2 |= hb << (16 * half);
                l2 |= lb << (16 * half);
            }
            wh[e] = h2;
            wl[e] = l2;
        }
        hi[s] = __builtin_bit_cast(bf16x8_t, make_uint4(wh[0], wh[1], wh[2], wh[3]));
        lo[s] = __builtin_bit_cast(bf16x8_t, make_uint4(wl[0], wl[1], wl[2], wl[3]));
    }
}

template <int D>
__global__ void __launch_bounds__(kFusedWaves * 64) score_err_fused_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, NW = kFusedWaves;
    extern __shared__ float lsm[];  // [G][nb] log-errors
    __shared__ float lse_h[8];
    __shared__ float pm[NW][8], ps[NW][8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    bf16x8_t bq[KS], bqh[KS], bql[KS];
    load_q_operand<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bq);
    square_q_operand<D>(bq, bqh, bql);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * 2 * RB, (uint32_t)p.nb * 2 * RB);
    __shared__ uint4 eslot[NW][32 * (RB / 16 + 1)];
    float m2 = kNegInf, s2 = 0.0f;
    for (int base = wave * 32; base < p.nb; base += NW * 32)
        err_tile_logits<D>(p, kr, bq, bqh, bql, base, lsm, p.nb, lane, m2, s2, eslot[wave]);
    merge_lse_groups(m2, s2);
    if (lane < 8) {
        pm[wave][lane] = m2;
        ps[wave][lane] = s2;
    }
    __syncthreads();
    if (threadIdx.x < (unsigned)p.G) {
        float M = kNegInf;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, pm[w][threadIdx.x]);
        float S = 0.0f;
        for (int w = 0; w < NW; ++w) S += ps[w][threadIdx.x] * rescale(pm[w][threadIdx.x], M);
        lse_h[threadIdx.x] = (M + log2f(S)) * kLn2;
    }
    __syncthreads();
    group_scores_in_lds<NW>(lsm, lse_h, p.G, p.nb, p.scores + (size_t)pair * p.nb, true);
}

// Split form: workgroup (pair, chunk), one tile per wave; the log-errors go to
// p.logits and each wave's log-sum-exp state of the summary logits, per head,
// to p.parts [pair][tile][8][2].
template <int D>
__global__ void __launch_bounds__(kSplitWaves * 64) score_err_split_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.x / p.chunks, chunk = blockIdx.x - pair * p.chunks;
    const int b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int tile = chunk * kSplitWaves + wave, base = tile * 32;
    if (base >= p.nb) return;  // whole wave; no barrier in this kernel
    bf16x8_t bq[KS], bqh[KS], bql[KS];
    load_q_operand<D>(p.q + ((size_t)b * p.Hq + (size_t)j * p.G) * RB, p.G, lane, bq);
    square_q_operand<D>(bq, bqh, bql);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * p.nb * 2 * RB, (uint32_t)p.nb * 2 * RB);
    __shared__ uint4 eslot[kSplitWaves][32 * (RB / 16 + 1)];
    float m2 = kNegInf, s2 = 0.0f;
    err_tile_logits<D>(p, kr, bq, bqh, bql, base, p.logits + (size_t)pair * p.G * p.nb, p.nb, lane, m2, s2,
                       eslot[wave]);
    merge_lse_groups(m2, s2);
    if (p.parts && lane < 8) {
        const int tiles = (p.nb + 31) / 32;
        float* dst = p.parts + (((size_t)pair * tiles + tile) * 8 + lane) * 2;
        dst[0] = m2;
        dst[1] = s2;
    }
}

// Normaliser (natural log) of one head from its tiles' log-sum-exp states,
// lane t holding those of tiles t, t + 64, ... (absent ones (-inf, 0)): the
// maximum, then the rescaled sum, over the wave.  Every lane returns lane 0's
// value.  States (-inf, 0) change neither the maximum nor the sum, so the
// result does not depend on PT.
template <int PT>
__device__ __forceinline__ float lse_merge(const float (&mv)[PT], const float (&sv)[PT])
{
#pragma clang fp contract(off)  // the same bits wherever it is inlined
    float M = kNegInf;
#pragma unroll
    for (int j = 0; j < PT; ++j) M = fmaxf(M, mv[j]);
    M = group_max<64>(M);
    float S = 0.0f;
#pragma unroll
    for (int j = 0; j < PT; ++j) S += sv[j] * rescale(mv[j], M);
    S = group_sum<64>(S);
    const float lse = (M + log2f(S)) * kLn2;
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lse)));
}

// The normaliser of one head from its tiles' states st[16 t], st[16 t + 1]
// (t < tiles <= 256).
__device__ __forceinline__ float lse_from_parts(const float* st, int tiles, int lane)
{
    constexpr int PT = 4;
    float mv[PT], sv[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int t = lane + 64 * j;
        mv[j] = t < tiles ? st[t * 16] : kNegInf;
        sv[j] = t < tiles ? st[t * 16 + 1] : 0.0f;
    }
    return lse_merge<PT>(mv, sv);
}

// The normalisers of every head h < G of one KV head (st: its states
// [tiles][8][2], tiles <= 64 PT), all loads first; lse[h] for h >= G is lse[0].
template <int PT>
__device__ __forceinline__ void lse_from_parts_heads(const float* st, int tiles, int G, int lane, float (&lse)[8])
{
    float mv[8][PT], sv[8][PT];
#pragma unroll
    for (int h = 0; h < 8; ++h)
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int t = lane + 64 * j;
            const bool ok = t < tiles && h < G;
            const float* s = st + (size_t)(ok ? t : 0) * 16 + (h < G ? h : 0) * 2;
            const float a = s[0], c = s[1];
            mv[h][j] = ok ? a : kNegInf;
            sv[h][j] = ok ? c : 0.0f;
        }
#pragma unroll
    for (int h = 0; h < 8; ++h) lse[h] = h < G ? lse_merge<PT>(mv[h], sv[h]) : 0.0f;
#pragma unroll
    for (int h = 1; h < 8; ++h)
        if (h >= G) lse[h] = lse[0];
}

// Group scores and top-k candidates of the split route beyond
// kLseFromLogitsMaxBlocks blocks: one wave per (KV head, chunk of kCandChunk
// blocks).  The normalisers come from the tiles' log-sum-exp states and the group
// scores from the logits, by the same functions as in score_finish_kernel (the
// same bits); the scores go to p.scores (G > 1; with one head the logits are the
// scores) and the chunk's min(k, chunk blocks) best, in ascending block order, to
// cand_score / cand_idx [pair][chunk][k].  The k best blocks of the KV head are
// the k best of the candidates, ties to the lower block as by position.
__global__ void __launch_bounds__(64) score_group_chunk_kernel(const FusedScoreParams p, float* cand_score,
                                                               int32_t* cand_idx)
{
    __shared__ uint32_t cand_sm[128];
    __shared__ float sc_sm[kCandChunk];
    const int lane = threadIdx.x, G = p.G, nb = p.nb, k = p.k;
    const int nchunks = (nb + kCandChunk - 1) / kCandChunk;
    // each XCD takes a contiguous eighth of the (pair, chunk) items (with the
    // merge likewise: 128K weighted-coreset step 25.11 -> 23.87 us)
    const int wg = gridDim.x % 8 == 0 ? (int)(blockIdx.x % 8) * (int)(gridDim.x / 8) + (int)(blockIdx.x / 8)
                                      : (int)blockIdx.x;
    const int pair = wg / nchunks, chunk = wg - pair * nchunks;
    const int lo = chunk * kCandChunk, len = min(kCandChunk, nb - lo);
    constexpr int PER = kCandChunk / 64;
    float v[PER];
    if (G > 1) {
        // the chunk's logits and every head's tile states go out together
        const int tiles = (nb + 31) / 32;
        const float* lg = p.logits + (size_t)pair * G * nb;
        float lv[PER][8];
#pragma unroll
        for (int u = 0; u < PER; ++u)
#pragma unroll
            for (int h = 0; h < 8; ++h) lv[u][h] = lg[(size_t)(h < G ? h : 0) * nb + lo + min(lane + 64 * u, len - 1)];
        float lse_h[8];
        const float* st = p.parts + (size_t)pair * tiles * 16;
        if (tiles <= 64)
            lse_from_parts_heads<1>(st, tiles, G, lane, lse_h);
        else
            lse_from_parts_heads<4>(st, tiles, G, lane, lse_h);
#pragma unroll
        for (int u = 0; u < PER; ++u) v[u] = group_score_v<8>(lv[u], lse_h, G);
        if (p.scores) {
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (lane + 64 * u < len) p.scores[(size_t)pair * nb + lo + lane + 64 * u] = v[u];
        }
    } else {
#pragma unroll
        for (int u = 0; u < PER; ++u) v[u] = p.logits[(size_t)pair * nb + lo + min(lane + 64 * u, len - 1)];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) sc_sm[lane + 64 * u] = v[u];
    wave_lds_fence();
    const size_t base = ((size_t)pair * nchunks + chunk) * k;
    wave_topk<PER>([&](int i) { return sc_sm[i]; }, len, min(k, len), lane, cand_sm, [&](int r, int i) {
        cand_score[base + r] = sc_sm[i];
        cand_idx[base + r] = lo + i;
    });
}

// Group scores (and the top-k when p.k > 0) of one KV head from split logits.
__global__ void __launch_bounds__(kFusedWaves * 64) score_finish_kernel(const FusedScoreParams p)
{
    constexpr int NW = kFusedWaves;
    extern __shared__ float lsm[];  // [G][nb] block logits, then the scores in row 0
    __shared__ float lse_h[8];
    __shared__ SelectSmem<NW> ss;
    const int lane = threadIdx.x & 63;
    const int pair = blockIdx.x, G = p.G, nb = p.nb;
    // copy the logits in (chunks of loads issued together: one memory round trip each;
    // a chunk covers kFusedMaxLogits, so one round trip)
    const float* src = p.logits + (size_t)pair * G * nb;
    constexpr int CH = kFusedMaxLogits / (NW * 64);
    for (int i0 = 0; i0 < G * nb; i0 += CH * NW * 64) {
        float v[CH];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = i0 + c * NW * 64 + threadIdx.x;
            v[c] = i < G * nb ? src[i] : 0.0f;
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int i = i0 + c * NW * 64 + threadIdx.x;
            if (i < G * nb) lsm[i] = v[c];
        }
    }
    if (p.parts) {  // normalisers from the tiles' log-sum-exp states: wave h merges head h's
        const int wave = threadIdx.x >> 6, tiles = (nb + 31) / 32;
        if (wave < G) {
            const float lse = lse_from_parts(p.parts + (size_t)pair * tiles * 16 + wave * 2, tiles, lane);
            if (lane == 0) lse_h[wave] = lse;
        }
    }
    __syncthreads();
    group_scores_in_lds<NW>(lsm, lse_h, G, nb, p.scores ? p.scores + (size_t)pair * nb : nullptr, p.parts != nullptr);
    if (p.k > 0) {
        __syncthreads();
        select_in_lds<NW>(lsm, nb, p.k, p.sel + (size_t)pair * p.k, ss);
    }
}

}  // namespace

bool fused_summary_score_ok(const Dims& s)
{
    return s.dtype == DT_BF16 && s.G <= 8 && s.G * s.nb <= kFusedMaxLogits;
}

FusedScoreParams summary_params(const Dims& s, const void* q, const void* Kbar, bool box)
{
    FusedScoreParams p{};
    p.q = static_cast<const char*>(q);
    p.Kbar = static_cast<const char*>(Kbar);
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.nb = s.nb;
    p.scale = s.scale;
    p.ln_L = box ? 0.0f : s.ln_L;  // the box score has no count term
    p.ln_last = box ? 0.0f : s.ln_last;
    return p;
}

hipError_t launch_score_summary_fused(const Dims& s, const void* q, const void* Kbar, float* scores, hipStream_t st,
                                      bool box, const int32_t* offsets, int32_t* sel, int k)
{
    FusedScoreParams p = summary_params(s, q, Kbar, box);
    p.scores = scores;
    p.offsets = offsets;
    p.sel = sel;
    p.k = k;
    const size_t shm = (size_t)s.G * s.nb * sizeof(float);
    const dim3 grid((unsigned)s.pairs()), block(kFusedWaves * 64);
    if (box) {
        if (s.d == 128)
            score_summary_fused_kernel<256, true><<<grid, block, shm, st>>>(p);
        else
            score_summary_fused_kernel<128, true><<<grid, block, shm, st>>>(p);
    } else {
        if (s.d == 128)
            score_summary_fused_kernel<128, false><<<grid, block, shm, st>>>(p);
        else
            score_summary_fused_kernel<64, false><<<grid, block, shm, st>>>(p);
    }
    return hipGetLastError();
}

bool split_select_ok(const Dims& s, int k)
{
    return k <= kFinishMaxK && s.nb <= kFinishMaxBlocks;
}

hipError_t launch_score_summary_split(const Dims& s, const void* q, const void* Kbar, float* logits, float* scores,
                                      int32_t* sel, int k, hipStream_t st, bool box, const int32_t* offsets,
                                      float* parts)
{
    FusedScoreParams p = summary_params(s, q, Kbar, box);
    p.offsets = offsets;
    p.parts = s.G > 1 && s.nb > kLseFromLogitsMaxBlocks ? parts : nullptr;
    p.logits = logits;
    p.scores = scores;
    p.sel = sel;
    p.k = k;
    const int tiles = (s.nb + 31) / 32;
    p.chunks = (tiles + kSplitWaves - 1) / kSplitWaves;
    const dim3 grid((unsigned)(s.pairs() * p.chunks)), block(kSplitWaves * 64);
    if (box) {
        if (s.d == 128)
            score_logits_split_kernel<256, true><<<grid, block, 0, st>>>(p);
        else
            score_logits_split_kernel<128, true><<<grid, block, 0, st>>>(p);
    } else {
        if (s.d == 128)
            score_logits_split_kernel<128, false><<<grid, block, 0, st>>>(p);
        else
            score_logits_split_kernel<64, false><<<grid, block, 0, st>>>(p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (s.G == 1 && k == 0) || k < 0) return e;  // G == 1: the logits are the scores
    return launch_score_finish(s, logits, scores, sel, k, st, p.parts);
}

hipError_t launch_score_group_chunks(const Dims& s, const float* logits, const float* parts, float* scores, int k,
                                     float* cand_score, int32_t* cand_idx, hipStream_t st)
{
    if (s.nb <= kLseFromLogitsMaxBlocks || k < 1 || k > kFinishMaxK || (s.G > 1 && !parts) || s.G > 8)
        return hipErrorInvalidValue;
    FusedScoreParams p{};
    p.logits = const_cast<float*>(logits);
    p.parts = const_cast<float*>(parts);
    p.scores = s.G > 1 ? scores : nullptr;
    p.G = s.G;
    p.nb = s.nb;
    p.k = k;
    const int nchunks = (s.nb + kCandChunk - 1) / kCandChunk;
    score_group_chunk_kernel<<<dim3((unsigned)(s.pairs() * nchunks)), dim3(64), 0, st>>>(p, cand_score, cand_idx);
    return hipGetLastError();
}

template <bool FP4>
hipError_t launch_score_cobs2_t(const Dims& s, const void* q, const void* Kcov, float* logits, float* scores,
                                hipStream_t st)
{
    FusedScoreParams p = summary_params(s, q, Kcov, false);
    p.scores = scores;
    p.logits = logits;
    // FP4 descriptors (528 B per block at d = 128): one workgroup per KV head when
    // there are enough of them.  bfloat16 descriptors (five rows per block): the
    // split kernels and the finishing kernel, whose many workgroups stream the
    // rows faster (41.8 against 44.8 us with one workgroup per KV head at 256 KV
    // heads over 512 blocks).
    if constexpr (FP4) {
        if (s.pairs() >= kFusedStepMinPairs) {
            const size_t shm = (size_t)s.G * s.nb * sizeof(float);
            const dim3 grid((unsigned)s.pairs()), block(kFusedWaves * 64);
            if (s.d == 128)
                score_cobs2_fused_kernel<128, FP4><<<grid, block, shm, st>>>(p);
            else
                score_cobs2_fused_kernel<64, FP4><<<grid, block, shm, st>>>(p);
            return hipGetLastError();
        }
    }
    const int tiles = (s.nb + 31) / 32;
    p.chunks = (tiles + kSplitWaves - 1) / kSplitWaves;
    const dim3 grid((unsigned)(s.pairs() * p.chunks)), block(kSplitWaves * 64);
    if (s.d == 128)
        score_cobs2_split_kernel<128, FP4><<<grid, block, 0, st>>>(p);
    else
        score_cobs2_split_kernel<64, FP4><<<grid, block, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.G == 1) return e;  // G == 1: the logits are the scores
    return launch_score_finish(s, logits, scores, nullptr, 0, st);
}

hipError_t launch_score_cobs2_sub(const Dims& s, int s_dim, const void* q, const void* Kcs, const float* U,
                                  float* logits, float* scores, hipStream_t st, bool fp4)
{
    FusedScoreParams p = summary_params(s, q, Kcs, false);
    p.scores = scores;
    p.logits = logits;
    p.U = U;
    p.s_dim = s_dim;
    p.sps = (s_dim + 7) / 8 * 8;
    const int kss = (p.sps + 31) / 32;  // also the FP4 code words per lane: spf / 32
    const int tiles = (s.nb + 31) / 32;
    // one workgroup per KV head when there are enough of them and the logits fit LDS
    const bool fused = s.pairs() >= kFusedStepMinPairs && fused_summary_score_ok(s);
    p.chunks = (tiles + kSplitWaves - 1) / kSplitWaves;
    const dim3 grid((unsigned)(fused ? s.pairs() : s.pairs() * p.chunks)),
        block(fused ? kFusedWaves * 64 : kSplitWaves * 64);
    const size_t shm = fused ? (size_t)s.G * s.nb * sizeof(float) : 0;
#define CSA_SUB_CASE(D, KSS)                                                                 \
    if (fused && fp4)                                                                        \
        score_cobs2_sub_fused_kernel<D, KSS, true><<<grid, block, shm, st>>>(p);             \
    else if (fused)                                                                          \
        score_cobs2_sub_fused_kernel<D, KSS, false><<<grid, block, shm, st>>>(p);            \
    else if (fp4)                                                                            \
        score_cobs2_sub_split_kernel<D, KSS, true><<<grid, block, 0, st>>>(p);               \
    else                                                                                     \
        score_cobs2_sub_split_kernel<D, KSS, false><<<grid, block, 0, st>>>(p)
    if (s.d == 128) {
        switch (kss) {
        case 1: CSA_SUB_CASE(128, 1); break;
        case 2: CSA_SUB_CASE(128, 2); break;
        case 3: CSA_SUB_CASE(128, 3); break;
        case 4: CSA_SUB_CASE(128, 4); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (kss) {
        case 1: CSA_SUB_CASE(64, 1); break;
        case 2: CSA_SUB_CASE(64, 2); break;
        default: return hipErrorInvalidValue;
        }
    }
#undef CSA_SUB_CASE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fused || s.G == 1) return e;  // G == 1: the logits are the scores
    return launch_score_finish(s, logits, scores, nullptr, 0, st);
}

hipError_t launch_score_cobs2(const Dims& s, const void* q, const void* Kcov, float* logits, float* scores,
                              hipStream_t st, bool fp4)
{
    return fp4 ? launch_score_cobs2_t<true>(s, q, Kcov, logits, scores, st)
               : launch_score_cobs2_t<false>(s, q, Kcov, logits, scores, st);
}

size_t score_err_parts_bytes(const Dims& s)
{
    return (size_t)s.pairs() * ((s.nb + 31) / 32) * 16 * sizeof(float);
}

hipError_t launch_score_err(const Dims& s, const void* q, const void* Kvar, float* logits, float* parts,
                            float* scores, hipStream_t st)
{
    FusedScoreParams p = summary_params(s, q, Kvar, false);
    p.scores = scores;
    p.logits = logits;
    if (s.pairs() >= kFusedStepMinPairs) {
        const size_t shm = (size_t)s.G * s.nb * sizeof(float);
        const dim3 grid((unsigned)s.pairs()), block(kFusedWaves * 64);
        if (s.d == 128)
            score_err_fused_kernel<128><<<grid, block, shm, st>>>(p);
        else
            score_err_fused_kernel<64><<<grid, block, shm, st>>>(p);
        return hipGetLastError();
    }
    p.parts = s.G == 1 ? nullptr : parts;
    const int tiles = (s.nb + 31) / 32;
    p.chunks = (tiles + kSplitWaves - 1) / kSplitWaves;
    const dim3 grid((unsigned)(s.pairs() * p.chunks)), block(kSplitWaves * 64);
    if (s.d == 128)
        score_err_split_kernel<128><<<grid, block, 0, st>>>(p);
    else
        score_err_split_kernel<64><<<grid, block, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.G == 1) return e;  // G == 1: the log-errors are the scores
    FusedScoreParams f{};
    f.logits = logits;
    f.scores = scores;
    f.parts = parts;
    f.G = s.G;
    f.nb = s.nb;
    const size_t shm = (size_t)s.G * s.nb * sizeof(float);
    score_finish_kernel<<<dim3((unsigned)s.pairs()), dim3(kFusedWaves * 64), shm, st>>>(f);
    return hipGetLastError();
}

bool score_finish_ok(const Dims& s)
{
    return s.G <= 8 && s.G * s.nb <= kFusedMaxLogits;
}

hipError_t launch_score_finish(const Dims& s, const float* logits, float* scores, int32_t* sel, int k, hipStream_t st,
                               const float* parts)
{
    FusedScoreParams p{};
    p.logits = const_cast<float*>(logits);
    p.parts = const_cast<float*>(parts);
    p.scores = scores;
    p.sel = sel;
    p.k = k;
    p.G = s.G;
    p.nb = s.nb;
    const size_t shm = (size_t)s.G * s.nb * sizeof(float);
    score_finish_kernel<<<dim3((unsigned)s.pairs()), dim3(kFusedWaves * 64), shm, st>>>(p);
    return hipGetLastError();
}

namespace {

template <int DT, int D, bool EXACT>
hipError_t launch_logits_dtd(const LogitParams& p, int hg, int pairs, int hchunks, hipStream_t st)
{
    const dim3 grid((unsigned)(pairs * p.chunks), (unsigned)hchunks, 1), block(kNW * 64);
#define CSA_LOGITS_CASE(HGV)                                                                        \
    case HGV:                                                                                       \
        if (EXACT)                                                                                  \
            logits_exact_kernel<DT, D, HGV, score_unroll(HGV)><<<grid, block, 0, st>>>(p);          \
        else                                                                                        \
            logits_summary_kernel<DT, D, HGV, score_unroll(HGV)><<<grid, block, 0, st>>>(p);        \
        break;
    switch (hg) {
        CSA_LOGITS_CASE(1)
        CSA_LOGITS_CASE(2)
        CSA_LOGITS_CASE(3)
        CSA_LOGITS_CASE(4)
        CSA_LOGITS_CASE(5)
        CSA_LOGITS_CASE(6)
        CSA_LOGITS_CASE(7)
        CSA_LOGITS_CASE(8)
    default: return hipErrorInvalidValue;
    }
#undef CSA_LOGITS_CASE
    return hipGetLastError();
}

// The matrix-core exact-mass kernel: bfloat16, a group of 2 to 16 heads (one
// head per KV head is already at the memory roofline on the vector units),
// whole 32-token tiles per block.
bool exact_mfma_ok(const Dims& s)
{
    // one head per KV head too: the matrix cores waste 15 of 16 columns, but the
    // kernel's whole-row loads stream faster than the VALU kernel's (350.7
    // against 389.8 us per MHA exact-mass step at 32 KV heads x 8 sequences)
    return s.dtype == DT_BF16 && s.G >= 1 && s.G <= 16 && s.L % 32 == 0;
}

template <bool EXACT>
hipError_t launch_logits(const Dims& s, const void* q, const void* keys, float* dst, hipStream_t st)
{
    LogitParams p{};
    p.q = static_cast<const char*>(q);
    p.keys = static_cast<const char*>(keys);
    p.dst = dst;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.n = s.n;
    p.L = s.L;
    p.nb = s.nb;
    p.scale = s.scale;
    p.ln_L = s.ln_L;
    p.ln_last = s.ln_last;
    p.scale_log2 = s.scale * kLog2e;
    const int hg = s.G <= 8 ? s.G : 8, hchunks = (s.G + hg - 1) / hg;
    const int items = s.pairs() * hchunks;
    if (EXACT) {
        // blocks per workgroup: aim for >= 4096 workgroups, at least one block per wave
        int per = (int)(((long long)s.nb * items + 4095) / 4096);
        per = per < kNW ? kNW : (per + kNW - 1) / kNW * kNW;
        p.items_per_wg = per;
        p.chunks = (s.nb + per - 1) / per;
    } else {
        const int elem = s.dtype == DT_F32 ? 4 : 2;
        const int tile = 64 / (s.d * elem / 16) * score_unroll(hg) * kNW;
        int per = (int)(((long long)s.nb * items + 1023) / 1024);
        per = per < tile ? tile : (per + tile - 1) / tile * tile;
        p.items_per_wg = per;
        p.chunks = (s.nb + per - 1) / per;
    }
    if (EXACT && exact_mfma_ok(s)) {
        // blocks per workgroup: about 4096 workgroups (sixteen per CU; two blocks per
        // wave at the GQA exact-mass shape: 97 us against 101 us with 1024)
        int per = (int)(((long long)s.nb * s.pairs() + 4095) / 4096);
        per = per < kExactWaves ? kExactWaves : (per + kExactWaves - 1) / kExactWaves * kExactWaves;
        p.items_per_wg = per;
        p.chunks = (s.nb + per - 1) / per;
        const dim3 grid((unsigned)(s.pairs() * p.chunks)), block(kExactWaves * 64);
        if (s.d == 128)
            logits_exact_mfma_kernel<128><<<grid, block, 0, st>>>(p);
        else
            logits_exact_mfma_kernel<64><<<grid, block, 0, st>>>(p);
        return hipGetLastError();
    }
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_logits_dtd<DT_BF16, 128, EXACT>(p, hg, s.pairs(), hchunks, st);
        if (s.d == 64) return launch_logits_dtd<DT_BF16, 64, EXACT>(p, hg, s.pairs(), hchunks, st);
    } else {
        if (s.d == 128) return launch_logits_dtd<DT_F32, 128, EXACT>(p, hg, s.pairs(), hchunks, st);
        if (s.d == 64) return launch_logits_dtd<DT_F32, 64, EXACT>(p, hg, s.pairs(), hchunks, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

namespace {

template <int DT, int D>
hipError_t launch_box_dtd(const LogitParams& p, int hg, int pairs, int hchunks, hipStream_t st)
{
    const dim3 grid((unsigned)(pairs * p.chunks), (unsigned)hchunks, 1), block(kNW * 64);
    switch (hg) {
    case 1: logits_box_kernel<DT, D, 1, score_unroll(1)><<<grid, block, 0, st>>>(p); break;
    case 2: logits_box_kernel<DT, D, 2, score_unroll(2)><<<grid, block, 0, st>>>(p); break;
    case 3: logits_box_kernel<DT, D, 3, score_unroll(3)><<<grid, block, 0, st>>>(p); break;
    case 4: logits_box_kernel<DT, D, 4, score_unroll(4)><<<grid, block, 0, st>>>(p); break;
    case 5: logits_box_kernel<DT, D, 5, score_unroll(5)><<<grid, block, 0, st>>>(p); break;
    case 6: logits_box_kernel<DT, D, 6, score_unroll(6)><<<grid, block, 0, st>>>(p); break;
    case 7: logits_box_kernel<DT, D, 7, score_unroll(7)><<<grid, block, 0, st>>>(p); break;
    case 8: logits_box_kernel<DT, D, 8, score_unroll(8)><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_logits_box(const Dims& s, const void* q, const void* Kbox, float* dst, hipStream_t st)
{
    LogitParams p{};
    p.q = static_cast<const char*>(q);
    p.keys = static_cast<const char*>(Kbox);
    p.dst = dst;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.n = s.n;
    p.L = s.L;
    p.nb = s.nb;
    p.scale = s.scale;
    const int hg = s.G <= 8 ? s.G : 8, hchunks = (s.G + hg - 1) / hg;
    const int items = s.pairs() * hchunks;
    const int elem = s.dtype == DT_F32 ? 4 : 2;
    const int tile = 64 / (s.d * elem / 16) * score_unroll(hg) * kNW;
    int per = (int)(((long long)s.nb * items + 1023) / 1024);
    per = per < tile ? tile : (per + tile - 1) / tile * tile;
    p.items_per_wg = per;
    p.chunks = (s.nb + per - 1) / per;
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_box_dtd<DT_BF16, 128>(p, hg, s.pairs(), hchunks, st);
        if (s.d == 64) return launch_box_dtd<DT_BF16, 64>(p, hg, s.pairs(), hchunks, st);
    } else {
        if (s.d == 128) return launch_box_dtd<DT_F32, 128>(p, hg, s.pairs(), hchunks, st);
        if (s.d == 64) return launch_box_dtd<DT_F32, 64>(p, hg, s.pairs(), hchunks, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_block_logits_summary(const Dims& s, const void* q, const void* Kbar, float* dst, hipStream_t st)
{
    return launch_logits<false>(s, q, Kbar, dst, st);
}

hipError_t launch_block_logits_exact(const Dims& s, const void* q, const void* K, float* dst, hipStream_t st)
{
    return launch_logits<true>(s, q, K, dst, st);
}

hipError_t launch_group_score(const Dims& s, const float* logits, float* scores, hipStream_t st)
{
    const size_t shm = (size_t)(s.G + 8) * sizeof(float);
    group_score_kernel<<<dim3((unsigned)s.pairs()), dim3(256), shm, st>>>(logits, scores, s.Hq, s.Hkv, s.G, s.nb);
    return hipGetLastError();
}

}  // namespace csa

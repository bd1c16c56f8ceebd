// select.hpp -- wave-level pieces of block scoring and top-k selection shared
// by the modular kernels and the fused decode step, so that both produce the
// same bits.
//
// Group score (additive GQA score of "COBS: Cumulant Order Block Sparse
// Attention", Eq. (5)): the mass that head h puts on block b is
// exp(l_hb - LSE_h) with LSE_h the log-normaliser of head h over the blocks;
// the group score of b is the log of its summed mass over the G heads of the
// KV head, ln sum_h exp(l_hb - LSE_h), which orders the blocks like the summed
// mass itself.  With one head per KV head the score is the block logit.
//
// Selection: the kk blocks with the largest scores, ties to the lower index,
// reported in ascending index order.
#pragma once

#include "device.hpp"

namespace csa {

// Monotone map float -> uint32 (larger float -> larger key); -0 ties with +0.
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Log-normaliser of one head's block logits row[0..nb) in LDS, by one wave;
// every lane returns it.  Lane l takes the logits l, l + 64, ... in that order;
// the loads of a chunk of CH per lane go out together (one LDS round trip per
// chunk instead of one per logit).
template <int CH = 8>
__device__ __forceinline__ float head_lse(const float* row, int nb, int lane)
{
#pragma clang fp contract(off)  // the same bits wherever it is inlined
    auto load_chunk = [&](int base, float (&v)[CH]) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int i = base + lane + 64 * j;
            v[j] = row[i < nb ? i : 0];
        }
    };
    float v[CH];
    float mx = kNegInf, sum = 0.0f;
    if (nb <= 64 * CH) {  // one chunk: both passes from registers
        load_chunk(0, v);
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (lane + 64 * j < nb) mx = fmaxf(mx, v[j]);
        mx = group_max<64>(mx);
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (lane + 64 * j < nb) sum += exp2_((v[j] - mx) * kLog2e);
    } else {
        for (int base = 0; base < nb; base += 64 * CH) {
            load_chunk(base, v);
#pragma unroll
            for (int j = 0; j < CH; ++j)
                if (base + lane + 64 * j < nb) mx = fmaxf(mx, v[j]);
        }
        mx = group_max<64>(mx);
        for (int base = 0; base < nb; base += 64 * CH) {
            load_chunk(base, v);
#pragma unroll
            for (int j = 0; j < CH; ++j)
                if (base + lane + 64 * j < nb) sum += exp2_((v[j] - mx) * kLog2e);
        }
    }
    sum = group_sum<64>(sum);
    return mx + logf(sum);
}

// Group score of one block from its head logits lv[h] and normalisers ls[h]
// (entries h >= G are ignored).
template <int MAXG>
__device__ __forceinline__ float group_score_v(const float (&lv)[MAXG], const float (&ls)[MAXG], int G)
{
#pragma clang fp contract(off)  // the same bits wherever it is inlined
    float x[MAXG];
#pragma unroll
    for (int h = 0; h < MAXG; ++h) x[h] = lv[h] - ls[h];
    float mx = kNegInf;
#pragma unroll
    for (int h = 0; h < MAXG; ++h)
        if (h < G) mx = fmaxf(mx, x[h]);
    if (mx == kNegInf) return kNegInf;  // no head gives the block any weight
    float sum = 0.0f;
#pragma unroll
    for (int h = 0; h < MAXG; ++h)
        if (h < G) sum += exp2_((x[h] - mx) * kLog2e);
    return mx + logf(sum);
}

// Group score of one block from its G <= MAXG head logits l[h * stride].
template <int MAXG>
__device__ __forceinline__ float group_score(const float* l, int stride, const float* lse_h, int G)
{
    float lv[MAXG], ls[MAXG];
#pragma unroll
    for (int h = 0; h < MAXG; ++h) {
        lv[h] = l[(h < G ? h : 0) * stride];
        ls[h] = lse_h[h < G ? h : 0];
    }
    return group_score_v<MAXG>(lv, ls, G);
}

// Key (hi, lo) = (order_key(score), ~index): larger key = larger score, then
// lower index.  Replaces (h, l) by the larger of itself and (oh, ol).
__device__ __forceinline__ void key_max(uint32_t& h, uint32_t& l, uint32_t oh, uint32_t ol)
{
    const bool gt = oh > h || (oh == h && ol > l);
    h = gt ? oh : h;
    l = gt ? ol : l;
}

// Largest key of the wave, in every lane (DPP within 16-lane rows, then the
// lane-swap instructions across rows).
__device__ __forceinline__ void wave_key_max(uint32_t& h, uint32_t& l)
{
    key_max(h, l, dpp_u32<DPP_QUAD_1032>(h), dpp_u32<DPP_QUAD_1032>(l));
    key_max(h, l, dpp_u32<DPP_QUAD_2301>(h), dpp_u32<DPP_QUAD_2301>(l));
    key_max(h, l, dpp_u32<DPP_ROW_HMIRROR>(h), dpp_u32<DPP_ROW_HMIRROR>(l));
    key_max(h, l, dpp_u32<DPP_ROW_MIRROR>(h), dpp_u32<DPP_ROW_MIRROR>(l));
    LanePair ph = swap16(h), pl = swap16(l);
    h = ph.a;
    l = pl.a;
    key_max(h, l, ph.b, pl.b);
    ph = swap32(h);
    pl = swap32(l);
    h = ph.a;
    l = pl.a;
    key_max(h, l, ph.b, pl.b);
}

// Largest uint32 of the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<DPP_QUAD_1032>(v));
    v = max(v, dpp_u32<DPP_QUAD_2301>(v));
    v = max(v, dpp_u32<DPP_ROW_HMIRROR>(v));
    v = max(v, dpp_u32<DPP_ROW_MIRROR>(v));
    LanePair r = swap16(v);
    v = max(r.a, r.b);
    r = swap32(v);
    return max(r.a, r.b);
}

// Number of lanes below this one whose bit is set in a wave-wide mask.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Top-kk (1 <= kk <= nb, kk <= 64, nb <= 64 * MAXPER) of the scores load(0..nb)
// by one wave.  Block i belongs to lane i % 64 (slot i / 64), which keeps the
// order keys of its blocks in registers.  At the end emit(r, i) is called, in
// lane r < kk, with the r-th smallest selected index i (ascending order).
// cand: 128 words of LDS owned by the wave.
//
// Candidates first: the kk-th largest of the 64 per-lane maximum keys is a
// lower bound tau for the kk-th largest key overall (the kk largest lane maxima
// are kk distinct blocks), so every selected block has key >= tau.  When at
// most 64 blocks reach tau, they are gathered one per lane, in ascending index
// order, and each is ranked against the others by (key, lower index); else
// (many equal scores) the blocks are taken one round at a time.
template <int MAXPER, typename Load, typename Emit>
__device__ __forceinline__ void wave_topk(Load load, int nb, int kk, int lane, uint32_t* cand, Emit emit)
{
    uint32_t key[MAXPER];
    uint32_t lmax = 0;
#pragma unroll
    for (int j = 0; j < MAXPER; ++j) {
        const int i = lane + 64 * j;
        const float f = load(i < nb ? i : 0);  // unconditional: the loads go out together
        key[j] = i < nb ? order_key(f) : 0u;
        lmax = max(lmax, key[j]);
    }
    // tau: the kk-th largest lane maximum, counting equal maxima separately
    // (lanes without a block drop out at once; at least kk lanes hold one, so
    // the loop ends within kk rounds)
    bool live = lane < nb;
    uint32_t tau = 0;  // stays 0 (every block a candidate) if the bound is not reached
    for (int got = 0, round = 0; round < 64; ++round) {
        const uint32_t mx = wave_max_u32(live ? lmax : 0u);
        const uint64_t hit = __ballot(live && lmax == mx);
        got += __popcll(hit);
        if (got >= kk) {
            tau = mx;
            break;
        }
        if (live && lmax == mx) live = false;
    }
    uint64_t cmask[MAXPER];
    int ncand = 0;
#pragma unroll
    for (int j = 0; j < MAXPER; ++j) {
        cmask[j] = __ballot(lane + 64 * j < nb && key[j] >= tau);
        ncand += __popcll(cmask[j]);
    }
    if (ncand <= 64) {
        int base = 0;
#pragma unroll
        for (int j = 0; j < MAXPER; ++j) {
            if ((cmask[j] >> lane) & 1u) {
                const int pos = base + lanes_below(cmask[j]);
                cand[pos] = key[j];
                cand[64 + pos] = (uint32_t)(lane + 64 * j);
            }
            base += __popcll(cmask[j]);
        }
        wave_lds_fence();
        const bool mine = lane < ncand;
        const uint32_t ck = mine ? cand[lane] : 0u, ci = mine ? cand[64 + lane] : 0u;
        int rank = 0;  // candidates ahead of this one: larger key, or equal key and lower index
        for (int q = 0; q < ncand; ++q) {
            const uint32_t qk = (uint32_t)__builtin_amdgcn_readlane((int)ck, q);
            const uint32_t qi = (uint32_t)__builtin_amdgcn_readlane((int)ci, q);
            rank += (qk > ck || (qk == ck && qi < ci)) ? 1 : 0;
        }
        const bool take = mine && rank < kk;
        const uint64_t tm = __ballot(take);
        if (take) emit(lanes_below(tm), (int)ci);
        wave_lds_fence();  // cand is reused by the next call
        return;
    }
    // fallback: kk rounds, each taking the wave's largest (key, lower index)
    uint32_t taken = 0;
    auto lane_best = [&](uint32_t& bh, uint32_t& bl) {
        bh = 0;
        bl = 0;  // below every real key: real keys have a nonzero low word
#pragma unroll
        for (int j = 0; j < MAXPER; ++j) {
            const int i = lane + 64 * j;
            if (i < nb && !((taken >> j) & 1u)) key_max(bh, bl, key[j], ~(uint32_t)i);
        }
    };
    uint32_t bh, bl;
    lane_best(bh, bl);
    int got = 0;  // lane r keeps the r-th block taken
    for (int it = 0; it < kk; ++it) {
        uint32_t h = bh, l = bl;
        wave_key_max(h, l);
        const int widx = (int)~l;
        if (lane == it) got = widx;
        if ((widx & 63) == lane) {
            taken |= 1u << (widx >> 6);
            lane_best(bh, bl);
        }
    }
    int rank = 0;  // place among the taken blocks in ascending order
    for (int j = 0; j < kk; ++j) rank += __builtin_amdgcn_readlane(got, j) < got ? 1 : 0;
    if (lane < kk) emit(rank, got);
}

// Top-kk of the blocks i < nb by a workgroup of NW waves, for kk <= NW: thread t
// holds the order keys of blocks t + 64 NW j (j < SPT) in key[j].  Every wave
// finds its largest key; the kk-th largest of the NW wave maxima (counting equal
// maxima separately) is a lower bound tau for the kk-th largest key overall, as
// the kk largest wave maxima belong to kk distinct blocks.  Each wave puts its
// blocks whose keys reach tau into its 64 / NW slots of LDS (ordered by j, then
// lane) and, when every wave's fit, wave 0 ranks each candidate against the
// others by (key, lower index) and calls emit(r, i) in lane r < kk with the
// r-th smallest selected index i.  When some wave has more candidates (many
// equal scores), or kk > NW, fallback() runs in wave 0 instead.  The whole
// workgroup must call it: it holds two workgroup barriers.  sm: 2 NW + 128
// words of LDS; 64 / NW slots per wave.
template <int NW, int SPT, typename Fallback, typename Emit>
__device__ __forceinline__ void block_topk(const uint32_t (&key)[SPT], int nb, int kk, uint32_t* sm, Fallback fallback,
                                           Emit emit)
{
    constexpr int T = NW * 64, CPW = 64 / NW;
    static_assert(CPW * NW == 64, "64 candidate slots over the waves");
    uint32_t* wmax = sm;                // [NW] largest key of each wave
    uint32_t* over = sm + NW;           // [NW] wave has more candidates than slots
    uint32_t* ck = sm + 2 * NW;         // [64] candidate keys, 0 for an empty slot
    uint32_t* ci = sm + 2 * NW + 64;    // [64] candidate indices
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    uint32_t lmax = 0;  // below every real key (the key of -inf is 0x007fffff)
#pragma unroll
    for (int j = 0; j < SPT; ++j)
        if ((int)threadIdx.x + T * j < nb) lmax = max(lmax, key[j]);
    const uint32_t wm = wave_max_u32(lmax);
    if (lane == 0) wmax[wave] = wm;
    __syncthreads();
    // tau: the kk-th largest wave maximum; 0 (every block a candidate) if kk > NW.
    // Lane w < NW ranks wave w's maximum against the others.
    uint32_t tau = 0;
    if (kk <= NW) {
        const uint32_t m = lane < NW ? wmax[lane] : 0u;
        int above = 0;  // wave maxima ranked before this lane's
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const uint32_t o = wmax[v];
            above += (o > m || (o == m && v < lane)) ? 1 : 0;
        }
        const uint64_t at = __ballot(lane < NW && above == kk - 1);
        tau = (uint32_t)__builtin_amdgcn_readlane((int)m, (int)__builtin_ctzll(at));
    }
    uint64_t cmask[SPT];
    int mine = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
        cmask[j] = __ballot((int)threadIdx.x + T * j < nb && key[j] >= tau);
        mine += __popcll(cmask[j]);
    }
    if (lane == 0) over[wave] = mine > CPW ? 1u : 0u;
    if (mine <= CPW) {
        if (lane >= mine && lane < CPW) {  // empty slots
            ck[CPW * wave + lane] = 0u;
            ci[CPW * wave + lane] = 0u;
        }
        int pos = CPW * wave;
#pragma unroll
        for (int j = 0; j < SPT; ++j) {
            if ((cmask[j] >> lane) & 1u) {
                ck[pos + lanes_below(cmask[j])] = key[j];
                ci[pos + lanes_below(cmask[j])] = (uint32_t)((int)threadIdx.x + T * j);
            }
            pos += __popcll(cmask[j]);
        }
    }
    __syncthreads();
    if (wave != 0) return;
    uint32_t overflow = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) overflow |= over[w];
    if (overflow) {
        fallback();
        return;
    }
    const uint32_t k0 = ck[lane], i0 = ci[lane];
    const bool live = k0 != 0u;
    int rank = 0;  // candidates ahead of this one: larger key, or equal key and lower index
    for (uint64_t m = __ballot(live); m; m &= m - 1) {
        const int c = (int)__builtin_ctzll(m);
        const uint32_t kc = (uint32_t)__builtin_amdgcn_readlane((int)k0, c);
        const uint32_t ic = (uint32_t)__builtin_amdgcn_readlane((int)i0, c);
        rank += (kc > k0 || (kc == k0 && ic < i0)) ? 1 : 0;
    }
    const bool take = live && rank < kk;
    const uint64_t tm = __ballot(take);
    int before;  // taken candidates with a lower index
    if constexpr (SPT == 1) {
        before = lanes_below(tm);  // one block per thread: the slots are in index order
    } else {
        before = 0;
        for (uint64_t m = tm; m; m &= m - 1)
            before += (uint32_t)__builtin_amdgcn_readlane((int)i0, (int)__builtin_ctzll(m)) < i0 ? 1 : 0;
    }
    if (take) emit(before, (int)i0);
}

}  // namespace csa

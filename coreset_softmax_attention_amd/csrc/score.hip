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
                kr[u] = ld16(base_ptr + (size_t)t * RB);
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
// Summary mode, whole group in one workgroup per KV head: the block logits of
// all G heads go to LDS (MFMA over the mean keys), then each head's
// log-normaliser, then the group score.  Used when G <= 8 and the logits fit
// in 64 KiB of LDS.
// ---------------------------------------------------------------------------

constexpr int kFusedWaves = 8;
constexpr int kFusedMaxLogits = 16384;  // G * nb floats in LDS

struct FusedScoreParams {
    const char* q;
    const char* Kbar;
    float* scores;
    int Hq, Hkv, G, nb;
    float scale, ln_L, ln_last;
};

template <int D>
__global__ void __launch_bounds__(kFusedWaves * 64) score_summary_fused_kernel(const FusedScoreParams p)
{
    constexpr int RB = D * 2, KS = D / 32, NW = kFusedWaves;
    extern __shared__ float lsm[];  // [G][nb] block logits
    __shared__ float lse_h[8];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, g16 = lane >> 4;
    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int G = p.G, nb = p.nb;

    bf16x8_t bq[KS];
    load_q_operand<D>(p.q + ((size_t)b * p.Hq + (size_t)j * G) * RB, G, lane, bq);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(p.Kbar + (size_t)pair * nb * RB, (uint32_t)nb * RB);

    for (int base = wave * 32; base < nb; base += NW * 32) {
        uint4 ak[2][KS];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const uint32_t off = (uint32_t)(base + rb * 16 + n16) * RB + g16 * 16;  // past nb: zeros
#pragma unroll
            for (int s = 0; s < KS; ++s) ak[rb][s] = buffer_ld16(kr, off + s * 64);
        }
        f32x4_t c[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                c[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ak[rb][s]), bq[s], c[rb],
                                                                0, 0, 0);
        if (n16 < G) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = base + rb * 16 + 4 * g16 + i;
                    if (row < nb) lsm[n16 * nb + row] = fmaf(c[rb][i], p.scale, row == nb - 1 ? p.ln_last : p.ln_L);
                }
        }
    }
    __syncthreads();

    if (G > 1) {
        for (int h = wave; h < G; h += NW) {
            const float lse = head_lse(lsm + h * nb, nb, lane);
            if (lane == 0) lse_h[h] = lse;
        }
        __syncthreads();
    }
    for (int i = threadIdx.x; i < nb; i += NW * 64) {
        const float v = G == 1 ? lsm[i] : group_score<8>(lsm + i, nb, lse_h, G);
        p.scores[(size_t)pair * nb + i] = v;
    }
}

}  // namespace

bool fused_summary_score_ok(const Dims& s)
{
    return s.dtype == DT_BF16 && s.G <= 8 && s.G * s.nb <= kFusedMaxLogits;
}

hipError_t launch_score_summary_fused(const Dims& s, const void* q, const void* Kbar, float* scores, hipStream_t st)
{
    FusedScoreParams p{};
    p.q = static_cast<const char*>(q);
    p.Kbar = static_cast<const char*>(Kbar);
    p.scores = scores;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.nb = s.nb;
    p.scale = s.scale;
    p.ln_L = s.ln_L;
    p.ln_last = s.ln_last;
    const size_t shm = (size_t)s.G * s.nb * sizeof(float);
    const dim3 grid((unsigned)s.pairs()), block(kFusedWaves * 64);
    if (s.d == 128)
        score_summary_fused_kernel<128><<<grid, block, shm, st>>>(p);
    else
        score_summary_fused_kernel<64><<<grid, block, shm, st>>>(p);
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
        // blocks per workgroup: aim for >= 1024 workgroups, at least one block per wave
        int per = (int)(((long long)s.nb * items + 1023) / 1024);
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

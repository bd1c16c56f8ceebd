// attn.hip -- one online-softmax pass over the virtual tokens of a KV head.
//
// The virtual-token list of KV head (b, j) is the concatenation of
//   [exact]    every token of the selected blocks, log-weight 0
//              (dense mode: all n tokens in order);
//   [weighted] m gathered tokens with their log-weights (weighted-coreset
//              attention, "WildCat: Near-Linear Attention in Theory and
//              Practice", Abstract);
//   [proxy]    one row per block of the summary arrays, key Kbar_b, value
//              Vbar_b, log-weight ln c_b; the rows of selected blocks are
//              masked.  This is the count-aware proxy of "OpenAttention reads
//              1% of the KV cache -- Count-aware tail proxy", section
//              "Skipping reviews without losing the verdict".
// Reading all summary rows contiguously and masking the few selected ones
// costs k extra rows but keeps the proxy reads fully coalesced.
//
// Work split: a workgroup owns a contiguous range of virtual rows of one KV
// head for up to 8 query heads of its group (split-K).  Each wave walks tiles
// of U row-loads; a row's 16-byte chunks sit in LPR consecutive lanes, so one
// wave-wide load moves 64/LPR whole rows.  Logits use the base-2 exponent:
// x = log2(e) (scale q.k + logw).  Each lane group keeps an online-softmax
// state (running max, sum, accumulator of its chunk of d); states are merged
// across lane groups (shuffles), waves (LDS) and splits (merge kernel), always
// in a fixed order, so results are bitwise reproducible.
#include "device.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kNW = 4;                // waves per workgroup
constexpr int kMaxSplitRows = 8192;   // rows per workgroup (bitmap capacity)
constexpr int kTargetWorkgroups = 2048;

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
    int k, m, proxies, dense;
    int Hq, Hkv, G, n, L, nb;
    int rows, exact_rows, splits, rows_per_split;
    float scale_log2;          // scale * log2(e)
    float log2_L, log2_last;   // log2 c_b of a full and of the last block
};

template <int DT, int D, int HG, int U>
__global__ void __launch_bounds__(kNW * 64) attn_kernel(const AttnParams p)
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
    const int pbeg = p.exact_rows + p.m;   // first proxy row

    // Bitmap of selected blocks among the proxy rows [pb_lo, pb_hi) of this range.
    const int pb_lo = max(r0 - pbeg, 0);
    const int pb_hi = p.proxies ? min(r1 - pbeg, p.nb) : 0;
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
            if (r < p.exact_rows) {
                int tok;
                if (p.dense) {
                    tok = r;
                } else {
                    const int slot = r / p.L;
                    tok = p.sel[(size_t)pair * p.k + slot] * p.L + (r - slot * p.L);
                }
                valid = valid && tok >= 0 && tok < p.n;
                row = kv_pair + (valid ? tok : 0);
            } else if (r < pbeg) {
                const int t = r - p.exact_rows;
                const int tok = p.tok_idx[(size_t)pair * p.m + t];
                valid = valid && tok >= 0 && tok < p.n;
                row = kv_pair + (valid ? tok : 0);
                w = p.tok_logw[(size_t)pair * p.m + t] * kLog2e;
            } else if (r < p.rows) {
                const int blk = r - pbeg;
                kb = p.Kbar;
                vb = p.Vbar;
                row = sm_pair + blk;
                w = blk == p.nb - 1 ? p.log2_last : p.log2_L;
                if (valid) valid = !((sel_bits[(blk - pb_lo) >> 5] >> ((blk - pb_lo) & 31)) & 1u);
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

// Merge the per-split states of a KV head in split order.
template <int D>
__global__ void __launch_bounds__(256) attn_merge_kernel(const float* part, int splits, int G, int Hq, int Hkv,
                                                         float* out, float* lse)
{
    const int pair = blockIdx.x;
    const int b = pair / Hkv, j = pair - b * Hkv;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int g = idx / D, e = idx - g * D;
        const float* st = part + ((size_t)pair * splits * G + g) * (D + 2);
        const size_t stride = (size_t)G * (D + 2);
        float M = kNegInf;
        for (int s = 0; s < splits; ++s) M = fmaxf(M, st[s * stride]);
        float Ls = 0.0f, A = 0.0f;
        for (int s = 0; s < splits; ++s) {
            const float a = rescale(st[s * stride], M);
            Ls += st[s * stride + 1] * a;
            A += st[s * stride + 2 + e] * a;
        }
        const int h = j * G + g;
        out[((size_t)b * Hq + h) * D + e] = A / Ls;
        if (e == 0 && lse) lse[(size_t)b * Hq + h] = (M + log2f(Ls)) * kLn2;
    }
}

template <int DT, int D>
hipError_t launch_dtd(const AttnParams& p, int hg, int pairs, int hchunks, hipStream_t st)
{
    const dim3 grid((unsigned)(pairs * p.splits), (unsigned)hchunks, 1);
    const dim3 block(kNW * 64);
    switch (hg) {
    case 1: attn_kernel<DT, D, 1, unroll_for(1)><<<grid, block, 0, st>>>(p); break;
    case 2: attn_kernel<DT, D, 2, unroll_for(2)><<<grid, block, 0, st>>>(p); break;
    case 3: attn_kernel<DT, D, 3, unroll_for(3)><<<grid, block, 0, st>>>(p); break;
    case 4: attn_kernel<DT, D, 4, unroll_for(4)><<<grid, block, 0, st>>>(p); break;
    case 5: attn_kernel<DT, D, 5, unroll_for(5)><<<grid, block, 0, st>>>(p); break;
    case 6: attn_kernel<DT, D, 6, unroll_for(6)><<<grid, block, 0, st>>>(p); break;
    case 7: attn_kernel<DT, D, 7, unroll_for(7)><<<grid, block, 0, st>>>(p); break;
    case 8: attn_kernel<DT, D, 8, unroll_for(8)><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    attn_merge_kernel<D><<<dim3((unsigned)pairs), dim3(256), 0, st>>>(p.part, p.splits, p.G, p.Hq, p.Hkv,
                                                                      p.out, p.lse);
    return hipGetLastError();
}

}  // namespace

AttnPlan plan_attention(const Dims& s, int k, int m, int proxies, int dense)
{
    AttnPlan pl{};
    pl.exact_rows = dense ? s.n : k * s.L;
    pl.rows = pl.exact_rows + m + (proxies ? s.nb : 0);
    pl.hg = s.G <= 8 ? s.G : 8;
    pl.hchunks = (s.G + pl.hg - 1) / pl.hg;
    if (pl.rows <= 0) {  // empty virtual-token set: nothing to plan (callers reject it)
        pl.splits = 1;
        pl.rows_per_split = 0;
        pl.ws_bytes = 0;
        return pl;
    }
    const int elem = s.dtype == DT_F32 ? 4 : 2;
    const int rpw = 64 / (s.d * elem / 16);
    const int tile = rpw * unroll_for(pl.hg);
    const int items = s.pairs() * pl.hchunks;
    const int max_splits = (pl.rows + tile - 1) / tile;
    int splits = (kTargetWorkgroups + items - 1) / items;
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    int per = (pl.rows + splits - 1) / splits;
    per = (per + tile - 1) / tile * tile;
    const int cap = kMaxSplitRows / tile * tile;
    if (per > cap) per = cap;
    pl.rows_per_split = per;
    pl.splits = (pl.rows + per - 1) / per;
    pl.ws_bytes = pl.splits > 1 ? (size_t)s.pairs() * pl.splits * s.G * (s.d + 2) * sizeof(float) : 0;
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
    p.splits = pl.splits;
    p.rows_per_split = pl.rows_per_split;
    p.scale_log2 = s.scale * kLog2e;
    p.log2_L = s.ln_L * kLog2e;
    p.log2_last = s.ln_last * kLog2e;
    const int pairs = s.pairs();
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_dtd<DT_BF16, 128>(p, pl.hg, pairs, pl.hchunks, st);
        if (s.d == 64) return launch_dtd<DT_BF16, 64>(p, pl.hg, pairs, pl.hchunks, st);
    } else {
        if (s.d == 128) return launch_dtd<DT_F32, 128>(p, pl.hg, pairs, pl.hchunks, st);
        if (s.d == 64) return launch_dtd<DT_F32, 64>(p, pl.hg, pairs, pl.hchunks, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa

// cluster.hip -- query-guided clusters: one count-aware proxy per cluster of
// keys that the queries see alike ("OpenAttention reads 1% of the KV cache --
// Count-aware tail proxy", section "Three helpers that make the proxy
// accurate": keys are projected onto the top eigenvectors of the queries and
// clustered by k-means in that space once after prefill).
//
// Build (prefill time), per KV head:
//   1. projections P_i = K_i U in fp64, the d products of a coordinate summed
//      in order (U [d, r] is the caller's basis);
//   2. centroids start at the projections of the caller's seed tokens;
//   3. rounds of: assign every token to the nearest centroid (squared distance
//      over the r coordinates in order, ties to the lower index); order the
//      tokens by cluster, token order within a cluster (a stable counting sort
//      by one wave, 64 tokens at a time); move each centroid to the mean of
//      its points, summed in that order (an empty cluster keeps its centroid);
//      the last round stops after the sort;
//   4. the cache in that order (Kg, Vg) and the mean key and value of each
//      cluster, summed in fp64 in token order and rounded once.
// All of it is fp64 with every product and sum rounded separately (this file
// is compiled without contraction), so assignments, order and means are the
// bits a plain sequential evaluation gives.
//
// Decode: cluster logits scale q . Kc + ln count (-inf for an empty cluster),
// scored and selected like block logits; attention over every token of the
// selected clusters (contiguous rows of Kg, Vg) and one proxy per other
// cluster, in the MFMA online-softmax engine.
#pragma clang fp contract(off)

#include "attn_engine.hpp"
#include "device.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kProjThreads = 256;

// Set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int R>
__device__ __forceinline__ double sq_dist(const double (&x)[R], const double* c)
{
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const double t = x[j] - c[j];
        acc += t * t;
    }
    return acc;
}

// P [pairs, n, R] = K U: one thread per token, coordinates summed in order.
template <int DT, int D, int R>
__global__ void __launch_bounds__(kProjThreads) project_kernel(const char* K, const float* U, double* P, int n)
{
    using Gm = RowGeom<DT, D>;
    __shared__ double u_sm[D * R];
    const int pair = blockIdx.y;
    const float* Up = U + (size_t)pair * D * R;
    for (int i = threadIdx.x; i < D * R; i += kProjThreads) u_sm[i] = (double)Up[i];
    __syncthreads();
    const int tok = blockIdx.x * kProjThreads + threadIdx.x;
    if (tok >= n) return;
    const char* row = K + ((size_t)pair * n + tok) * Gm::row_bytes;
    double acc[R];
#pragma unroll
    for (int j = 0; j < R; ++j) acc[j] = 0.0;
    for (int ch = 0; ch < Gm::lpr; ++ch) {
        float f[Gm::epl];
        unpack<DT>(ld16(row + ch * 16), f);
#pragma unroll
        for (int e = 0; e < Gm::epl; ++e) {
            const double x = (double)f[e];
            const double* u = u_sm + (ch * Gm::epl + e) * R;
#pragma unroll
            for (int j = 0; j < R; ++j) acc[j] += x * u[j];
        }
    }
    double* out = P + ((size_t)pair * n + tok) * R;
#pragma unroll
    for (int j = 0; j < R; ++j) out[j] = acc[j];
}

// Centroids start at the seed tokens' projections (a seed outside [0, n) gives 0).
template <int R>
__global__ void __launch_bounds__(256) seed_kernel(const double* P, const int32_t* seeds, double* cent, int n, int C)
{
    const int pair = blockIdx.x;
    for (int i = threadIdx.x; i < C * R; i += 256) {
        const int c = i / R, j = i - c * R;
        const int t = seeds[(size_t)pair * C + c];
        cent[(size_t)pair * C * R + i] = (t >= 0 && t < n) ? P[((size_t)pair * n + t) * R + j] : 0.0;
    }
}

// Nearest centroid of every token; equal distances go to the lower index.
template <int R>
__global__ void __launch_bounds__(kProjThreads) assign_kernel(const double* P, const double* cent, int32_t* assign,
                                                             int n, int C)
{
    extern __shared__ double c_sm[];  // [C, R]
    const int pair = blockIdx.y;
    const double* cp = cent + (size_t)pair * C * R;
    for (int i = threadIdx.x; i < C * R; i += kProjThreads) c_sm[i] = cp[i];
    __syncthreads();
    const int tok = blockIdx.x * kProjThreads + threadIdx.x;
    if (tok >= n) return;
    double x[R];
    const double* pp = P + ((size_t)pair * n + tok) * R;
#pragma unroll
    for (int j = 0; j < R; ++j) x[j] = pp[j];
    int best = 0;
    double bd = sq_dist<R>(x, c_sm);
    for (int c = 1; c < C; ++c) {
        const double dc = sq_dist<R>(x, c_sm + c * R);
        if (dc < bd) {
            bd = dc;
            best = c;
        }
    }
    assign[(size_t)pair * n + tok] = best;
}

// Stable counting sort of one KV head's tokens by cluster: counts (LDS
// atomics), ranges, then one wave places the tokens 64 at a time in token
// order.  Within a wave's 64 tokens the lanes of one cluster are ranked by
// lane, and that cluster's cursor then moves past them.
__global__ void __launch_bounds__(256) sort_kernel(const int32_t* assign, int32_t* order, int32_t* offsets, int n,
                                                   int C)
{
    extern __shared__ int32_t cur[];  // [C] counts, then cursors
    const int pair = blockIdx.x;
    const int32_t* a = assign + (size_t)pair * n;
    int32_t* ord = order + (size_t)pair * n;
    int32_t* off = offsets + (size_t)pair * (C + 1);
    for (int c = threadIdx.x; c < C; c += 256) cur[c] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) atomicAdd(&cur[a[i]], 1);
    __syncthreads();
    if (threadIdx.x >= 64) return;  // one wave from here on
    const int lane = threadIdx.x;
    {  // exclusive scan of the counts: each lane a contiguous share, then the lanes in order
        const int per = (C + 63) / 64, lo = min(C, lane * per), hi = min(C, lo + per);
        int s = 0;
        for (int c = lo; c < hi; ++c) s += cur[c];
        int base = 0;
        for (int l = 0; l < 64; ++l) {
            const int sl = __builtin_amdgcn_readlane(s, l);
            if (l < lane) base += sl;
        }
        for (int c = lo; c < hi; ++c) {
            const int cnt = cur[c];
            off[c] = base;
            cur[c] = base;
            base += cnt;
        }
        if (lane == 63) off[C] = n;
    }
    wave_lds_fence();
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const int cid = i < n ? a[i] : -1;
        bool todo = i < n;
        for (uint64_t left = __ballot(todo); left; left = __ballot(todo)) {
            const int leader = (int)__builtin_ctzll(left);
            const int lc = __builtin_amdgcn_readlane(cid, leader);
            const uint64_t grp = __ballot(todo && cid == lc);
            const int base = cur[lc];  // every lane reads the cursor before the leader moves it
            if (todo && cid == lc) {
                ord[base + lanes_below(grp)] = i;
                todo = false;
            }
            wave_lds_fence();
            if (lane == leader) cur[lc] = base + (int)__popcll(grp);
            wave_lds_fence();
        }
    }
}

// Each non-empty cluster's centroid moves to the mean of its points' projections,
// summed in token order (the order of the sorted list); an empty one stays.
template <int R>
__global__ void __launch_bounds__(256) update_kernel(const double* P, const int32_t* order, const int32_t* offsets,
                                                     double* cent, int n, int C)
{
    const int pair = blockIdx.x;
    const int32_t* ord = order + (size_t)pair * n;
    const int32_t* off = offsets + (size_t)pair * (C + 1);
    const double* pp = P + (size_t)pair * n * R;
    for (int i = blockIdx.y * 256 + threadIdx.x; i < C * R; i += gridDim.y * 256) {
        const int c = i / R, j = i - c * R;
        const int lo = off[c], hi = off[c + 1];
        if (hi == lo) continue;
        double s = 0.0;
        for (int o = lo; o < hi; ++o) s += pp[(size_t)ord[o] * R + j];
        cent[(size_t)pair * C * R + i] = s / (double)(hi - lo);
    }
}

// Kg, Vg: the cache rows (RB bytes each) in cluster order, a lane group of
// RB / 16 lanes per row.
template <int RB>
__global__ void __launch_bounds__(256) gather_kernel(const char* K, const char* V, const int32_t* order, char* Kg,
                                                     char* Vg, int n)
{
    constexpr int LPR = RB / 16, RPB = 256 / LPR;
    const int pair = blockIdx.y;
    const int o = blockIdx.x * RPB + threadIdx.x / LPR, ch = threadIdx.x % LPR;
    if (o >= n) return;
    const int t = order[(size_t)pair * n + o];
    const size_t src = ((size_t)pair * n + t) * RB + ch * 16, dst = ((size_t)pair * n + o) * RB + ch * 16;
    *reinterpret_cast<uint4*>(Kg + dst) = ld16_nt(K + src);
    *reinterpret_cast<uint4*>(Vg + dst) = ld16_nt(V + src);
}

// Mean key and value of each cluster: fp64 sums of its rows of Kg, Vg in
// order, divided by the count, rounded once; zero rows for an empty cluster.
template <int DT, int D>
__global__ void __launch_bounds__(D) means_kernel(const char* Kg, const char* Vg, const int32_t* offsets, char* Kc,
                                                  char* Vc, int n, int C)
{
    const int c = blockIdx.x, pair = blockIdx.y, t = threadIdx.x;
    const int32_t* off = offsets + (size_t)pair * (C + 1);
    const int lo = off[c], hi = off[c + 1];
    double sk = 0.0, sv = 0.0;
    for (int o = lo; o < hi; ++o) {
        const size_t e = ((size_t)pair * n + o) * D + t;
        if constexpr (DT == DT_F32) {
            sk += (double)reinterpret_cast<const float*>(Kg)[e];
            sv += (double)reinterpret_cast<const float*>(Vg)[e];
        } else {
            sk += (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Kg)[e] << 16);
            sv += (double)__uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Vg)[e] << 16);
        }
    }
    const double m = (double)(hi - lo);
    const double mk = hi > lo ? sk / m : 0.0, mv = hi > lo ? sv / m : 0.0;
    const size_t e = ((size_t)pair * C + c) * D + t;
    if constexpr (DT == DT_F32) {
        reinterpret_cast<float*>(Kc)[e] = (float)mk;
        reinterpret_cast<float*>(Vc)[e] = (float)mv;
    } else {
        reinterpret_cast<uint16_t*>(Kc)[e] = bf16_from_f64(mk);
        reinterpret_cast<uint16_t*>(Vc)[e] = bf16_from_f64(mv);
    }
}

// ---- decode: cluster logits ------------------------------------------------

constexpr int kLogitClusters = 64;  // clusters per workgroup

// logits [B, Hq, C] = scale q_h . Kc_c + ln count_c (-inf when empty); a thread
// per (cluster, head), the d products summed in fp32 in order.
template <int DT, int D>
__global__ void __launch_bounds__(256) cluster_logits_kernel(const char* q, const char* Kc, const int32_t* offsets,
                                                             float* logits, int Hq, int Hkv, int G, int C, float scale)
{
    const int pair = blockIdx.x, b = pair / Hkv, j = pair - b * Hkv;
    const int c0 = blockIdx.y * kLogitClusters;
    const int32_t* off = offsets + (size_t)pair * (C + 1);
    for (int it = threadIdx.x; it < kLogitClusters * G; it += 256) {
        const int c = c0 + it / G, g = it - (it / G) * G;
        if (c >= C) continue;
        const int h = j * G + g;
        const int cnt = off[c + 1] - off[c];
        float v = kNegInf;
        if (cnt > 0) {
            float acc = 0.0f;
            for (int t = 0; t < D; ++t) {
                float qv, kv;
                if constexpr (DT == DT_F32) {
                    qv = reinterpret_cast<const float*>(q)[((size_t)b * Hq + h) * D + t];
                    kv = reinterpret_cast<const float*>(Kc)[((size_t)pair * C + c) * D + t];
                } else {
                    qv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(q)[((size_t)b * Hq + h) * D + t] << 16);
                    kv = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(Kc)[((size_t)pair * C + c) * D + t]
                                         << 16);
                }
                acc = fmaf(qv, kv, acc);
            }
            v = fmaf(acc, scale, logf((float)cnt));
        }
        logits[((size_t)b * Hq + h) * C + c] = v;
    }
}

// ---- decode: attention over the selected clusters and the proxies ----------

constexpr int kClusterWaves = 8;

struct ClusterAttnParams {
    const char* q;
    const char* Kg;
    const char* Vg;
    const char* Kc;
    const char* Vc;
    const int32_t* offsets;
    const int32_t* sel;
    float* out;
    float* lse;
    int Hq, Hkv, G, n, C, k, proxies;
    float scale_log2;
};

// One workgroup per (KV head, chunk of HG query heads).  Rows: the C proxies (tiles of 32; a proxy of a
// selected or empty cluster has log-weight -inf), then the tokens of the
// selected clusters, sel order, each cluster's rows contiguous in Kg / Vg.
template <int D, int HG>
__global__ void __launch_bounds__(kClusterWaves * 64) cluster_attn_kernel(const ClusterAttnParams p)
{
    constexpr int NW = kClusterWaves, TR = kTileRows;
    using E = MfmaEngine<D, HG, NW>;
    constexpr int RB = E::RB;
    __shared__ typename E::Smem sm;
    __shared__ int32_t cum_sm[kClusterMaxSel + 1];  // first exact row of each selected cluster
    __shared__ int32_t start_sm[kClusterMaxSel];    // its first row in Kg / Vg
    __shared__ uint32_t bits_sm[kClusterMaxClusters / 32];

    const int pair = blockIdx.x, b = pair / p.Hkv, j = pair - b * p.Hkv;
    const int nh = min(HG, p.G - (int)blockIdx.y * HG);
    const int h0 = j * p.G + blockIdx.y * HG;
    const int32_t* off = p.offsets + (size_t)pair * (p.C + 1);
    for (int w = threadIdx.x; w < (p.C + 31) / 32; w += NW * 64) bits_sm[w] = 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int s = 0; s < p.k; ++s) {
            const int c = p.sel[(size_t)pair * p.k + s];
            const bool ok = c >= 0 && c < p.C;
            cum_sm[s] = acc;
            start_sm[s] = ok ? off[c] : 0;
            acc += ok ? off[c + 1] - off[c] : 0;
            if (ok) bits_sm[c >> 5] |= 1u << (c & 31);
        }
        cum_sm[p.k] = acc;
    }
    __syncthreads();

    E eng(sm, p.q + (size_t)(b * p.Hq + h0) * RB, nh);
    const int lane = eng.lane, wave = eng.wave;
    const int exact = cum_sm[p.k];
    const int nP = p.proxies ? (p.C + TR - 1) / TR : 0;
    const int nT = nP + (exact + TR - 1) / TR;
    const int Tw = wave < nT ? (nT - wave + NW - 1) / NW : 0;
    const char* const kc = p.Kg + (size_t)pair * p.n * RB;
    const char* const vc = p.Vg + (size_t)pair * p.n * RB;
    const char* const ks = p.Kc + (size_t)pair * p.C * RB;
    const char* const vs = p.Vc + (size_t)pair * p.C * RB;
    const uint32_t cbytes = (uint32_t)p.n * RB, sbytes = (uint32_t)p.C * RB;

    auto set_rows = [&](int t, int tb) {
        if (lane < TR) {
            uint32_t row;
            float lw = kNegInf;
            if (t < nP) {  // proxy of cluster c
                const int c = t * TR + lane;
                row = (uint32_t)p.C;  // past the buffer: zeros, no traffic
                if (c < p.C) {
                    const int cnt = off[c + 1] - off[c];
                    row = (uint32_t)c;
                    if (cnt > 0 && !((bits_sm[c >> 5] >> (c & 31)) & 1u)) lw = log2f((float)cnt);
                }
            } else {  // exact row e of the selected clusters' tokens
                const int e = (t - nP) * TR + lane;
                row = (uint32_t)p.n;
                if (e < exact) {  // the last selected cluster whose rows start at or before e
                    int s = 0, hi = p.k;
                    while (hi - s > 1) {
                        const int mid = (s + hi) >> 1;
                        if (cum_sm[mid] <= e) s = mid;
                        else hi = mid;
                    }
                    row = (uint32_t)(start_sm[s] + (e - cum_sm[s]));
                    lw = 0.0f;
                }
            }
            eng.set_row(tb, lane, row, lw);
        }
    };
    auto rsrc = [&](int t, bool keys) {
        const bool proxy = t < nP;  // uniform over the wave
        const uint32_t bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)(proxy ? sbytes : cbytes));
        return buffer_rsrc(proxy ? (keys ? ks : vs) : (keys ? kc : vc), bytes);
    };
    auto issue = [&](int jt, typename E::Tile& tile, int tb) {
        const bool live = jt < Tw;
        const int t = live ? wave + jt * NW : 0;
        if (live) set_rows(t, tb);
        const __amdgpu_buffer_rsrc_t kr = live ? rsrc(t, true) : buffer_rsrc(kc, 0u);
        const __amdgpu_buffer_rsrc_t vr = live ? rsrc(t, false) : buffer_rsrc(vc, 0u);
        eng.issue(tile, tb, kr, vr, true);
    };
    auto compute = [&](const typename E::Tile& tile, int tb) {
        float x[8];
        eng.logits_mfma(tile, tb, p.scale_log2, x);
        eng.softmax(x);
    };

    typename E::Tile A, B;
    issue(0, A, 0);
    int jt = 0;
    for (; jt + 1 < Tw; jt += 2) {
        compute(A, 0);
        issue(jt + 1, B, 1);
        eng.accumulate(A);
        compute(B, 1);
        issue(jt + 2, A, 0);
        eng.accumulate(B);
    }
    if (jt < Tw) {
        compute(A, 0);
        eng.accumulate(A);
    }
    eng.finish(nh, p.out + ((size_t)b * p.Hq + h0) * D, p.lse ? p.lse + (size_t)b * p.Hq + h0 : nullptr, nullptr);
}

template <int R>
hipError_t build_r(const Dims& s, const ClusterBuild& cb, hipStream_t st)
{
    const int pairs = s.pairs(), n = s.n, C = cb.C;
    double* P = cb.proj;
    double* cent = cb.cent;
    const dim3 tgrid((unsigned)((n + kProjThreads - 1) / kProjThreads), (unsigned)pairs);
    if (s.dtype == DT_BF16) {
        if (s.d == 128) project_kernel<DT_BF16, 128, R><<<tgrid, kProjThreads, 0, st>>>((const char*)cb.K, cb.U, P, n);
        else project_kernel<DT_BF16, 64, R><<<tgrid, kProjThreads, 0, st>>>((const char*)cb.K, cb.U, P, n);
    } else {
        if (s.d == 128) project_kernel<DT_F32, 128, R><<<tgrid, kProjThreads, 0, st>>>((const char*)cb.K, cb.U, P, n);
        else project_kernel<DT_F32, 64, R><<<tgrid, kProjThreads, 0, st>>>((const char*)cb.K, cb.U, P, n);
    }
    seed_kernel<R><<<dim3((unsigned)pairs), 256, 0, st>>>(P, cb.seeds, cent, n, C);
    const size_t cent_lds = (size_t)C * R * sizeof(double);
    const unsigned upd_y = (unsigned)((C * R + 255) / 256 < 16 ? (C * R + 255) / 256 : 16);
    for (int it = 0; it <= cb.iters; ++it) {
        assign_kernel<R><<<tgrid, kProjThreads, cent_lds, st>>>(P, cent, cb.assign, n, C);
        sort_kernel<<<dim3((unsigned)pairs), 256, (size_t)C * sizeof(int32_t), st>>>(cb.assign, cb.order, cb.offsets,
                                                                                     n, C);
        if (it < cb.iters)
            update_kernel<R><<<dim3((unsigned)pairs, upd_y), 256, 0, st>>>(P, cb.order, cb.offsets, cent, n, C);
    }
    return hipGetLastError();
}

}  // namespace

bool cluster_build_ok(int C, int r)
{
    return C >= 1 && C <= kClusterMaxClusters && (r == 4 || r == 8 || r == 16 || r == 32) &&
           (size_t)C * r * sizeof(double) <= kClusterCentroidLds;
}

size_t cluster_build_ws_bytes(const Dims& s, int C, int r)
{
    const size_t a = ((size_t)s.pairs() * s.n * r * sizeof(double) + 255) & ~(size_t)255;
    return a + (size_t)s.pairs() * C * r * sizeof(double);
}

hipError_t launch_cluster_build(const Dims& s, const ClusterBuild& cb, hipStream_t st)
{
    hipError_t e = cb.r == 4    ? build_r<4>(s, cb, st)
                   : cb.r == 8  ? build_r<8>(s, cb, st)
                   : cb.r == 16 ? build_r<16>(s, cb, st)
                                : build_r<32>(s, cb, st);
    if (e != hipSuccess) return e;
    const int pairs = s.pairs(), n = s.n;
    const int rb = s.d * (s.dtype == DT_F32 ? 4 : 2), rpb = 256 / (rb / 16);
    const dim3 g((unsigned)((n + rpb - 1) / rpb), (unsigned)pairs);
    const char* K = static_cast<const char*>(cb.K);
    const char* V = static_cast<const char*>(cb.V);
    char* Kg = static_cast<char*>(cb.Kg);
    char* Vg = static_cast<char*>(cb.Vg);
    switch (rb) {
    case 128: gather_kernel<128><<<g, 256, 0, st>>>(K, V, cb.order, Kg, Vg, n); break;
    case 256: gather_kernel<256><<<g, 256, 0, st>>>(K, V, cb.order, Kg, Vg, n); break;
    default: gather_kernel<512><<<g, 256, 0, st>>>(K, V, cb.order, Kg, Vg, n); break;
    }
    const dim3 mg((unsigned)cb.C, (unsigned)pairs);
    char* Kc = static_cast<char*>(cb.Kc);
    char* Vc = static_cast<char*>(cb.Vc);
    if (s.dtype == DT_BF16) {
        if (s.d == 128) means_kernel<DT_BF16, 128><<<mg, 128, 0, st>>>(Kg, Vg, cb.offsets, Kc, Vc, n, cb.C);
        else means_kernel<DT_BF16, 64><<<mg, 64, 0, st>>>(Kg, Vg, cb.offsets, Kc, Vc, n, cb.C);
    } else {
        if (s.d == 128) means_kernel<DT_F32, 128><<<mg, 128, 0, st>>>(Kg, Vg, cb.offsets, Kc, Vc, n, cb.C);
        else means_kernel<DT_F32, 64><<<mg, 64, 0, st>>>(Kg, Vg, cb.offsets, Kc, Vc, n, cb.C);
    }
    return hipGetLastError();
}

hipError_t launch_cluster_logits(const Dims& s, int C, const void* q, const void* Kc, const int32_t* offsets,
                                 float* logits, hipStream_t st)
{
    const dim3 g((unsigned)s.pairs(), (unsigned)((C + kLogitClusters - 1) / kLogitClusters));
    const char* qc = static_cast<const char*>(q);
    const char* kc = static_cast<const char*>(Kc);
    if (s.dtype == DT_BF16) {
        if (s.d == 128) cluster_logits_kernel<DT_BF16, 128><<<g, 256, 0, st>>>(qc, kc, offsets, logits, s.Hq, s.Hkv, s.G, C, s.scale);
        else cluster_logits_kernel<DT_BF16, 64><<<g, 256, 0, st>>>(qc, kc, offsets, logits, s.Hq, s.Hkv, s.G, C, s.scale);
    } else {
        if (s.d == 128) cluster_logits_kernel<DT_F32, 128><<<g, 256, 0, st>>>(qc, kc, offsets, logits, s.Hq, s.Hkv, s.G, C, s.scale);
        else cluster_logits_kernel<DT_F32, 64><<<g, 256, 0, st>>>(qc, kc, offsets, logits, s.Hq, s.Hkv, s.G, C, s.scale);
    }
    return hipGetLastError();
}

hipError_t launch_cluster_attention(const Dims& s, const ClusterAttn& ca, hipStream_t st)
{
    ClusterAttnParams p{};
    p.q = static_cast<const char*>(ca.q);
    p.Kg = static_cast<const char*>(ca.Kg);
    p.Vg = static_cast<const char*>(ca.Vg);
    p.Kc = static_cast<const char*>(ca.Kc);
    p.Vc = static_cast<const char*>(ca.Vc);
    p.offsets = ca.offsets;
    p.sel = ca.sel;
    p.out = ca.out;
    p.lse = ca.lse;
    p.Hq = s.Hq;
    p.Hkv = s.Hkv;
    p.G = s.G;
    p.n = s.n;
    p.C = ca.C;
    p.k = ca.k;
    p.proxies = ca.proxies;
    p.scale_log2 = s.scale * kLog2e;
    // all heads of a KV head (up to 8) share a workgroup, so its cluster rows are
    // read once (with P V on the matrix cores eight heads fit two waves per SIMD)
    const int hg = s.G;
    const dim3 grid((unsigned)s.pairs(), (unsigned)((s.G + hg - 1) / hg)), block(kClusterWaves * 64);
#define CSA_CLUSTER_ATTN(D)                                                                \
    switch (hg) {                                                                          \
    case 1: cluster_attn_kernel<D, 1><<<grid, block, 0, st>>>(p); break;                   \
    case 2: cluster_attn_kernel<D, 2><<<grid, block, 0, st>>>(p); break;                   \
    case 3: cluster_attn_kernel<D, 3><<<grid, block, 0, st>>>(p); break;                   \
    case 4: cluster_attn_kernel<D, 4><<<grid, block, 0, st>>>(p); break;                   \
    case 5: cluster_attn_kernel<D, 5><<<grid, block, 0, st>>>(p); break;                   \
    case 6: cluster_attn_kernel<D, 6><<<grid, block, 0, st>>>(p); break;                   \
    case 7: cluster_attn_kernel<D, 7><<<grid, block, 0, st>>>(p); break;                   \
    case 8: cluster_attn_kernel<D, 8><<<grid, block, 0, st>>>(p); break;                   \
    default: return hipErrorInvalidValue;                                                  \
    }
    if (s.d == 128) {
        CSA_CLUSTER_ATTN(128)
    } else {
        CSA_CLUSTER_ATTN(64)
    }
#undef CSA_CLUSTER_ATTN
    return hipGetLastError();
}

}  // namespace csa

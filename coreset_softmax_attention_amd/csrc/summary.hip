// summary.hip -- per-block mean key and mean value; the key box and the
// variance token of the alternative block scores.
//
// The count-aware proxy of an unread block is one virtual token whose value is
// the mean value of the block's tokens ("OpenAttention reads 1% of the KV cache
// -- Count-aware tail proxy", section "Skipping reviews without losing the
// verdict"); its key is the mean key, the mean-pool summary of "COBS: Cumulant
// Order Block Sparse Attention", Eq. (18).
//
// Each lane owns one 16-byte chunk of a row; the LPR lanes of a lane group own
// one block and walk its tokens in order, summing in fp64.  The sums are then
// divided by the block's token count in fp64 and rounded once to the storage
// type (round to nearest, ties to even).  Summing token by token in fp64 makes
// the result independent of any reduction tree.
#include "device.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kNW = 4;
constexpr int kU = 8;  // rows in flight per lane group and tensor

template <int DT, int D>
__global__ void __launch_bounds__(kNW * 64)
    summary_kernel(const char* K, const char* V, char* Kbar, char* Vbar, int n, int L, int nb, long long total)
{
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const long long gblk = ((long long)blockIdx.x * kNW + wave) * RPW + gi;
    if (gblk >= total) return;  // no cross-lane operations below
    const long long pair = gblk / nb;
    const int blk = (int)(gblk - pair * nb);
    const int t0 = blk * L, c = min(L, n - t0);
    const char* kp = K + ((size_t)pair * n + t0) * RB + li * 16;
    const char* vp = V + ((size_t)pair * n + t0) * RB + li * 16;

    double sk[EPL], sv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) sk[e] = sv[e] = 0.0;

    for (int i = 0; i < c; i += kU) {
        uint4 kr[kU], vr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int t = min(i + u, c - 1);
            kr[u] = ld16_nt(kp + (size_t)t * RB);
            vr[u] = ld16_nt(vp + (size_t)t * RB);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (i + u < c) {  // tokens in order
                float kf[EPL], vf[EPL];
                unpack<DT>(kr[u], kf);
                unpack<DT>(vr[u], vf);
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    sk[e] += (double)kf[e];
                    sv[e] += (double)vf[e];
                }
            }
        }
    }

    const double cd = (double)c;
    const size_t out_off = ((size_t)pair * nb + blk) * RB + li * 16;
    uint32_t wk[4], wv[4];
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wk[e] = __float_as_uint((float)(sk[e] / cd));
            wv[e] = __float_as_uint((float)(sv[e] / cd));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wk[e] = (uint32_t)bf16_from_f64(sk[2 * e] / cd) | ((uint32_t)bf16_from_f64(sk[2 * e + 1] / cd) << 16);
            wv[e] = (uint32_t)bf16_from_f64(sv[2 * e] / cd) | ((uint32_t)bf16_from_f64(sv[2 * e + 1] / cd) << 16);
        }
    }
    *reinterpret_cast<uint4*>(Kbar + out_off) = make_uint4(wk[0], wk[1], wk[2], wk[3]);
    *reinterpret_cast<uint4*>(Vbar + out_off) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

template <int DT, int D>
hipError_t launch_dtd(const Dims& s, const void* K, const void* V, void* Kbar, void* Vbar, hipStream_t st)
{
    using Gm = RowGeom<DT, D>;
    const long long total = (long long)s.pairs() * s.nb;
    const long long per_wg = (long long)kNW * Gm::rpw;
    const long long wgs = (total + per_wg - 1) / per_wg;
    summary_kernel<DT, D><<<dim3((unsigned)wgs), dim3(kNW * 64), 0, st>>>(
        static_cast<const char*>(K), static_cast<const char*>(V), static_cast<char*>(Kbar), static_cast<char*>(Vbar),
        s.n, s.L, s.nb, total);
    return hipGetLastError();
}

// Box summaries (Quest, as analysed in "COBS: Cumulant Order Block Sparse
// Attention", section on escaping the first-order ceiling): the element-wise
// minimum and maximum of each block's keys, Kbox [pairs, nb, 2, d].  Strict
// comparisons in token order keep the first of equal values (so -0 and +0
// resolve the same way everywhere); a minimum or maximum of stored values is a
// stored value, so nothing is rounded.
template <int DT, int D>
__global__ void __launch_bounds__(kNW * 64) box_kernel(const char* K, char* Kbox, int n, int L, int nb, long long total)
{
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const long long gblk = ((long long)blockIdx.x * kNW + wave) * RPW + gi;
    if (gblk >= total) return;  // no cross-lane operations below
    const long long pair = gblk / nb;
    const int blk = (int)(gblk - pair * nb);
    const int t0 = blk * L, c = min(L, n - t0);
    const char* kp = K + ((size_t)pair * n + t0) * RB + li * 16;

    float lo[EPL], hi[EPL];
    {
        float kf[EPL];
        unpack<DT>(ld16_nt(kp), kf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) lo[e] = hi[e] = kf[e];
    }
    for (int i = 1; i < c; i += kU) {
        uint4 kr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) kr[u] = ld16_nt(kp + (size_t)min(i + u, c - 1) * RB);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (i + u < c) {  // tokens in order
                float kf[EPL];
                unpack<DT>(kr[u], kf);
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    if (kf[e] < lo[e]) lo[e] = kf[e];
                    if (kf[e] > hi[e]) hi[e] = kf[e];
                }
            }
        }
    }
    uint32_t wl[4], wh[4];
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wl[e] = __float_as_uint(lo[e]);
            wh[e] = __float_as_uint(hi[e]);
        }
    } else {  // the values are bfloat16 widened exactly: keep their upper halves
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wl[e] = (__float_as_uint(lo[2 * e]) >> 16) | (__float_as_uint(lo[2 * e + 1]) & 0xffff0000u);
            wh[e] = (__float_as_uint(hi[2 * e]) >> 16) | (__float_as_uint(hi[2 * e + 1]) & 0xffff0000u);
        }
    }
    char* out = Kbox + ((size_t)pair * nb + blk) * 2 * RB + li * 16;
    *reinterpret_cast<uint4*>(out) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    *reinterpret_cast<uint4*>(out + RB) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
}

template <int DT, int D>
hipError_t launch_box_dtd(const Dims& s, const void* K, void* Kbox, hipStream_t st)
{
    using Gm = RowGeom<DT, D>;
    const long long total = (long long)s.pairs() * s.nb;
    const long long per_wg = (long long)kNW * Gm::rpw;
    const long long wgs = (total + per_wg - 1) / per_wg;
    box_kernel<DT, D><<<dim3((unsigned)wgs), dim3(kNW * 64), 0, st>>>(static_cast<const char*>(K),
                                                                        static_cast<char*>(Kbox), s.n, s.L, s.nb, total);
    return hipGetLastError();
}

// Mean and variance tokens (the proxy-error ranking of "OpenAttention reads 1%
// of the KV cache -- Count-aware tail proxy", section "Three helpers that make
// the proxy accurate"): Kvar [pairs, nb, 2, d], row 0 the mean key (the bits of
// the summary kernel: token-order fp64 sum over the count, rounded once), row 1
// the per-coordinate variance about the exact fp64 mean, (1/c) sum_i (k_i -
// mean)^2, also summed token by token in fp64 (no fused multiply-add, so the
// sum is the same sequence of roundings everywhere) and rounded once.  The
// keys are read twice; the second pass finds them in cache.
template <int DT, int D>
__global__ void __launch_bounds__(kNW * 64) var_kernel(const char* K, char* Kvar, int n, int L, int nb, long long total)
{
#pragma clang fp contract(off)
    using Gm = RowGeom<DT, D>;
    constexpr int LPR = Gm::lpr, RPW = Gm::rpw, EPL = Gm::epl, RB = Gm::row_bytes;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int gi = lane / LPR, li = lane % LPR;
    const long long gblk = ((long long)blockIdx.x * kNW + wave) * RPW + gi;
    if (gblk >= total) return;  // no cross-lane operations below
    const long long pair = gblk / nb;
    const int blk = (int)(gblk - pair * nb);
    const int t0 = blk * L, c = min(L, n - t0);
    const char* kp = K + ((size_t)pair * n + t0) * RB + li * 16;

    double s1[EPL], s2[EPL], mean[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) s1[e] = s2[e] = 0.0;
    for (int i = 0; i < c; i += kU) {
        uint4 kr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) kr[u] = ld16(kp + (size_t)min(i + u, c - 1) * RB);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (i + u < c) {  // tokens in order
                float kf[EPL];
                unpack<DT>(kr[u], kf);
#pragma unroll
                for (int e = 0; e < EPL; ++e) s1[e] += (double)kf[e];
            }
        }
    }
    const double cd = (double)c;
#pragma unroll
    for (int e = 0; e < EPL; ++e) mean[e] = s1[e] / cd;
    for (int i = 0; i < c; i += kU) {
        uint4 kr[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) kr[u] = ld16_nt(kp + (size_t)min(i + u, c - 1) * RB);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (i + u < c) {
                float kf[EPL];
                unpack<DT>(kr[u], kf);
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    const double dv = (double)kf[e] - mean[e];
                    s2[e] += dv * dv;
                }
            }
        }
    }
    uint32_t wm[4], wv[4];
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wm[e] = __float_as_uint((float)mean[e]);
            wv[e] = __float_as_uint((float)(s2[e] / cd));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wm[e] = (uint32_t)bf16_from_f64(mean[2 * e]) | ((uint32_t)bf16_from_f64(mean[2 * e + 1]) << 16);
            wv[e] = (uint32_t)bf16_from_f64(s2[2 * e] / cd) | ((uint32_t)bf16_from_f64(s2[2 * e + 1] / cd) << 16);
        }
    }
    char* out = Kvar + ((size_t)pair * nb + blk) * 2 * RB + li * 16;
    *reinterpret_cast<uint4*>(out) = make_uint4(wm[0], wm[1], wm[2], wm[3]);
    *reinterpret_cast<uint4*>(out + RB) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

template <int DT, int D>
hipError_t launch_var_dtd(const Dims& s, const void* K, void* Kvar, hipStream_t st)
{
    using Gm = RowGeom<DT, D>;
    const long long total = (long long)s.pairs() * s.nb;
    const long long per_wg = (long long)kNW * Gm::rpw;
    const long long wgs = (total + per_wg - 1) / per_wg;
    var_kernel<DT, D><<<dim3((unsigned)wgs), dim3(kNW * 64), 0, st>>>(static_cast<const char*>(K),
                                                                        static_cast<char*>(Kvar), s.n, s.L, s.nb, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_var(const Dims& s, const void* K, void* Kvar, hipStream_t st)
{
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_var_dtd<DT_BF16, 128>(s, K, Kvar, st);
        if (s.d == 64) return launch_var_dtd<DT_BF16, 64>(s, K, Kvar, st);
    } else {
        if (s.d == 128) return launch_var_dtd<DT_F32, 128>(s, K, Kvar, st);
        if (s.d == 64) return launch_var_dtd<DT_F32, 64>(s, K, Kvar, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_box(const Dims& s, const void* K, void* Kbox, hipStream_t st)
{
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_box_dtd<DT_BF16, 128>(s, K, Kbox, st);
        if (s.d == 64) return launch_box_dtd<DT_BF16, 64>(s, K, Kbox, st);
    } else {
        if (s.d == 128) return launch_box_dtd<DT_F32, 128>(s, K, Kbox, st);
        if (s.d == 64) return launch_box_dtd<DT_F32, 64>(s, K, Kbox, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_summary(const Dims& s, const void* K, const void* V, void* Kbar, void* Vbar, hipStream_t st)
{
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_dtd<DT_BF16, 128>(s, K, V, Kbar, Vbar, st);
        if (s.d == 64) return launch_dtd<DT_BF16, 64>(s, K, V, Kbar, Vbar, st);
    } else {
        if (s.d == 128) return launch_dtd<DT_F32, 128>(s, K, V, Kbar, Vbar, st);
        if (s.d == 64) return launch_dtd<DT_F32, 64>(s, K, V, Kbar, Vbar, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa

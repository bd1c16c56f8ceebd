// cov.hip -- second-order block descriptors of "COBS: Cumulant Order Block
// Sparse Attention": per block the mean key and the top-r scaled eigenvectors
// xi_i = sqrt(lambda_i) u_i of the within-block key covariance
// Sigma_b = (1/c) sum_i (k_i - kbar)(k_i - kbar)^T (the second cumulant of the
// block's keys, kept in the low-rank spectral form of the section on
// compressing the covariance).  Output Kcov [pairs, nb, 1 + r, d]: row 0 the
// mean key (the same bits as kv_summary_build), rows 1..r the xi_i by
// decreasing eigenvalue, each signed so that its largest-magnitude coordinate
// is positive (the first such coordinate on ties).
//
// One wave per block (c <= 64 tokens).  With X the centred c x d key matrix,
// the nonzero spectrum of Sigma is that of the c x c Gram matrix G = X X^T
// over c: if G v = mu v with |v| = 1 then xi = X^T v / sqrt(c) (its squared
// norm is mu / c = lambda).  Lane l owns row l of X (in LDS) and of G (in
// registers).  The top eigenvectors of G come from a Lanczos run with full
// reorthogonalisation run to the whole Krylov space (so the Ritz pairs are the
// eigenpairs); the Ritz values are found by bisection on Sturm counts
// of the tridiagonal matrix, all 64 lanes testing shifts at once, and their
// vectors by inverse iteration.  Everything is fp32 except the mean.
#include "device.hpp"
#include "launch.hpp"

namespace csa {
namespace {

constexpr int kCovWaves = 2;    // waves (blocks) per workgroup
constexpr int kCovMaxRows = 64; // tokens per block
constexpr int kLanczos = 64;    // Lanczos steps: the whole Krylov space of a 64-token block

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// LDS of one wave.
template <int D>
struct CovSmem {
    float x[kCovMaxRows][D + 1];  // centred keys (+1: no bank conflicts on column walks)
    float v[kLanczos + 1][kCovMaxRows];  // Lanczos vectors
    float alpha[kLanczos], beta[kLanczos];
    float theta[4];               // Ritz values, largest first
    float y[4][kLanczos];         // their eigenvectors of the tridiagonal matrix
    float cp[4][kLanczos], dp[4][kLanczos];  // tridiagonal elimination
};

template <int DT, int D, int R>
__global__ void __launch_bounds__(kCovWaves * 64) cov_kernel(const char* K, char* Kcov, int n, int L, int nb,
                                                             long long total)
{
    constexpr int RB = D * Elem<DT>::bytes;  // bytes per key row
    constexpr int CPL = D / 64;              // columns per lane
    __shared__ CovSmem<D> smem[kCovWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    CovSmem<D>& sm = smem[wave];
    const long long gblk = (long long)blockIdx.x * kCovWaves + wave;
    if (gblk >= total) return;  // whole wave; no workgroup barrier in this kernel
    const long long pair = gblk / nb;
    const int blk = (int)(gblk - pair * nb);
    const int t0 = blk * L, c = min(L, n - t0);
    const char* kp = K + ((size_t)pair * n + t0) * RB;
    char* out = Kcov + ((size_t)pair * nb + blk) * (1 + R) * RB;

    // ---- keys -> LDS (row per lane), mean row (fp64, token order, one rounding)
    if (lane < c) {
#pragma unroll
        for (int ch = 0; ch < RB / 16; ++ch) {
            float f[Elem<DT>::per16];
            unpack<DT>(ld16(kp + (size_t)lane * RB + ch * 16), f);
#pragma unroll
            for (int e = 0; e < Elem<DT>::per16; ++e) sm.x[lane][ch * Elem<DT>::per16 + e] = f[e];
        }
    } else {
        for (int t = 0; t < D; ++t) sm.x[lane][t] = 0.0f;
    }
    wave_lds_fence();
    double mean[CPL];
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
        const int t = lane + 64 * u;
        double s = 0.0;
        for (int i = 0; i < c; ++i) s += (double)sm.x[i][t];
        mean[u] = s / (double)c;
    }
#pragma unroll
    for (int u = 0; u < CPL; ++u) {
        const int t = lane + 64 * u;
        if constexpr (DT == DT_F32) {
            reinterpret_cast<float*>(out)[t] = (float)mean[u];
        } else {
            reinterpret_cast<uint16_t*>(out)[t] = bf16_from_f64(mean[u]);
        }
    }
    // centre
    for (int i = 0; i < c; ++i) {
#pragma unroll
        for (int u = 0; u < CPL; ++u) sm.x[i][lane + 64 * u] -= (float)mean[u];
    }
    wave_lds_fence();

    // ---- Gram matrix row of this lane: g[j] = x_lane . x_j
    float g[kCovMaxRows];
#pragma unroll
    for (int j = 0; j < kCovMaxRows; ++j) g[j] = 0.0f;
    for (int t = 0; t < D; ++t) {
        const float xl = sm.x[lane][t];
#pragma unroll
        for (int j = 0; j < kCovMaxRows; ++j) g[j] = fmaf(xl, sm.x[j][t], g[j]);
    }
    if (lane >= c) {
#pragma unroll
        for (int j = 0; j < kCovMaxRows; ++j) g[j] = 0.0f;
    }

    // ---- Lanczos with full reorthogonalisation
    const int steps = min(kLanczos, c);
    // start: a fixed pseudo-random vector over the block's rows (the all-ones
    // vector is in G's null space: the rows are centred)
    float v = 0.0f;
    if (lane < c) {
        uint32_t h = (uint32_t)lane * 0x9E3779B1u + 0x7F4A7C15u;
        h ^= h >> 15;
        h *= 0x2C1B3C6Du;
        h ^= h >> 12;
        v = (float)(h & 0xFFFF) / 65536.0f + 0.5f;
    }
    v /= sqrtf(wave_sum(v * v));
    int m = 0;  // Lanczos vectors kept
    float gnorm = 0.0f;
    for (int k = 0; k < steps; ++k) {
        sm.v[k][lane] = v;
        wave_lds_fence();
        float w = 0.0f;
#pragma unroll
        for (int j = 0; j < kCovMaxRows; ++j) w = fmaf(g[j], sm.v[k][j], w);
        const float a = wave_sum(w * v);
        sm.alpha[k] = a;
        m = k + 1;
        // w -= a v + beta v_{k-1}, then against every kept vector, twice
        w -= a * v;
        if (k > 0) w -= sm.beta[k - 1] * sm.v[k - 1][lane];
        for (int pass = 0; pass < 2; ++pass)
            for (int i = 0; i <= k; ++i) {
                const float vi = sm.v[i][lane];
                w -= wave_sum(w * vi) * vi;
            }
        const float b = sqrtf(wave_sum(w * w));
        gnorm = fmaxf(gnorm, fabsf(a) + b);
        if (k + 1 == steps || b <= 1e-6f * gnorm) break;  // Krylov space exhausted
        sm.beta[k] = b;
        v = w / b;
    }
    wave_lds_fence();

    // ---- Ritz values: the R largest eigenvalues of the m x m tridiagonal T,
    // by multisection on Sturm counts (all lanes test one shift each)
    // number of eigenvalues of T below x
    auto below = [&](float x) {
        int cnt = 0;
        float dk = sm.alpha[0] - x;
        if (dk < 0.0f) ++cnt;
        for (int k = 1; k < m; ++k) {
            const float dd = dk == 0.0f ? 1e-30f : dk;
            dk = sm.alpha[k] - x - sm.beta[k - 1] * sm.beta[k - 1] / dd;
            if (dk < 0.0f) ++cnt;
        }
        return cnt;
    };
    float glo = 0.0f, ghi = 0.0f;  // Gershgorin interval
    for (int k = 0; k < m; ++k) {
        const float r = (k > 0 ? fabsf(sm.beta[k - 1]) : 0.0f) + (k + 1 < m ? fabsf(sm.beta[k]) : 0.0f);
        glo = fminf(glo, sm.alpha[k] - r);
        ghi = fmaxf(ghi, sm.alpha[k] + r);
    }
    ghi *= 1.0001f;
    for (int i = 0; i < R; ++i) {
        const int idx = m - 1 - i;  // eigenvalue index in ascending order
        float lo = glo, hi = ghi;
        if (idx >= 0) {
            for (int round = 0; round < 5; ++round) {
                // lane l tests lo + (l + 1) (hi - lo) / 65
                const float x = lo + (float)(lane + 1) * ((hi - lo) / 65.0f);
                const bool above = below(x) <= idx;  // the eigenvalue lies at or above x
                const uint64_t mk = __ballot(above);
                const int nab = __popcll(mk);  // lanes 0..nab-1 have x below the eigenvalue
                const float nlo = lo + (float)nab * ((hi - lo) / 65.0f);
                const float nhi = lo + (float)(nab + 1) * ((hi - lo) / 65.0f);
                lo = nlo;
                hi = nhi;
            }
        }
        if (lane == 0) sm.theta[i] = idx >= 0 ? fmaxf(0.5f * (lo + hi), 0.0f) : 0.0f;
    }
    wave_lds_fence();

    // ---- eigenvectors of T by inverse iteration (lane i < R solves for theta_i)
    if (lane < R) {
        float* y = sm.y[lane];
        float* cp = sm.cp[lane];
        float* dp = sm.dp[lane];
        const float th = sm.theta[lane] + 1e-6f * gnorm;  // a shift just off the eigenvalue
        const float tiny = 1e-12f * fmaxf(gnorm, 1e-30f);
        for (int k = 0; k < m; ++k) y[k] = 1.0f;
        for (int it = 0; it < 3; ++it) {
            // solve (T - th I) z = y by elimination on the tridiagonal
            float den = sm.alpha[0] - th;
            den = fabsf(den) < tiny ? (den < 0.0f ? -tiny : tiny) : den;
            cp[0] = m > 1 ? sm.beta[0] / den : 0.0f;
            dp[0] = y[0] / den;
            for (int k = 1; k < m; ++k) {
                den = sm.alpha[k] - th - sm.beta[k - 1] * cp[k - 1];
                den = fabsf(den) < tiny ? (den < 0.0f ? -tiny : tiny) : den;
                cp[k] = k + 1 < m ? sm.beta[k] / den : 0.0f;
                dp[k] = (y[k] - sm.beta[k - 1] * dp[k - 1]) / den;
            }
            y[m - 1] = dp[m - 1];
            for (int k = m - 2; k >= 0; --k) y[k] = dp[k] - cp[k] * y[k + 1];
            float nn = 0.0f;
            for (int k = 0; k < m; ++k) nn += y[k] * y[k];
            if (!(nn > 0.0f && nn < 3.0e38f)) {  // degenerate: fall back to a unit vector
                for (int k = 0; k < m; ++k) y[k] = k == 0 ? 1.0f : 0.0f;
                break;
            }
            const float inv = 1.0f / sqrtf(nn);
            for (int k = 0; k < m; ++k) y[k] *= inv;
        }
    }
    wave_lds_fence();

    // ---- xi_i = X^T (V y_i) / sqrt(c); sign: largest-magnitude coordinate positive
    const float inv_sqrt_c = 1.0f / sqrtf((float)c);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        // Ritz vector component of this lane's row, through LDS for the X^T product
        float z = 0.0f;
        for (int k = 0; k < m; ++k) z = fmaf(sm.v[k][lane], sm.y[i][k], z);
        if (i >= m) z = 0.0f;  // fewer Lanczos vectors than descriptors: nothing left
        wave_lds_fence();
        sm.v[kLanczos][lane] = z;
        wave_lds_fence();
        float xi[CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int t = lane + 64 * u;
            float s = 0.0f;
            for (int l = 0; l < c; ++l) s = fmaf(sm.x[l][t], sm.v[kLanczos][l], s);
            xi[u] = s * inv_sqrt_c;
        }
        // the first coordinate of largest magnitude decides the sign
        float best = -1.0f;
        int bt = 0;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const float a = fabsf(xi[u]);
            if (a > best) {
                best = a;
                bt = lane + 64 * u;
            }
        }
        // wave-wide (magnitude, -index) maximum
        uint32_t hkey = __float_as_uint(best), lkey = ~(uint32_t)bt;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const uint32_t oh = __shfl_xor(hkey, off), ol = __shfl_xor(lkey, off);
            if (oh > hkey || (oh == hkey && ol > lkey)) {
                hkey = oh;
                lkey = ol;
            }
        }
        const int at = (int)~lkey;
        float sgn_src = 0.0f;
#pragma unroll
        for (int u = 0; u < CPL; ++u)
            if (lane + 64 * u == at) sgn_src = xi[u];
        const float sgn = __shfl(sgn_src, at & 63) < 0.0f ? -1.0f : 1.0f;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
            const int t = lane + 64 * u;
            const float val = xi[u] * sgn;
            if constexpr (DT == DT_F32) {
                reinterpret_cast<float*>(out + (size_t)(1 + i) * RB)[t] = val;
            } else {
                reinterpret_cast<uint16_t*>(out + (size_t)(1 + i) * RB)[t] = bf16_from_f64((double)val);
            }
        }
    }
}

template <int DT, int D>
hipError_t launch_cov_dtd(const Dims& s, const void* K, void* Kcov, hipStream_t st)
{
    const long long total = (long long)s.pairs() * s.nb;
    const long long wgs = (total + kCovWaves - 1) / kCovWaves;
    cov_kernel<DT, D, kCobsRank><<<dim3((unsigned)wgs), dim3(kCovWaves * 64), 0, st>>>(
        static_cast<const char*>(K), static_cast<char*>(Kcov), s.n, s.L, s.nb, total);
    return hipGetLastError();
}

}  // namespace

bool cov_build_ok(const Dims& s)
{
    return s.L <= kCovMaxRows;
}

hipError_t launch_cov(const Dims& s, const void* K, void* Kcov, hipStream_t st)
{
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_cov_dtd<DT_BF16, 128>(s, K, Kcov, st);
        if (s.d == 64) return launch_cov_dtd<DT_BF16, 64>(s, K, Kcov, st);
    } else {
        if (s.d == 128) return launch_cov_dtd<DT_F32, 128>(s, K, Kcov, st);
        if (s.d == 64) return launch_cov_dtd<DT_F32, 64>(s, K, Kcov, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace csa

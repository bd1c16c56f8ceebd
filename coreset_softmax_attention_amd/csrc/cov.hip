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
// One workgroup of one wave per block (c <= 64 tokens; ~38 KiB of LDS, so four
// blocks share a compute unit).  With X the centred c x d key matrix, the
// nonzero spectrum of Sigma is that of the c x c Gram matrix G = X X^T over c:
// if G v = mu v with |v| = 1 then xi = X^T v / sqrt(c) (its squared norm is
// mu / c = lambda).  Lane l owns row l of X (in LDS) and of G (in registers).
// The top eigenvectors of G come from a Lanczos run with full
// reorthogonalisation (two batched classical Gram-Schmidt passes per step, no
// cross-lane sums) run to the whole Krylov space, so the Ritz pairs are the
// eigenpairs; the Ritz values are found by multisection on Sturm counts of the
// tridiagonal matrix (a group of 16 lanes per eigenvalue) and their vectors by
// inverse iteration; xi reads the keys again.  Everything is fp32 except the
// mean.
#include "device.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kCovMaxRows = 64; // tokens per block
constexpr int kLanczos = 64;    // Lanczos steps: the whole Krylov space of a 64-token block
constexpr int kSubMax = 128;    // query-subspace dimensions held per block (two columns per lane)

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// LDS of one wave (one block per workgroup).  The centred keys are needed only
// to form the Gram matrix; their space then holds the Lanczos vectors.  Rows
// are padded to a multiple of 4 floats plus 4, so that 16-byte row reads by 16
// lanes at once fall on distinct banks.
template <int D, bool SUB>
struct CovSmem {
    union {
        float x[kCovMaxRows][D + 4];  // centred keys
        struct {
            float v[kLanczos + 1][kCovMaxRows + 4];  // Lanczos vectors, row k = v_k
            float w[kCovMaxRows];                    // the vector being orthogonalised
            float h[kLanczos];                       // its coefficients on v_0 .. v_k
        } lz;
    };
    float alpha[kLanczos], beta[kLanczos];
    float theta[4];                          // Ritz values, largest first
    float y[4][kLanczos];                    // their eigenvectors of the tridiagonal matrix
    float cp[4][kLanczos], dp[4][kLanczos];  // tridiagonal elimination
    float z[4][kCovMaxRows];                 // Ritz vectors over the block's rows
    // query subspace: the centred keys' coordinates in it, row per token (kept
    // to the end: the factors are formed from them)
    float ys[SUB ? kCovMaxRows : 1][SUB ? kSubMax + 4 : 4];
};

// E2M1 code of r: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 by magnitude, ties to the
// even mantissa (code bit 0 clear); a zero magnitude is +0.
__device__ __forceinline__ uint32_t e2m1_code(float r)
{
    const float a = fabsf(r);
    const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f  ? 4u : a < 3.5f  ? 5u : a <= 5.0f  ? 6u : 7u;
    return c | ((r < 0.0f && c != 0u) ? 8u : 0u);
}

// FP4: the descriptor is stored as [mean: d bfloat16][R fp32 scales][R x d/2 bytes of
// E2M1 codes] per block (bfloat16 caches): each eigenvector, rounded to bfloat16 as
// in the plain descriptor, is divided by its scale max_t |xi_t| / 6 and rounded to
// E2M1; byte t of a row holds coordinates 2t (low nibble) and 2t + 1 (high nibble).
//
// SUB (the query-subspace descriptor of the same page: the covariance kept only
// within the span of the caller's basis U [Hkv, d, s], the top eigenvectors of the
// queries' second moment): the centred keys are projected on U first (Y = X U,
// fp32, the d products of a coordinate in order), the Gram matrix is Y Y^T, and
// the factors xi = Y^T v / sqrt(c) are the scaled eigenvectors of U^T Sigma U.
// Stored as [mean: d][R x sps] per block, sps = s rounded up to 8 (zeros after s).
template <int DT, int D, int R, bool FP4, bool SUB>
__global__ void __launch_bounds__(64) cov_kernel(const char* K, char* Kcov, int n, int L, int nb, const float* U,
                                                 int s_dim, int Hkv)
{
    constexpr int EB = Elem<DT>::bytes;
    constexpr int RB = D * EB;      // bytes per key row
    constexpr int CPL = D / 64;     // columns per lane: lane owns CPL lane .. CPL lane + CPL - 1
    static_assert(R <= 4, "at most four descriptors");
    __shared__ CovSmem<D, SUB> sm;
    const int lane = threadIdx.x;
    const long long gblk = blockIdx.x;
    const long long pair = gblk / nb;
    const int blk = (int)(gblk - pair * nb);
    const int t0 = blk * L, c = min(L, n - t0);
    const char* kp = K + ((size_t)pair * n + t0) * RB;
    static_assert(!FP4 || (DT == DT_BF16 && (D == 128 || D == 64)), "FP4 descriptors are for bfloat16 caches");
    static_assert(!(SUB && FP4) || kSubMax == 128, "two subspace coordinates per lane");
    const int sps = SUB ? (s_dim + 7) / 8 * 8 : 0;     // stored subspace row length
    const int spf = SUB ? (s_dim + 31) / 32 * 32 : 0;  // FP4 subspace factor: coordinates with codes
    const int BB = FP4 ? (SUB ? 2 * D + 4 * R + R * spf / 2 : 2 * D + 4 * R + R * D / 2)
                       : SUB ? RB + R * sps * EB : (1 + R) * RB;  // bytes per block
    char* out = Kcov + ((size_t)pair * nb + blk) * BB;

    // ---- keys -> LDS (row per lane), mean of this lane's columns (fp64, token
    // order, one rounding: the bits of the summary)
    if (lane < c) {
#pragma unroll
        for (int ch = 0; ch < RB / 16; ++ch) {
            float f[Elem<DT>::per16];
            unpack<DT>(ld16(kp + (size_t)lane * RB + ch * 16), f);
#pragma unroll
            for (int e = 0; e < Elem<DT>::per16; e += 4)
                *reinterpret_cast<float4*>(&sm.x[lane][ch * Elem<DT>::per16 + e]) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
        }
    } else {
        for (int t = 0; t < D; t += 4) *reinterpret_cast<float4*>(&sm.x[lane][t]) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    wave_lds_fence();
    double mean[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
        const int t = CPL * lane + e;
        double s = 0.0;
        for (int i = 0; i < c; ++i) s += (double)sm.x[i][t];
        mean[e] = s / (double)c;
    }
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) reinterpret_cast<float*>(out)[CPL * lane + e] = (float)mean[e];
    } else {
#pragma unroll
        for (int e = 0; e < CPL; ++e) reinterpret_cast<uint16_t*>(out)[CPL * lane + e] = bf16_from_f64(mean[e]);
    }
    float meanf[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) meanf[e] = (float)mean[e];
    // centre (rows past the block stay zero)
    for (int i = 0; i < c; ++i) {
#pragma unroll
        for (int e = 0; e < CPL; ++e) sm.x[i][CPL * lane + e] -= meanf[e];
    }
    wave_lds_fence();

    // ---- query subspace: this lane's row of Y = X U, eight columns at a time
    // (U's rows are the same for every lane: scalar loads), zero past s
    const int syp = SUB ? (s_dim + 3) / 4 * 4 : 0;  // Y columns the Gram matrix reads
    if constexpr (SUB) {
        const float* Uj = U + (size_t)(pair % Hkv) * D * s_dim;
        for (int c0 = 0; c0 < syp; c0 += 8) {
            float acc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
            for (int t = 0; t < D; ++t) {
                const float xv = sm.x[lane][t];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(xv, c0 + e < s_dim ? Uj[(size_t)t * s_dim + c0 + e] : 0.0f, acc[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (c0 + e < syp) sm.ys[lane][c0 + e] = acc[e];
        }
        wave_lds_fence();
    }

    // ---- Gram matrix row of this lane: g[j] = x_lane . x_j (16-byte LDS reads;
    // of the subspace coordinates y with SUB)
    float g[kCovMaxRows];
#pragma unroll
    for (int j = 0; j < kCovMaxRows; ++j) g[j] = 0.0f;
    auto gram = [&](const float* rows, int stride, int cols) {
        for (int t = 0; t < cols; t += 4) {
            const float4 xl = *reinterpret_cast<const float4*>(rows + lane * stride + t);
#pragma unroll
            for (int j = 0; j < kCovMaxRows; ++j) {
                const float4 xj = *reinterpret_cast<const float4*>(rows + j * stride + t);
                g[j] = fmaf(xl.x, xj.x, g[j]);
                g[j] = fmaf(xl.y, xj.y, g[j]);
                g[j] = fmaf(xl.z, xj.z, g[j]);
                g[j] = fmaf(xl.w, xj.w, g[j]);
            }
        }
    };
    if constexpr (SUB)
        gram(&sm.ys[0][0], kSubMax + 4, syp);
    else
        gram(&sm.x[0][0], D + 4, D);
    if (lane >= c) {
#pragma unroll
        for (int j = 0; j < kCovMaxRows; ++j) g[j] = 0.0f;
    }
    wave_lds_fence();  // the keys' space is reused for the Lanczos vectors
    // start from zeros there: the batched projections read rows past the last
    // vector (with zero weights), which must not hold stale non-finite bits
    {
        float* vz = &sm.lz.v[0][0];
        constexpr int NV = (kLanczos + 1) * (kCovMaxRows + 4);
        for (int i = 4 * lane; i < NV; i += 256) *reinterpret_cast<float4*>(vz + i) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    wave_lds_fence();

    // ---- Lanczos with full reorthogonalisation (classical Gram-Schmidt, two
    // passes, batched: lane i forms the coefficient on v_i from its row of V, then
    // lane l subtracts sum_i h_i v_i[l] reading its column; no cross-lane sums)
    const int steps = min(kLanczos, c);
    // start: a fixed pseudo-random vector over the block's rows (the all-ones
    // vector is in G's null space: the rows are centred)
    float v = 0.0f;
    if (lane < c) {
        uint32_t hsh = (uint32_t)lane * 0x9E3779B1u + 0x7F4A7C15u;
        hsh ^= hsh >> 15;
        hsh *= 0x2C1B3C6Du;
        hsh ^= hsh >> 12;
        v = (float)(hsh & 0xFFFF) / 65536.0f + 0.5f;
    }
    v /= sqrtf(wave_sum(v * v));
    int m = 0;  // Lanczos vectors kept
    float gnorm = 0.0f;
    for (int k = 0; k < steps; ++k) {
        sm.lz.v[k][lane] = v;
        wave_lds_fence();
        float w = 0.0f;
#pragma unroll
        for (int j = 0; j < kCovMaxRows; j += 4) {
            const float4 vj = *reinterpret_cast<const float4*>(&sm.lz.v[k][j]);
            w = fmaf(g[j], vj.x, w);
            w = fmaf(g[j + 1], vj.y, w);
            w = fmaf(g[j + 2], vj.z, w);
            w = fmaf(g[j + 3], vj.w, w);
        }
        const float a = wave_sum(w * v);
        sm.alpha[k] = a;
        m = k + 1;
        w -= a * v;
        if (k > 0) w -= sm.beta[k - 1] * sm.lz.v[k - 1][lane];
        for (int pass = 0; pass < 2; ++pass) {
            sm.lz.w[lane] = w;
            wave_lds_fence();
            // lane i <= k: v_i . w (every load of the row issued before the products)
            float4 vi[kCovMaxRows / 4], wl[kCovMaxRows / 4];
#pragma unroll
            for (int u = 0; u < kCovMaxRows / 4; ++u) {
                vi[u] = *reinterpret_cast<const float4*>(&sm.lz.v[lane][4 * u]);
                wl[u] = *reinterpret_cast<const float4*>(&sm.lz.w[4 * u]);
            }
            float h0 = 0.0f, h1 = 0.0f;
#pragma unroll
            for (int u = 0; u < kCovMaxRows / 4; u += 2) {
                h0 = fmaf(vi[u].x, wl[u].x, h0);
                h0 = fmaf(vi[u].y, wl[u].y, h0);
                h0 = fmaf(vi[u].z, wl[u].z, h0);
                h0 = fmaf(vi[u].w, wl[u].w, h0);
                h1 = fmaf(vi[u + 1].x, wl[u + 1].x, h1);
                h1 = fmaf(vi[u + 1].y, wl[u + 1].y, h1);
                h1 = fmaf(vi[u + 1].z, wl[u + 1].z, h1);
                h1 = fmaf(vi[u + 1].w, wl[u + 1].w, h1);
            }
            sm.lz.h[lane] = lane <= k ? h0 + h1 : 0.0f;  // rows past v_k hold stale data
            wave_lds_fence();
            // w -= sum_{i <= k} h_i v_i, eight terms per round (h_i = 0 past k)
            for (int i0 = 0; i0 <= k; i0 += 8) {
                const float4 ha = *reinterpret_cast<const float4*>(&sm.lz.h[i0]);
                const float4 hb = *reinterpret_cast<const float4*>(&sm.lz.h[i0 + 4]);
                float vv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) vv[u] = sm.lz.v[i0 + u][lane];
                const float pa = (ha.x * vv[0] + ha.y * vv[1]) + (ha.z * vv[2] + ha.w * vv[3]);
                const float pb = (hb.x * vv[4] + hb.y * vv[5]) + (hb.z * vv[6] + hb.w * vv[7]);
                w -= pa + pb;
            }
            wave_lds_fence();  // w and h are rewritten by the next pass
        }
        const float b = sqrtf(wave_sum(w * w));
        gnorm = fmaxf(gnorm, fabsf(a) + b);
        if (k + 1 == steps || b <= 1e-6f * gnorm) break;  // Krylov space exhausted
        sm.beta[k] = b;
        v = w / b;
    }
    wave_lds_fence();

    // ---- Ritz values: the R largest eigenvalues of the m x m tridiagonal T, by
    // multisection on Sturm counts, all R at once: lane group r = lane / 16 brackets
    // eigenvalue r with 16 shifts per round (4 bits per round)
    auto below = [&](float x) {  // number of eigenvalues of T below x
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
    {
        const int r = lane >> 4, sub = lane & 15;
        const int idx = m - 1 - r;  // eigenvalue index in ascending order
        float lo = glo, hi = ghi;
        for (int round = 0; round < 8; ++round) {
            // lane (r, sub) tests lo + (sub + 1) (hi - lo) / 17
            const float step = (hi - lo) / 17.0f;
            const float x = lo + (float)(sub + 1) * step;
            const bool above = idx >= 0 && below(x) <= idx;  // the eigenvalue lies at or above x
            const uint64_t mk = __ballot(above);
            const int nab = __popcll((mk >> (16 * r)) & 0xffffull);  // shifts of group r below it
            const float nlo = lo + (float)nab * step;
            hi = lo + (float)(nab + 1) * step;
            lo = nlo;
        }
        if (sub == 0 && r < R) sm.theta[r] = idx >= 0 ? fmaxf(0.5f * (lo + hi), 0.0f) : 0.0f;
    }
    wave_lds_fence();

    // ---- eigenvectors of T by inverse iteration (lane i < R solves for theta_i);
    // the elimination carries its last pivot and right-hand side in registers
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
            float cprev = m > 1 ? sm.beta[0] / den : 0.0f;
            float dprev = y[0] / den;
            cp[0] = cprev;
            dp[0] = dprev;
            for (int k = 1; k < m; ++k) {
                const float bk1 = sm.beta[k - 1];
                den = sm.alpha[k] - th - bk1 * cprev;
                den = fabsf(den) < tiny ? (den < 0.0f ? -tiny : tiny) : den;
                const float inv = 1.0f / den;
                cprev = k + 1 < m ? sm.beta[k] * inv : 0.0f;
                dprev = (y[k] - bk1 * dprev) * inv;
                cp[k] = cprev;
                dp[k] = dprev;
            }
            float yk = dprev;
            y[m - 1] = yk;
            float nn = yk * yk;
            for (int k = m - 2; k >= 0; --k) {
                yk = dp[k] - cp[k] * yk;
                y[k] = yk;
                nn += yk * yk;
            }
            if (!(nn > 0.0f && nn < 3.0e38f)) {  // degenerate: fall back to a unit vector
                for (int k = 0; k < m; ++k) y[k] = k == 0 ? 1.0f : 0.0f;
                break;
            }
            const float inv = 1.0f / sqrtf(nn);
            for (int k = 0; k < m; ++k) y[k] *= inv;
        }
    }
    wave_lds_fence();

    // ---- Ritz vectors over the rows: z_i[l] = sum_k v_k[l] y_i[k]
#pragma unroll
    for (int i = 0; i < R; ++i) {
        float zz = 0.0f;
        if (i < m)
            for (int k = 0; k < m; ++k) zz = fmaf(sm.lz.v[k][lane], sm.y[i][k], zz);
        sm.z[i][lane] = lane < c ? zz : 0.0f;
    }
    wave_lds_fence();

    // ---- xi_i = X^T z_i / sqrt(c), the centred keys read again from memory (the
    // same fp32 values as in LDS before); sign: largest-magnitude coordinate positive.
    // SUB: xi_i = Y^T z_i / sqrt(c) from the subspace coordinates in LDS, columns
    // 2 lane and 2 lane + 1 of each lane.
    constexpr int XC = SUB ? kSubMax / 64 : CPL;  // coordinates per lane
    float xi[R][XC];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int e = 0; e < XC; ++e) xi[i][e] = 0.0f;
    if constexpr (SUB) {
        for (int l = 0; l < c; ++l) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const float zi = sm.z[i][l];
#pragma unroll
                for (int e = 0; e < XC; ++e) {
                    const int col = XC * lane + e;
                    xi[i][e] = fmaf(col < s_dim ? sm.ys[l][col] : 0.0f, zi, xi[i][e]);
                }
            }
        }
    }
    for (int l = 0; l < (SUB ? 0 : c); ++l) {
        float f[CPL];
        const char* row = kp + (size_t)l * RB + CPL * lane * EB;
        if constexpr (DT == DT_F32) {
            if constexpr (CPL == 2) {
                const float2 v2 = *reinterpret_cast<const float2*>(row);
                f[0] = v2.x;
                f[1] = v2.y;
            } else {
                f[0] = *reinterpret_cast<const float*>(row);
            }
        } else {
            if constexpr (CPL == 2) {
                const uint32_t u = *reinterpret_cast<const uint32_t*>(row);
                f[0] = __uint_as_float(u << 16);
                f[1] = __uint_as_float(u & 0xffff0000u);
            } else {
                f[0] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(row) << 16);
            }
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) f[e] -= meanf[e];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const float zi = sm.z[i][l];
#pragma unroll
            for (int e = 0; e < CPL; ++e) xi[i][e] = fmaf(f[e], zi, xi[i][e]);
        }
    }
    (void)syp;
    const float inv_sqrt_c = 1.0f / sqrtf((float)c);
#pragma unroll
    for (int i = 0; i < R; ++i) {
        float best = -1.0f;
        int bt = 0;
#pragma unroll
        for (int e = 0; e < XC; ++e) {
            xi[i][e] *= inv_sqrt_c;
            const float a = fabsf(xi[i][e]);
            if (a > best) {
                best = a;
                bt = XC * lane + e;
            }
        }
        // wave-wide (magnitude, -index) maximum: the first coordinate of largest magnitude
        uint32_t hkey = __float_as_uint(best), lkey = ~(uint32_t)bt;
        wave_key_max(hkey, lkey);
        const int at = (int)~lkey;
        float sgn_src = 0.0f;
#pragma unroll
        for (int e = 0; e < XC; ++e)
            if (XC * lane + e == at) sgn_src = xi[i][e];
        const float sgn = __shfl(sgn_src, at / XC) < 0.0f ? -1.0f : 1.0f;
        if constexpr (SUB && FP4) {
            // the bfloat16-rounded coordinates (zero past s), the scale from their largest
            // magnitude, one byte of two codes per lane (coordinates 2 lane, 2 lane + 1)
            float vb[XC];
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < XC; ++e) {
                const int col = XC * lane + e;
                vb[e] = col < s_dim ? __uint_as_float((uint32_t)bf16_from_f64((double)(xi[i][e] * sgn)) << 16) : 0.0f;
                amax = fmaxf(amax, fabsf(vb[e]));
            }
            amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));
            const float sc = amax / 6.0f;
            if (lane == 0) *reinterpret_cast<float*>(out + 2 * D + 4 * i) = sc;
            uint32_t code[XC];
#pragma unroll
            for (int e = 0; e < XC; ++e) code[e] = sc > 0.0f ? e2m1_code(vb[e] / sc) : 0u;
            static_assert(XC == 2, "two coordinates, one byte of codes per lane");
            if (2 * lane < spf)
                reinterpret_cast<uint8_t*>(out + 2 * D + 4 * R + i * (spf / 2))[lane] = (uint8_t)(code[0] | (code[1] << 4));
        } else if constexpr (SUB) {
#pragma unroll
            for (int e = 0; e < XC; ++e) {
                const int col = XC * lane + e;
                if (col < sps) {
                    const float val = col < s_dim ? xi[i][e] * sgn : 0.0f;
                    char* row = out + RB + (size_t)i * sps * EB;
                    if constexpr (DT == DT_F32)
                        reinterpret_cast<float*>(row)[col] = val;
                    else
                        reinterpret_cast<uint16_t*>(row)[col] = bf16_from_f64((double)val);
                }
            }
        } else if constexpr (FP4) {
            float vb[CPL];  // the bfloat16-rounded coordinates, widened exactly
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                vb[e] = __uint_as_float((uint32_t)bf16_from_f64((double)(xi[i][e] * sgn)) << 16);
                amax = fmaxf(amax, fabsf(vb[e]));
            }
            amax = __uint_as_float(wave_max_u32(__float_as_uint(amax)));  // non-negative: bits order as values
            const float sc = amax / 6.0f;
            if (lane == 0) *reinterpret_cast<float*>(out + 2 * D + 4 * i) = sc;
            uint32_t code[CPL];
#pragma unroll
            for (int e = 0; e < CPL; ++e) code[e] = sc > 0.0f ? e2m1_code(vb[e] / sc) : 0u;
            uint8_t* row = reinterpret_cast<uint8_t*>(out + 2 * D + 4 * R + i * (D / 2));
            if constexpr (CPL == 2) {
                row[lane] = (uint8_t)(code[0] | (code[1] << 4));
            } else {
                const uint32_t hi = (uint32_t)__shfl_xor((int)code[0], 1);
                if ((lane & 1) == 0) row[lane >> 1] = (uint8_t)(code[0] | (hi << 4));
            }
        } else {
#pragma unroll
            for (int e = 0; e < CPL; ++e) {
                const int t = CPL * lane + e;
                const float val = xi[i][e] * sgn;
                if constexpr (DT == DT_F32) {
                    reinterpret_cast<float*>(out + (size_t)(1 + i) * RB)[t] = val;
                } else {
                    reinterpret_cast<uint16_t*>(out + (size_t)(1 + i) * RB)[t] = bf16_from_f64((double)val);
                }
            }
        }
    }
}

template <int DT, int D, bool FP4, bool SUB = false>
hipError_t launch_cov_dtd(const Dims& s, const void* K, void* Kcov, hipStream_t st, const float* U = nullptr,
                          int s_dim = 0)
{
    const long long total = (long long)s.pairs() * s.nb;  // one workgroup (one wave) per block
    cov_kernel<DT, D, kCobsRank, FP4, SUB><<<dim3((unsigned)total), dim3(64), 0, st>>>(
        static_cast<const char*>(K), static_cast<char*>(Kcov), s.n, s.L, s.nb, U, s_dim, s.Hkv);
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
        if (s.d == 128) return launch_cov_dtd<DT_BF16, 128, false>(s, K, Kcov, st);
        if (s.d == 64) return launch_cov_dtd<DT_BF16, 64, false>(s, K, Kcov, st);
    } else {
        if (s.d == 128) return launch_cov_dtd<DT_F32, 128, false>(s, K, Kcov, st);
        if (s.d == 64) return launch_cov_dtd<DT_F32, 64, false>(s, K, Kcov, st);
    }
    return hipErrorInvalidValue;
}

bool cov_sub_ok(const Dims& s, int s_dim)
{
    return cov_build_ok(s) && s_dim >= 1 && s_dim <= s.d && s_dim <= kSubMax;
}

hipError_t launch_cov_sub(const Dims& s, int s_dim, const void* K, const float* U, void* Kcs, hipStream_t st)
{
    if (s.dtype == DT_BF16) {
        if (s.d == 128) return launch_cov_dtd<DT_BF16, 128, false, true>(s, K, Kcs, st, U, s_dim);
        if (s.d == 64) return launch_cov_dtd<DT_BF16, 64, false, true>(s, K, Kcs, st, U, s_dim);
    } else {
        if (s.d == 128) return launch_cov_dtd<DT_F32, 128, false, true>(s, K, Kcs, st, U, s_dim);
        if (s.d == 64) return launch_cov_dtd<DT_F32, 64, false, true>(s, K, Kcs, st, U, s_dim);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cov_sub4(const Dims& s, int s_dim, const void* K, const float* U, void* Kcs4, hipStream_t st)
{
    if (s.dtype != DT_BF16) return hipErrorInvalidValue;
    if (s.d == 128) return launch_cov_dtd<DT_BF16, 128, true, true>(s, K, Kcs4, st, U, s_dim);
    if (s.d == 64) return launch_cov_dtd<DT_BF16, 64, true, true>(s, K, Kcs4, st, U, s_dim);
    return hipErrorInvalidValue;
}

hipError_t launch_cov4(const Dims& s, const void* K, void* Kcov4, hipStream_t st)
{
    if (s.dtype != DT_BF16) return hipErrorInvalidValue;
    if (s.d == 128) return launch_cov_dtd<DT_BF16, 128, true>(s, K, Kcov4, st);
    if (s.d == 64) return launch_cov_dtd<DT_BF16, 64, true>(s, K, Kcov4, st);
    return hipErrorInvalidValue;
}

}  // namespace csa

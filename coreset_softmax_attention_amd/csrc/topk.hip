// topk.hip -- the k largest block scores of each row, ties to the lower index.
//
// One block set is chosen per KV head and shared by its query heads ("COBS:
// Cumulant Order Block Sparse Attention", Eqs. (4)-(5)).  One workgroup per
// row:
//   1. scores are mapped to order-preserving unsigned keys (+0 and -0 map to
//      the same key, so they tie);
//   2. a most-significant-digit radix select (4 passes of 8 bits, histograms
//      in LDS) finds the k-th largest key T and how many keys equal to T are
//      needed after all keys greater than T;
//   3. a scan in index order writes every index with key > T and the lowest
//      indices with key == T, so the output is ascending by index.
// Integer histograms and scans only: the result does not depend on timing.
//
// Small k (k <= 8, nb <= 512) uses a workgroup of eight waves per row: each
// wave's largest score, the k-th largest of those as a lower bound, and a rank
// among the few scores that reach it.  Other small k (k <= 32, nb <= 2048) use
// one wavefront per row: every lane
// holds up to 32 packed keys (order-preserving score bits, then the inverted
// index, so a larger key is a higher score or, on a tie, a lower index); k
// rounds of a wave-wide maximum pick the winners, and a prefix count over the
// lanes writes them in index order.
#include "device.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace csa {
namespace {

constexpr int kThreads = 256;

// Exclusive prefix sum over the workgroup (256 threads); also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* sm /* >= 4 ints */)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) sm[wave] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        if (w < wave) before += sm[w];
        all += sm[w];
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

__global__ void __launch_bounds__(kThreads) topk_kernel(const float* scores, int32_t* sel, int nb, int k)
{
    __shared__ int hist[256];
    __shared__ int scan_sm[4];
    __shared__ uint32_t sh_digit;
    __shared__ int sh_rem;

    const int row = blockIdx.x, tid = threadIdx.x;
    const int kk = min(k, nb);
    const float* s = scores + (size_t)row * nb;
    int32_t* out = sel + (size_t)row * kk;
    if (kk == 0) return;
    if (kk == nb) {
        for (int i = tid; i < nb; i += kThreads) out[i] = i;
        return;
    }

    uint32_t prefix = 0, mask = 0;
    int remaining = kk;
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < nb; i += kThreads) {
            const uint32_t u = order_key(s[i]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
        }
        __syncthreads();
        // thread d: keys of the current prefix whose digit is above d (reverse scan)
        const int d = 255 - tid;
        const int cnt = hist[d];
        int tot;
        const int above = block_exclusive_scan(cnt, &tot, scan_sm);
        if (above < remaining && above + cnt >= remaining) {
            sh_digit = (uint32_t)d;
            sh_rem = remaining - above;
        }
        __syncthreads();
        prefix |= sh_digit << shift;
        mask |= 0xffu << shift;
        remaining = sh_rem;
        __syncthreads();
    }
    const uint32_t T = prefix;
    const int need_eq = remaining;  // keys equal to T still to take, lowest index first

    const int per = (nb + kThreads - 1) / kThreads;
    const int i0 = min(nb, tid * per), i1 = min(nb, i0 + per);
    int eq = 0;
    for (int i = i0; i < i1; ++i) eq += order_key(s[i]) == T;
    int tot;
    int eq_before = block_exclusive_scan(eq, &tot, scan_sm);
    int take = 0;
    {
        int e = eq_before;
        for (int i = i0; i < i1; ++i) {
            const uint32_t u = order_key(s[i]);
            if (u > T) {
                ++take;
            } else if (u == T) {
                if (e < need_eq) ++take;
                ++e;
            }
        }
    }
    int pos = block_exclusive_scan(take, &tot, scan_sm);
    {
        int e = eq_before;
        for (int i = i0; i < i1; ++i) {
            const uint32_t u = order_key(s[i]);
            bool keep = false;
            if (u > T) {
                keep = true;
            } else if (u == T) {
                keep = e < need_eq;
                ++e;
            }
            if (keep) out[pos++] = i;
        }
    }
}


constexpr int kWaveTopkMaxK = 32;
constexpr int kWaveTopkMaxPer = 32;  // keys per lane

// One wave per row (k <= 32, nb <= 64 * PER).
template <int PER>
__global__ void __launch_bounds__(256) topk_wave_kernel(const float* scores, int32_t* sel, int rows, int nb, int k)
{
    __shared__ uint32_t cand[4][128];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave;
    if (row >= rows) return;  // whole wave; no workgroup barrier below
    const float* s = scores + (size_t)row * nb;
    int32_t* out = sel + (size_t)row * k;
    wave_topk<PER>([&](int i) { return s[i]; }, nb, k, lane, cand[wave], [&](int r, int idx) { out[r] = idx; });
}

constexpr int kBlockTopkWaves = 8;
constexpr int kBlockTopkMaxK = kBlockTopkWaves;  // the bound from the waves' maxima needs k <= waves
constexpr int kBlockTopkMaxBlocks = kBlockTopkWaves * 64;

// One workgroup of eight waves per row (k <= 8, nb <= 512): the bound from the
// waves' maxima, one wave over all scores when it does not apply.
__global__ void __launch_bounds__(kBlockTopkWaves * 64) topk_block_kernel(const float* scores, int32_t* sel, int nb,
                                                                            int k)
{
    constexpr int NW = kBlockTopkWaves;
    __shared__ uint32_t cand[128];
    __shared__ uint32_t topk_sm[2 * NW + 128];
    const int row = blockIdx.x, lane = threadIdx.x & 63;
    const float* s = scores + (size_t)row * nb;
    int32_t* out = sel + (size_t)row * k;
    uint32_t key[1] = {(int)threadIdx.x < nb ? order_key(s[threadIdx.x]) : 0u};
    auto emit = [&](int r, int idx) { out[r] = idx; };
    auto one_wave_topk = [&]() { wave_topk<kBlockTopkMaxBlocks / 64>([&](int i) { return s[i]; }, nb, k, lane, cand, emit); };
    block_topk<NW, 1>(key, nb, k, topk_sm, one_wave_topk, emit);
}

}  // namespace

hipError_t launch_topk(int rows, int nb, int k, const float* scores, int32_t* sel, hipStream_t st)
{
    if (k < nb && k <= kBlockTopkMaxK && nb <= kBlockTopkMaxBlocks) {
        topk_block_kernel<<<dim3((unsigned)rows), dim3(kBlockTopkWaves * 64), 0, st>>>(scores, sel, nb, k);
        return hipGetLastError();
    }
    const int per = (nb + 63) / 64;
    if (k < nb && k <= kWaveTopkMaxK && per <= kWaveTopkMaxPer) {
        const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
        if (per <= 1) topk_wave_kernel<1><<<grid, block, 0, st>>>(scores, sel, rows, nb, k);
        else if (per <= 2) topk_wave_kernel<2><<<grid, block, 0, st>>>(scores, sel, rows, nb, k);
        else if (per <= 4) topk_wave_kernel<4><<<grid, block, 0, st>>>(scores, sel, rows, nb, k);
        else if (per <= 8) topk_wave_kernel<8><<<grid, block, 0, st>>>(scores, sel, rows, nb, k);
        else if (per <= 16) topk_wave_kernel<16><<<grid, block, 0, st>>>(scores, sel, rows, nb, k);
        else topk_wave_kernel<32><<<grid, block, 0, st>>>(scores, sel, rows, nb, k);
        return hipGetLastError();
    }
    topk_kernel<<<dim3((unsigned)rows), dim3(kThreads), 0, st>>>(scores, sel, nb, k);
    return hipGetLastError();
}

}  // namespace csa

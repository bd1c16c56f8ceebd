// attn_engine.hpp -- the per-wave online-softmax engine of the bfloat16
// attention kernels (sparse_decode_attn, dense_decode_attn and the fused
// decode step).
//
// A wave processes tiles of 32 virtual rows, two in flight at a time.  For each
// tile:
//   1. lanes 0..31 resolve the tile's rows into one of two per-wave LDS tables
//      (row index in its source array, log2-weight; -inf for a row that does not
//      count);
//   2. the tile's rows are loaded with non-temporal buffer loads, whole rows per
//      lane group (16-byte chunks, coalesced: RB / 16 lanes per row); the key
//      rows then pass through a per-wave LDS slot into the layout of the A
//      operand of v_mfma_f32_16x16x32_bf16 (lane (n16, g16): row n16 of a
//      16-row block, 16-byte chunks 4 s + g16);
//   3. logits for up to 8 query heads come from two 16x16x32 MFMA chains (rows
//      x heads, heads padded to 16 columns), or from LDS when the caller has
//      them already; the online-softmax update runs once per (row, head) on the
//      MFMA output lanes and the probabilities go through LDS to the value lanes;
//   4. the value lanes accumulate P V in fp32.
// All lane groups of a wave share one running maximum per head, so their
// partial sums add directly; waves are merged through LDS at the end.
#pragma once

#include "device.hpp"

namespace csa {

constexpr int kTileRows = 32;

template <int D, int HG, int NW>
struct MfmaEngine {
    static constexpr int RB = D * 2;            // row bytes
    static constexpr int KS = D / 32;           // MFMA k-steps per row
    static constexpr int TR = kTileRows;
    static constexpr int LPV = RB / 16;         // lanes per value row
    static constexpr int RPV = 64 / LPV;        // value rows per wave-wide load
    static constexpr int NVI = TR / RPV;        // value loads per lane per tile
    static constexpr int NI = TR / RPV;         // key loads per lane per tile (rows RPV j + gv)
    static constexpr int HP = HG <= 4 ? 4 : 8;  // padded heads per probability row
    static_assert(KS * 32 == D && HG <= 8 && (LPV == 8 || LPV == 16), "unsupported geometry");
    static_assert(NI == 2 * KS && RPV * NI / 2 == 16, "a half tile of key loads covers one 16-row MFMA block");
    // Key rows go through LDS (coalesced non-temporal loads, then the layout
    // change) up to six heads; with seven or eight the value accumulators leave
    // no room for it, and the keys are loaded in the operand layout directly
    // (kr[KS rb + s] = operand s of block rb).
    static constexpr bool kLdsKeys = HG <= 6;

    static constexpr int NTAB = 4;  // row tables per wave (tiles in flight or pending)

    struct Smem {
        uint32_t tab_row[NTAB][NW][TR];
        float tab_lw[NTAB][NW][TR] __attribute__((aligned(16)));
        float p[NW][TR][HP] __attribute__((aligned(16)));
        float alpha[NW][HP] __attribute__((aligned(16)));
        float m[NW][HG];
        float l[NW][HG];
        float acc[NW][HG][D];
        uint4 kt[kLdsKeys ? NW : 1][16 * (LPV + 1)];  // per-wave staging of 16 key rows (layout change)
    };

    // One tile's rows in registers, as loaded: kr[j] and vr[j] hold 16-byte
    // chunk cv of key and value row RPV j + gv (four or eight consecutive rows
    // per instruction; one row offset serves both).
    struct Tile {
        uint4 kr[NI];
        uint4 vr[NVI];
    };

    Smem& sm;
    const int lane, wave, n16, g16, gv, cv;
    bf16x8_t bq[KS];
    float m_run, l_part;  // MFMA lanes: head n16
    float acc[HG][8];     // value lanes: chunk cv of the rows RPV j + gv

    __device__ __forceinline__ MfmaEngine(Smem& s, const char* q_first_head, int nh)
        : sm(s),
          lane(threadIdx.x & 63),
          wave(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)),
          n16(threadIdx.x & 15),
          g16((threadIdx.x & 63) >> 4),
          gv((threadIdx.x & 63) / LPV),
          cv((threadIdx.x & 63) % LPV),
          m_run(kNegInf),
          l_part(0.0f)
    {
        load_q_operand<D>(q_first_head, nh, lane, bq);
#pragma unroll
        for (int g = 0; g < HG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
    }

    // Row table entry (lanes 0..31 of the wave) of table `tb` (0 or 1).
    __device__ __forceinline__ void set_row(int tb, int i, uint32_t row, float lw)
    {
        sm.tab_row[tb][wave][i] = row;
        sm.tab_lw[tb][wave][i] = lw;
    }

    // Issue the loads of a tile whose row table `tb` is written.  with_keys: also
    // the key rows (otherwise the caller supplies the logits).
    __device__ __forceinline__ void issue(Tile& t, int tb, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                          bool with_keys)
    {
        wave_lds_fence();
        if constexpr (kLdsKeys) {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const uint32_t off = sm.tab_row[tb][wave][RPV * j + gv] * RB + cv * 16;
                if (with_keys) t.kr[j] = buffer_ld16_nt(kr, off);
                t.vr[j] = buffer_ld16_nt(vr, off);
            }
        } else {
            if (with_keys) operand_keys(t.kr, tb, kr);
#pragma unroll
            for (int j = 0; j < NVI; ++j) t.vr[j] = buffer_ld16_nt(vr, sm.tab_row[tb][wave][RPV * j + gv] * RB + cv * 16);
        }
    }

    // Key rows in the operand layout: lane (n16, g16) loads chunk 4 s + g16 of
    // row 16 rb + n16 into kr[KS rb + s] (half a cache line per row per load).
    __device__ __forceinline__ void operand_keys(uint4 (&kr)[NI], int tb, __amdgpu_buffer_rsrc_t r)
    {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const uint32_t off = sm.tab_row[tb][wave][rb * 16 + n16] * RB + g16 * 16;
#pragma unroll
            for (int s = 0; s < KS; ++s) kr[KS * rb + s] = buffer_ld16(r, off + s * 64);
        }
    }

    // Issue only the key rows of a tile whose row table `tb` is written (its
    // value rows follow with issue_values).
    __device__ __forceinline__ void issue_keys(Tile& t, int tb, __amdgpu_buffer_rsrc_t kr)
    {
        wave_lds_fence();
        if constexpr (kLdsKeys) {
#pragma unroll
            for (int j = 0; j < NI; ++j) t.kr[j] = buffer_ld16_nt(kr, sm.tab_row[tb][wave][RPV * j + gv] * RB + cv * 16);
        } else {
            operand_keys(t.kr, tb, kr);
        }
    }

    // Key rows as loaded (kr[j]: chunk cv of row RPV j + gv) -> A operand of the
    // 16-row MFMA block rb (a[s]: chunk 4 s + g16 of row 16 rb + n16), through
    // the wave's LDS slot.  Slot rows are padded to LPV + 1 chunks, which puts the
    // 16 rows' starts on 16 different groups of four banks: the lanes of a write
    // (whole rows) and of a read (one chunk of 16 rows) hit different banks, and
    // every access is one base address plus an immediate offset.
    __device__ __forceinline__ void key_block(const uint4 (&kr)[NI], int rb, uint4 (&a)[KS])
    {
        if constexpr (!kLdsKeys) {
#pragma unroll
            for (int s = 0; s < KS; ++s) a[s] = kr[KS * rb + s];
            return;
        }
        uint4* slot = sm.kt[wave];
#pragma unroll
        for (int j = 0; j < NI / 2; ++j) slot[(RPV * j + gv) * (LPV + 1) + cv] = kr[rb * (NI / 2) + j];
        wave_lds_fence();
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = slot[n16 * (LPV + 1) + 4 * s + g16];
        wave_lds_fence();  // the slot is rewritten next
    }

    // q K^T of the tile's two 16-row blocks: c[rb][i] is head n16 of row 16 rb + 4 g16 + i.
    __device__ __forceinline__ void qk_tile(const uint4 (&kr)[NI], f32x4_t (&c)[2])
    {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            uint4 a[KS];
            key_block(kr, rb, a);
            c[rb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                c[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[s]), bq[s], c[rb], 0, 0, 0);
        }
    }

    // Issue only the value rows of a tile (its logits come from the caller).
    __device__ __forceinline__ void issue_values(uint4 (&vr)[NVI], int tb, __amdgpu_buffer_rsrc_t rsrc)
    {
        wave_lds_fence();
#pragma unroll
        for (int u = 0; u < NVI; ++u) vr[u] = buffer_ld16_nt(rsrc, sm.tab_row[tb][wave][RPV * u + gv] * RB + cv * 16);
    }

    // Logits (log2 units) of the tile from its key rows: lane (n16, g16) gets
    // head n16 of rows 16 rb + 4 g16 + i as x[4 rb + i].
    __device__ __forceinline__ void logits_mfma(const Tile& t, int tb, float scale_log2, float (&x)[8])
    {
        f32x4_t c[2];
        qk_tile(t.kr, c);
        const f32x4_t c0 = c[0], c1 = c[1];
        const float4 lw0 = *reinterpret_cast<const float4*>(&sm.tab_lw[tb][wave][4 * g16]);
        const float4 lw1 = *reinterpret_cast<const float4*>(&sm.tab_lw[tb][wave][16 + 4 * g16]);
        const float lws[8] = {lw0.x, lw0.y, lw0.z, lw0.w, lw1.x, lw1.y, lw1.z, lw1.w};
        const float cs[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = lws[i] == kNegInf ? kNegInf : fmaf(cs[i], scale_log2, lws[i]);
    }

    // Logits (log2 units) of the tile from natural-log logits in LDS: head n16's
    // values for the tile's 32 rows start at `row_logits` (16-byte aligned); a
    // table log-weight of -inf masks the row, any other value is ignored.
    __device__ __forceinline__ void logits_lds(int tb, const float* row_logits, float (&x)[8])
    {
        const float4 lw0 = *reinterpret_cast<const float4*>(&sm.tab_lw[tb][wave][4 * g16]);
        const float4 lw1 = *reinterpret_cast<const float4*>(&sm.tab_lw[tb][wave][16 + 4 * g16]);
        const float4 v0 = *reinterpret_cast<const float4*>(row_logits + 4 * g16);
        const float4 v1 = *reinterpret_cast<const float4*>(row_logits + 16 + 4 * g16);
        const float lws[8] = {lw0.x, lw0.y, lw0.z, lw0.w, lw1.x, lw1.y, lw1.z, lw1.w};
        const float vs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = lws[i] == kNegInf ? kNegInf : vs[i] * kLog2e;
    }

    // Online-softmax update with the tile's logits; probabilities to LDS.
    __device__ __forceinline__ void softmax(float (&x)[8])
    {
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
        mx = max_xor32(max_xor16(mx));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = rescale(m_run, m_new);
        m_run = m_new;
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = x[i] == kNegInf ? 0.0f : exp2_(x[i] - m_new);
            l_part += x[i];
        }
        if (n16 < HG) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sm.p[wave][4 * g16 + i][n16] = x[i];
                sm.p[wave][16 + 4 * g16 + i][n16] = x[4 + i];
            }
            if (g16 == 0) sm.alpha[wave][n16] = alpha;
        }
        wave_lds_fence();
    }

    // P V of the tile on the value lanes.
    __device__ __forceinline__ void accumulate(const Tile& t) { accumulate_values(t.vr); }

    __device__ __forceinline__ void accumulate_values(const uint4 (&vr)[NVI])
    {
        float al[HP];
        *reinterpret_cast<float4*>(&al[0]) = *reinterpret_cast<const float4*>(&sm.alpha[wave][0]);
        if constexpr (HP == 8) *reinterpret_cast<float4*>(&al[4]) = *reinterpret_cast<const float4*>(&sm.alpha[wave][4]);
#pragma unroll
        for (int g = 0; g < HG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] *= al[g];
#pragma unroll
        for (int u = 0; u < NVI; ++u) {
            float pr[HP];
            *reinterpret_cast<float4*>(&pr[0]) = *reinterpret_cast<const float4*>(&sm.p[wave][RPV * u + gv][0]);
            if constexpr (HP == 8)
                *reinterpret_cast<float4*>(&pr[4]) = *reinterpret_cast<const float4*>(&sm.p[wave][RPV * u + gv][4]);
            float vf[8];
            unpack<DT_BF16>(vr[u], vf);
#pragma unroll
            for (int g = 0; g < HG; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pr[g], vf[e], acc[g][e]);
        }
        wave_lds_fence();  // p / alpha are rewritten by the next tile
    }

    // Merge the waves (the whole workgroup must call this).  Writes, for each
    // active head g < nh and element e, either the normalised output and the
    // lse (part == nullptr) or the partial state (max, sum, unnormalised output)
    // at part + g * (D + 2).
    __device__ __forceinline__ void finish(int nh, float* out, float* lse, float* part)
    {
        l_part = add_xor32(add_xor16(l_part));
        // sum the lane groups holding the same value columns (lanes l ^ LPV, ...)
#pragma unroll
        for (int g = 0; g < HG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float a = acc[g][e];
                if constexpr (LPV == 8) a += dpp<DPP_ROW_ROR8>(a);
                a = add_xor32(add_xor16(a));
                acc[g][e] = a;
            }
        if (gv == 0) {
#pragma unroll
            for (int g = 0; g < HG; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) sm.acc[wave][g][cv * 8 + e] = acc[g][e];
        }
        if (lane < HG) {
            sm.m[wave][lane] = m_run;
            sm.l[wave][lane] = l_part;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < HG * D; idx += NW * 64) {
            const int g = idx / D, e = idx - g * D;
            if (g >= nh) continue;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][g]);
            float Ls = 0.0f, A = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float a = rescale(sm.m[w][g], M);
                Ls += sm.l[w][g] * a;
                A += sm.acc[w][g][e] * a;
            }
            if (part == nullptr) {
                out[(size_t)g * D + e] = A / Ls;
                if (e == 0 && lse) lse[g] = (M + log2f(Ls)) * kLn2;
            } else {
                float* st = part + (size_t)g * (D + 2);
                if (e == 0) {
                    st[0] = M;
                    st[1] = Ls;
                }
                st[2 + e] = A;
            }
        }
    }
};

}  // namespace csa

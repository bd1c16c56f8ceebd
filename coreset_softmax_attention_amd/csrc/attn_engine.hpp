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
//      MFMA output lanes, which keep the probabilities;
//   4. P V on the matrix cores: the probabilities, split into two bfloat16
//      terms (hi + lo equals the fp32 value to about 2^-17), are the A operand
//      as they lie in the lanes; the value rows go through the wave's LDS slot
//      and come back transposed (ds_read_b64_tr_b16) as the B operand; the
//      output of all heads x d columns accumulates in D / 16 fp32 MFMA tiles.
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
    static_assert(KS * 32 == D && HG <= 8 && (LPV == 8 || LPV == 16), "unsupported geometry");
    static_assert(NI == 2 * KS && RPV * NI / 2 == 16, "a half tile of key loads covers one 16-row MFMA block");
    // Key rows go through LDS (coalesced non-temporal loads, then the layout
    // change).  The other form, keys loaded in the operand layout directly
    // (kr[KS rb + s] = operand s of block rb), stays for comparison: with P V on
    // the matrix cores every head count has the registers for the LDS route,
    // which took the 64-head step from 23.6 to 23.0 us (the 7-head weighted-
    // coreset step, latency-bound, from 30.4 to 30.8 us).
    static constexpr bool kLdsKeys = true;

    static constexpr int NTAB = 4;  // row tables per wave (tiles in flight or pending)

    // Per-wave LDS slot: 16 key rows padded to LPV + 1 chunks (layout change of
    // the keys), or the tile's 32 value rows padded by 32 bytes (the transposed
    // reads of a 16-lane group then cover four rows on disjoint banks).
    static constexpr int VRS = RB + 32;  // value row stride in the slot (bytes)
    static constexpr int SLOT = (TR * VRS > 16 * (LPV + 1) * 16 ? TR * VRS : 16 * (LPV + 1) * 16);
    static_assert(SLOT % 16 == 0 && VRS % 16 == 0, "16-byte aligned slot rows");
    static_assert(SLOT >= HG * D * 4, "a wave's output fits in its own slot");

    struct Smem {
        uint32_t tab_row[NTAB][NW][TR];
        float tab_lw[NTAB][NW][TR] __attribute__((aligned(16)));
        float alpha[NW][16] __attribute__((aligned(16)));
        float m[NW][HG];
        float l[NW][HG];
        union {
            uint4 slot[NW][SLOT / 16];  // while tiles stream; then the wave's output [HG][D] at its start
        } u;
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
    float m_run, l_part;     // MFMA lanes: head n16
    bf16x8_t pa_hi, pa_lo;   // the tile's probabilities, head n16, rows of k-slots 8 g16 .. 8 g16 + 7
    f32x4_t oacc[D / 16];    // output: heads 4 g16 + i, column 16 c + n16

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
        for (int c = 0; c < D / 16; ++c) oacc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
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
        uint4* slot = sm.u.slot[wave];
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
        logits_given(tb, *reinterpret_cast<const float4*>(row_logits + 4 * g16),
                     *reinterpret_cast<const float4*>(row_logits + 16 + 4 * g16), x);
    }

    // The same from the lane's own natural-log logits: v0 rows 4 g16 + i, v1 rows
    // 16 + 4 g16 + i of head n16.
    __device__ __forceinline__ void logits_given(int tb, float4 v0, float4 v1, float (&x)[8])
    {
        const float4 lw0 = *reinterpret_cast<const float4*>(&sm.tab_lw[tb][wave][4 * g16]);
        const float4 lw1 = *reinterpret_cast<const float4*>(&sm.tab_lw[tb][wave][16 + 4 * g16]);
        const float lws[8] = {lw0.x, lw0.y, lw0.z, lw0.w, lw1.x, lw1.y, lw1.z, lw1.w};
        const float vs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = lws[i] == kNegInf ? kNegInf : vs[i] * kLog2e;
    }

    // Online-softmax update with the tile's logits.  The probabilities stay in
    // the lanes as the A operand of P V: lane (n16, g16) holds head n16 at rows
    // 4 g16 + i and 16 + 4 g16 + i, which become its k-slots 0..3 and 4..7 (the
    // value rows are read in the same order).  The rescale factor of each head
    // goes to LDS for the output lanes.
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
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = x[i] == kNegInf ? 0.0f : exp2_(x[i] - m_new);
            l_part += x[i];
            // x = hi + lo: hi its leading 8 significant bits, lo the rest rounded to bfloat16
            const uint32_t hb = __float_as_uint(x[i]) >> 16;
            const float r = x[i] - __uint_as_float(hb << 16);
            const uint32_t ru = __float_as_uint(r);
            const uint32_t lb = (ru + 0x7fffu + ((ru >> 16) & 1u)) >> 16;
            if (i & 1) {
                hw[i >> 1] |= hb << 16;
                lw[i >> 1] |= lb << 16;
            } else {
                hw[i >> 1] = hb;
                lw[i >> 1] = lb;
            }
        }
        pa_hi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        pa_lo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        if (g16 == 0) sm.alpha[wave][n16] = alpha;
        wave_lds_fence();
    }

    // P V of the tile on the value lanes.
    __device__ __forceinline__ void accumulate(const Tile& t) { accumulate_values(t.vr); }

    __device__ __forceinline__ void accumulate_values(const uint4 (&vr)[NVI])
    {
        // rescale: lane (n16, g16) holds heads 4 g16 + i
        const float4 al = *reinterpret_cast<const float4*>(&sm.alpha[wave][4 * g16]);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            oacc[c][0] *= al.x;
            oacc[c][1] *= al.y;
            oacc[c][2] *= al.z;
            oacc[c][3] *= al.w;
        }
        // the value rows into the slot, as loaded (row RPV u + gv, chunk cv)
        char* slot = reinterpret_cast<char*>(sm.u.slot[wave]);
#pragma unroll
        for (int u = 0; u < NVI; ++u) *reinterpret_cast<uint4*>(slot + (RPV * u + gv) * VRS + cv * 16) = vr[u];
        wave_lds_fence();
        // B operand of column block c: lane (t, g16), t = lane % 16, k-slots 0..3 are
        // rows 4 g16 + 0..3 and 4..7 rows 16 + 4 g16 + 0..3, column 16 c + t.  A
        // transposed read over a 16-lane group gives lane 4 a + b element b of the
        // chunks addressed by lanes 4 j + a (j = 0..3): lane 4 j + a addresses row
        // j of the four, columns 16 c + 4 a .. + 3.
        const int t = lane & 15;
        const char* b0 = slot + (4 * g16 + (t >> 2)) * VRS + (t & 3) * 8;
        const char* b1 = b0 + 16 * VRS;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            typedef short v4i16_t __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) v4i16_t* lds_v4i16_ptr;
            const v4i16_t lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(b0 + c * 32));
            const v4i16_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_ptr)(b1 + c * 32));
            const uint2 l2 = __builtin_bit_cast(uint2, lo4), h2 = __builtin_bit_cast(uint2, hi4);
            const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
            oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi, bv, oacc[c], 0, 0, 0);
            oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo, bv, oacc[c], 0, 0, 0);
        }
        wave_lds_fence();  // the slot and alpha are rewritten by the next tile
    }

    // Merge the waves (the whole workgroup must call this).  Writes, for each
    // active head g < nh and element e, either the normalised output and the
    // lse (part == nullptr) or the partial state (max, sum, unnormalised output)
    // at part + g * (D + 2).
    __device__ __forceinline__ void finish(int nh, float* out, float* lse, float* part)
    {
        l_part = add_xor32(add_xor16(l_part));
        // the wave's output takes the place of its own slot (no other wave reads it)
        float* mine = reinterpret_cast<float*>(sm.u.slot[wave]);
        // output lanes: heads 4 g16 + i, column 16 c + n16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * g16 + i;
            if (g < HG) {
#pragma unroll
                for (int c = 0; c < D / 16; ++c) mine[g * D + 16 * c + n16] = oacc[c][i];
            }
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
                A += reinterpret_cast<const float*>(sm.u.slot[w])[g * D + e] * a;
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

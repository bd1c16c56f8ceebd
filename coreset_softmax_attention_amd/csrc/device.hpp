// device.hpp -- device helpers shared by the gfx950 kernels of libcsa.
//
// Row layout used by every kernel: a row of d elements is read as 16-byte
// chunks, one chunk per lane, so a row occupies LPR = d * elem_bytes / 16
// consecutive lanes of a 64-wide wavefront and one wave-wide load instruction
// covers 64 / LPR whole rows (fully coalesced).  Dot products are reduced over
// the LPR lanes of a row with DPP lane permutes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

enum : int { DT_F32 = 0, DT_BF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

template <int DT>
struct Elem;
template <>
struct Elem<DT_F32> {
    static constexpr int bytes = 4;
    static constexpr int per16 = 4;  // elements per 16-byte chunk
};
template <>
struct Elem<DT_BF16> {
    static constexpr int bytes = 2;
    static constexpr int per16 = 8;
};

// Geometry of a row of D elements of type DT in a 64-lane wavefront.
template <int DT, int D>
struct RowGeom {
    static constexpr int row_bytes = D * Elem<DT>::bytes;
    static constexpr int lpr = row_bytes / 16;  // lanes per row
    static constexpr int rpw = 64 / lpr;        // rows per wave-wide load
    static constexpr int epl = Elem<DT>::per16; // elements per lane
    static_assert(lpr >= 8 && lpr <= 32 && (lpr & (lpr - 1)) == 0, "unsupported row width");
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Nontemporal 16-byte load: data read once, do not keep it in the caches.
__device__ __forceinline__ uint4 ld16_nt(const void* p)
{
    const uint4* q = reinterpret_cast<const uint4*>(p);
    uint4 r;
    r.x = __builtin_nontemporal_load(&reinterpret_cast<const uint32_t*>(q)[0]);
    r.y = __builtin_nontemporal_load(&reinterpret_cast<const uint32_t*>(q)[1]);
    r.z = __builtin_nontemporal_load(&reinterpret_cast<const uint32_t*>(q)[2]);
    r.w = __builtin_nontemporal_load(&reinterpret_cast<const uint32_t*>(q)[3]);
    return r;
}

// 16 bytes -> per16 floats.  A bfloat16 is the upper half of a binary32.
template <int DT>
__device__ __forceinline__ void unpack(const uint4& r, float* f)
{
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
    if constexpr (DT == DT_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
}

// DPP lane permutes (gfx9 encodings).
enum : int {
    DPP_QUAD_1032 = 0xB1,     // quad_perm [1,0,3,2]
    DPP_QUAD_2301 = 0x4E,     // quad_perm [2,3,0,1]
    DPP_ROW_MIRROR = 0x140,   // lane i <-> 15 - i within 16 lanes
    DPP_ROW_HMIRROR = 0x141,  // lane i <-> 7 - i within 8 lanes
    DPP_ROW_ROR8 = 0x128,     // lane i <- lane (i + 8) mod 16 within 16 lanes, i.e. i ^ 8
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __builtin_amdgcn_update_dpp(0.0f, v, CTRL, 0xf, 0xf, false);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

// Values of lanes l and l ^ 16 (Swap16) or l and l ^ 32 (Swap32), from the
// gfx950 lane-swap instructions: v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second, v_permlane32_swap
// the upper half of the first with the lower half of the second.  Given the
// same register twice, every lane ends up holding its own value and its
// partner's (in .a and .b, in an order that depends on the lane's row, which
// does not matter for the commutative combines below).  These are ALU
// instructions, unlike ds_bpermute, which goes through the LDS pipeline.
struct LanePair {
    uint32_t a, b;
};
__device__ __forceinline__ LanePair swap16(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return {r[0], r[1]};
}
__device__ __forceinline__ LanePair swap32(uint32_t v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return {r[0], r[1]};
}
__device__ __forceinline__ float add_xor16(float v)
{
    const LanePair r = swap16(__float_as_uint(v));
    return __uint_as_float(r.a) + __uint_as_float(r.b);
}
__device__ __forceinline__ float add_xor32(float v)
{
    const LanePair r = swap32(__float_as_uint(v));
    return __uint_as_float(r.a) + __uint_as_float(r.b);
}
__device__ __forceinline__ float max_xor16(float v)
{
    const LanePair r = swap16(__float_as_uint(v));
    return fmaxf(__uint_as_float(r.a), __uint_as_float(r.b));
}
__device__ __forceinline__ float max_xor32(float v)
{
    const LanePair r = swap32(__float_as_uint(v));
    return fmaxf(__uint_as_float(r.a), __uint_as_float(r.b));
}

// Sum over aligned groups of W lanes (W = 8, 16, 32 or 64); every lane of the
// group receives the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    v += dpp<DPP_QUAD_1032>(v);
    v += dpp<DPP_QUAD_2301>(v);
    v += dpp<DPP_ROW_HMIRROR>(v);
    if constexpr (W >= 16) v += dpp<DPP_ROW_MIRROR>(v);
    if constexpr (W >= 32) v = add_xor16(v);
    if constexpr (W >= 64) v = add_xor32(v);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v)
{
    v = fmaxf(v, dpp<DPP_QUAD_1032>(v));
    v = fmaxf(v, dpp<DPP_QUAD_2301>(v));
    v = fmaxf(v, dpp<DPP_ROW_HMIRROR>(v));
    if constexpr (W >= 16) v = fmaxf(v, dpp<DPP_ROW_MIRROR>(v));
    if constexpr (W >= 32) v = max_xor16(v);
    if constexpr (W >= 64) v = max_xor32(v);
    return v;
}

// 2^x with 2^-inf = 0.
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Scale factor 2^(m_old - m_new) of an online-softmax state, 0 for an empty state.
__device__ __forceinline__ float rescale(float m_old, float m_new)
{
    return m_old == kNegInf ? 0.0f : exp2_(m_old - m_new);
}

// ---- matrix-core and buffer-load helpers ----------------------------------

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// Raw buffer resource over [base, base + bytes): loads outside return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The same with the non-temporal hint: for rows streamed once.  Loads that cover
// whole 128-byte lines stream faster with it (measured on a plain read of the
// decode step's bytes: 6.2 against 5.5 TB/s); loads that take half a line per
// instruction get slower, so it goes only on whole-row loads.
__device__ __forceinline__ uint4 buffer_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t buffer_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Ordering point for LDS data passed between lanes of one wave (a wave
// executes its LDS instructions in order; this keeps the compiler from
// moving loads and stores across it).
__device__ __forceinline__ void wave_lds_fence()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// q of up to 16 heads as the B operand of v_mfma_f32_16x16x32_bf16 for a
// 32-element k-step s: lane (n16, g16) holds head n16 (zero past nh), 16-byte
// chunk 4 s + g16 of the row.  Rows are loaded as the A operand with the same
// chunk assignment (row n16 of the 16-row block, chunk 4 s + g16), so the MFMA
// sums q . k over the chunks of the k-step; over all D/32 steps it is q . k.
template <int D>
__device__ __forceinline__ void load_q_operand(const char* q_first_head, int nh, int lane, bf16x8_t (&bq)[D / 32])
{
    const int n16 = lane & 15, g16 = lane >> 4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (n16 < nh) v = ld16(q_first_head + (size_t)n16 * D * 2 + (4 * s + g16) * 16);
        bq[s] = __builtin_bit_cast(bf16x8_t, v);
    }
}

// fp64 -> bfloat16 bit pattern, round to nearest with ties to even, in one step.
__device__ __forceinline__ uint16_t bf16_from_f64(double x)
{
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
    const uint64_t mag = u & 0x7fffffffffffffffull;
    if (mag > 0x7ff0000000000000ull) return 0x7fc0;  // NaN
    if ((mag >> 52) >= 897) {                        // |x| >= 2^-126: a normal bfloat16
        // keep 7 of the 52 fraction bits; add half an ulp minus one, plus the kept lsb
        const uint64_t r = (mag + 0x00000fffffffffffull + ((mag >> 45) & 1u)) >> 45;
        const uint64_t b = r - (static_cast<uint64_t>(1023 - 127) << 7);  // rebias exponent
        return b >= 0x7f80u ? static_cast<uint16_t>(sign | 0x7f80u) : static_cast<uint16_t>(sign | b);
    }
    // below 2^-126 the spacing is 2^-133: round |x| * 2^133 to an integer (0..128)
    const double q = __builtin_rint(__builtin_ldexp(__builtin_fabs(x), 133));
    return static_cast<uint16_t>(sign | static_cast<uint16_t>(q));
}

}  // namespace csa

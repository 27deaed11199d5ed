// Device-side helpers shared by the gfx950 kernels: element conversions,
// 16-byte vector loads/stores and wave64 cross-lane reductions built from DPP
// and the gfx950 permlane swaps (no LDS round trip, no ds_bpermute).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)bits16);
}

// float -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the default
// rounding mode).
__device__ __forceinline__ uint32_t f32_to_half_bits(float f)
{
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)f);
}

// A binary16 input or output element.  bf16 elements are carried as plain
// uint16_t bit patterns; this distinct type selects the binary16 conversions.
struct f16_t {
    uint16_t bits;
};
template <typename T> struct is_f16 { static constexpr bool value = false; };
template <> struct is_f16<f16_t> { static constexpr bool value = true; };

// The low / high element of a 32-bit word holding two 2-byte inputs of type T
// (bf16 bits or binary16).
template <typename T> __device__ __forceinline__ float lo16(uint32_t w)
{
    if constexpr (is_f16<T>::value) return half_bits_to_f32(w & 0xffffu);
    else return bf16_lo(w);
}
template <typename T> __device__ __forceinline__ float hi16(uint32_t w)
{
    if constexpr (is_f16<T>::value) return half_bits_to_f32(w >> 16);
    else return bf16_hi(w);
}

// ------------------------------------------------------------ loads / stores

template <typename T>
__device__ __forceinline__ T ld_nt(const T *p) { return __builtin_nontemporal_load(p); }

template <typename T>
__device__ __forceinline__ void st_nt(T *p, T v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ float load_one(const float *p) { return *p; }
__device__ __forceinline__ float load_one(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
__device__ __forceinline__ float load_one(const f16_t *p) { return half_bits_to_f32(p->bits); }

// Store 4 consecutive outputs (fp32: 16 bytes, bf16 / binary16: 8 bytes).
__device__ __forceinline__ void store_out4(float *p, const float (&o)[4])
{
    f32x4 t = {o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4 *>(p) = t;
}
__device__ __forceinline__ void store_out4(uint16_t *p, const float (&o)[4])
{
    u32x2 t = {f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16),
               f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16)};
    *reinterpret_cast<u32x2 *>(p) = t;
}
__device__ __forceinline__ void store_out4(f16_t *p, const float (&o)[4])
{
    u32x2 t = {f32_to_half_bits(o[0]) | (f32_to_half_bits(o[1]) << 16),
               f32_to_half_bits(o[2]) | (f32_to_half_bits(o[3]) << 16)};
    *reinterpret_cast<u32x2 *>(p) = t;
}
__device__ __forceinline__ void store_one(float *p, float o) { *p = o; }
__device__ __forceinline__ void store_one(uint16_t *p, float o) { *p = (uint16_t)f32_to_bf16(o); }
__device__ __forceinline__ void store_one(f16_t *p, float o) { p->bits = (uint16_t)f32_to_half_bits(o); }

// ------------------------------------------------------------ lane exchange

// DPP controls (gfx9 encoding).
enum : int {
    DPP_QUAD_XOR1 = 0xB1,     // quad_perm [1,0,3,2]
    DPP_QUAD_XOR2 = 0x4E,     // quad_perm [2,3,0,1]
    DPP_ROW_ROR8 = 0x128,     // rotate right by 8 within a 16-lane row == xor 8
    DPP_ROW_MIRROR = 0x140,   // lane i <- lane 15-i within a row
    DPP_ROW_HALF_MIRROR = 0x141 // lane i <- lane 7-i within each 8-lane half row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum of lanes l and l^16 in every lane (gfx950 v_permlane16_swap: odd 16-lane
// rows of the first operand trade places with even rows of the second).  The
// operands are added in the same order in both lanes, so the pair holds
// bitwise-identical sums.
__device__ __forceinline__ float sum_xor16(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor8(float x)
{
    // lane l reads l^8; fp add is commutative so both lanes get the same bits
    return x + dpp<DPP_ROW_ROR8>(x);
}

// Sum over lane bits FIRST..5 (i.e. over the 64 >> FIRST lane groups that
// share the low FIRST bits); every participating lane receives the total.
template <int FIRST>
__device__ __forceinline__ float sum_lane_bits(float x)
{
    static_assert(FIRST >= 3 && FIRST <= 6, "reductions start at lane bit 3, 4 or 5");
    if constexpr (FIRST <= 3) x = sum_xor8(x);
    if constexpr (FIRST <= 4) x = sum_xor16(x);
    if constexpr (FIRST <= 5) x = sum_xor32(x);
    return x;
}

// Reduce-scatter of 8 column partials over lane bits 4 and 5 (4 row groups of
// 16 lanes): one v_permlane16_swap pairs column c of the even 16-lane rows with
// column c + 4 of the odd rows, so a single add leaves the even rows holding
// column c and the odd rows column c + 4 (no copies); v_permlane32_swap then
// does the same between lane halves for columns c and c + 2.  Afterwards lane
// l holds, in o[0..1], the full 4-row-group sums of its columns
// 4 * bit4(l) + 2 * bit5(l) + {0, 1}.  Sums are ((g0 + g1) + (g2 + g3)).
__device__ __forceinline__ void reduce_scatter_rows4(const float (&a)[8], float (&o)[2])
{
    float s1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[c]), __float_as_uint(a[c + 4]),
                                                  false, false);
        s1[c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s1[c]),
                                                  __float_as_uint(s1[c + 2]), false, false);
        o[c] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

// Column offset (within the lane's 8) of o[0] after reduce_scatter_rows4.
__device__ __forceinline__ int reduce_scatter_rows4_col(int lane)
{
    return 4 * ((lane >> 4) & 1) + 2 * ((lane >> 5) & 1);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}

// Maximum of non-negative finite floats over the low NB lane bits (NB = 2:
// groups of 4 lanes, 3: groups of 8, 4: groups of 16).  Non-negative IEEE floats order like
// their bit patterns as unsigned integers, so the reduction runs on v_max_u32
// with the DPP lane exchange fused into it (no NaN canonicalisation).  max is
// exact, so any pairing pattern gives the same result.
template <int NB>
__device__ __forceinline__ float max_low_lane_bits(float x)
{
    static_assert(NB >= 2 && NB <= 4, "groups of 4, 8 or 16 lanes");
    uint32_t u = __float_as_uint(x);
    u = max(u, dpp_u32<DPP_QUAD_XOR1>(u));
    u = max(u, dpp_u32<DPP_QUAD_XOR2>(u));
    if constexpr (NB >= 3) u = max(u, dpp_u32<DPP_ROW_HALF_MIRROR>(u));
    if constexpr (NB == 4) u = max(u, dpp_u32<DPP_ROW_MIRROR>(u));
    return __uint_as_float(u);
}

} // namespace hla

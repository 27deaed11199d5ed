// INT8 / FP16 row codec on gfx950 registers, shared by the mixed-precision
// state step ("DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization",
// §3.2 Eq. (5)-(6)) and the INT8 checkpoint kernels ("dasc: Decay-Aware State
// Compression for Hybrid Linear-Attention Serving", App. E.1 Eq. (8)): symmetric
// codes in [-127, 127], no zero point, s = max(amax, 1e-8) / 127 in FP32.
//
//   scale s = fl(max(amax, 1e-8) / 127), bit-identical to the IEEE division
//     (reciprocal multiply + one FMA correction, see div127);
//   inv = v_rcp_f32(s), within an ulp of 1/s;
//   code = round-half-even of the exact product x * inv, formed as the low
//     byte of fma(x, inv, 1.5 * 2^23): the FMA adds 1.5 * 2^23 before its
//     single rounding, where the FP32 ulp is 1, so the rounding is exactly
//     rne(x * inv), and the low 8 mantissa bits are the two's-complement code.
//     |x * inv| <= amax * inv < 127.5 because s >= amax/127 * (1 - 2^-24) and
//     inv <= (1/s)(1 + 2^-22), so no clamp is needed for finite values.
//   This differs from rne(fl(x / s)) only when x / s lies within about 2e-5
//   of a half-integer.
#pragma once

#include <hip/hip_runtime.h>

#include "hla_device.h"

namespace hla {

constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23


template <int CG>
struct Log2;
template <>
struct Log2<8> { static constexpr int v = 3; };
template <>
struct Log2<16> { static constexpr int v = 4; };

// Correctly rounded fl(a / 127) for normal a: one multiply by fl(1/127) and one
// FMA correction of the residual.  Checked exhaustively against the IEEE
// division over all 2^23 FP32 significands (the result only depends on the
// significand for normal inputs).
__device__ __forceinline__ float div127(float a)
{
    constexpr float y = 1.0f / 127.0f;
    const float q0 = a * y;
    const float r = fmaf(-q0, 127.0f, a);
    return fmaf(r, y, q0);
}

// Dequantise one packed 8-value row segment, scaled by `a` (decay, or 1).
__device__ __forceinline__ void decode_fp16(const uint32_t (&w)[4], float a, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = half_bits_to_f32(w[i] & 0xffffu) * a;
        x[2 * i + 1] = half_bits_to_f32(w[i] >> 16) * a;
    }
}

// code * (a * s) for the 8 signed bytes of w0 (values 0..3) and w1 (4..7).
__device__ __forceinline__ void decode_int8(uint32_t w0, uint32_t w1, float as, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = (float)(int)(int8_t)(w0 >> (8 * i)) * as;
        x[4 + i] = (float)(int)(int8_t)(w1 >> (8 * i)) * as;
    }
}

__device__ __forceinline__ void encode_fp16(const float (&x)[8], uint32_t (&w)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = f32_to_half_bits(x[2 * i]) | (f32_to_half_bits(x[2 * i + 1]) << 16);
}

// Quantise the lane's 8 values of a row whose full-row maximum is amax.
// Returns the FP32 scale s = fl(max(amax, 1e-8) / 127); the codes land in w0
// (values 0..3) and w1 (4..7).  inv is v_rcp_f32's reciprocal of s (within an
// ulp): amax * inv stays below 127.5, so every code lies in [-127, 127].
__device__ __forceinline__ float encode_int8(const float (&x)[8], float amax, uint32_t &w0,
                                             uint32_t &w1)
{
    const float s = div127(fmaxf(amax, 1e-8f));
    const float inv = __builtin_amdgcn_rcpf(s);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __float_as_uint(fmaf(x[i], inv, kRoundMagic));
    // gather the low bytes: perm(hi, lo, sel) picks bytes of {hi:lo}
    const uint32_t a01 = __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u);
    const uint32_t a23 = __builtin_amdgcn_perm(c[3], c[2], 0x0c0c0400u);
    const uint32_t a45 = __builtin_amdgcn_perm(c[5], c[4], 0x0c0c0400u);
    const uint32_t a67 = __builtin_amdgcn_perm(c[7], c[6], 0x0c0c0400u);
    w0 = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
    w1 = __builtin_amdgcn_perm(a67, a45, 0x05040100u);
    return s;
}

// max |x_i| of 8 finite floats.  v_max3_f32 takes |.| source modifiers, so the
// whole row segment is 3 max3 + 1 max (the compiler's maxnum lowering would
// first canonicalise every |x_i| in IEEE mode).  max is exact and the inputs
// are finite FMA results, so the result equals the plain definition.
__device__ __forceinline__ float row_absmax8(const float (&x)[8])
{
    float m;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(m) : "v"(x[0]), "v"(x[1]), "v"(x[2]));
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(m) : "v"(m), "v"(x[3]), "v"(x[4]));
    asm("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(m) : "v"(m), "v"(x[5]), "v"(x[6]));
    asm("v_max_f32 %0, %1, |%2|" : "=v"(m) : "v"(m), "v"(x[7]));
    return m;
}

} // namespace hla

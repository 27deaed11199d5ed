// gfx950 kernels for the mixed-precision recurrent state ("DAMP: Decay-Aware
// Mixed-Precision Recurrent-State Quantization", §3.2-§3.3 and §5.2 / App. A.4):
// K_hi key-channel rows per head in FP16, the rest symmetric INT8 with one
// FP32 scale per row, updated by one fused dequantise -> FP32 update and
// readout -> requantise pass.
//
// Work decomposition.  The requantisation needs the maximum of each row over
// all dv columns and the update needs column sums over all dk rows, so one
// workgroup owns a whole head: (dk/8) x (dv/8) threads, thread (rg, cg) holds
// an 8 x 8 block, rows 8*rg.., columns 8*cg...  A row block of dv values is
// spread over dv/8 consecutive lanes (one DPP row for dv = 128), so the row
// maximum is a 4-step DPP max.  Column sums run in-lane over 8 rows, then over
// the row blocks of the wave (permlane swaps), then over the waves through a
// 4 KiB LDS table.  Each INT8 load/store instruction covers 128 contiguous
// bytes per row.
//
// Codec arithmetic (FP32 throughout, as the pages state for the quantiser):
//   dequantise + decay in one FMA: with w = code ^ 0x80 read as an unsigned
//     byte (code + 128), a * (code * s) = fl((w - 128) * fl(a * s)) is
//     fma(w, as, -128 as), exact apart from the final rounding;
//   scale s = fl(max(amax, 1e-8) / 127) with an IEEE division (bit-identical
//     to the definition), inv = fl(1 / s);
//   code = round-half-even of the exact product x * inv, formed as the low
//     byte of fma(x, inv, 1.5 * 2^23): the FMA adds 1.5 * 2^23 before its
//     single rounding, where the FP32 ulp is 1, so the rounding is exactly
//     rne(x * inv), and the low 8 mantissa bits are the two's-complement code.
//     |x * inv| <= amax * inv < 127.5 because s >= amax/127 * (1 - 2^-24) and
//     inv >= 1/s * (1 - 2^-24), so no clamp is needed for finite states.
//   This differs from rne(fl(x / s)) only when x / s lies within about 1e-5
//   of a half-integer.
#include <hip/hip_runtime.h>

#include "hla.h"
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23

template <int CG>
struct Log2;
template <>
struct Log2<8> { static constexpr int v = 3; };
template <>
struct Log2<16> { static constexpr int v = 4; };

// Dequantise one packed 8-value row segment, scaled by `a` (decay, or 1).
__device__ __forceinline__ void decode_fp16(const uint32_t (&w)[4], float a, float (&x)[8])
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = half_bits_to_f32(w[i] & 0xffffu) * a;
        x[2 * i + 1] = half_bits_to_f32(w[i] >> 16) * a;
    }
}

__device__ __forceinline__ void decode_int8(uint32_t w0, uint32_t w1, float as, float (&x)[8])
{
    const float nb = -128.0f * as;  // exact: power-of-two multiple
    w0 ^= 0x80808080u;
    w1 ^= 0x80808080u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = fmaf((float)((w0 >> (8 * i)) & 0xffu), as, nb);
        x[4 + i] = fmaf((float)((w1 >> (8 * i)) & 0xffu), as, nb);
    }
}

__device__ __forceinline__ void encode_fp16(const float (&x)[8], uint32_t (&w)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = f32_to_half_bits(x[2 * i]) | (f32_to_half_bits(x[2 * i + 1]) << 16);
}

// Quantise the lane's 8 values of a row whose full-row maximum is amax.
// Returns the FP32 scale; the codes land in w0 (values 0..3), w1 (4..7).
__device__ __forceinline__ float encode_int8(const float (&x)[8], float amax, uint32_t &w0,
                                             uint32_t &w1)
{
    const float s = __fdiv_rn(fmaxf(amax, 1e-8f), 127.0f);
    const float inv = __frcp_rn(s);
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

__device__ __forceinline__ float row_absmax8(const float (&x)[8])
{
    float m = fabsf(x[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
    return m;
}

// ------------------------------------------------------------------ step

template <int DK, int DV, typename TIn, typename TOut, bool VEC>
__global__ void __launch_bounds__((DK / 8) * (DV / 8))
k_damp_step(uint16_t *__restrict__ hi, int8_t *__restrict__ lo, float *__restrict__ lo_scale,
            int n_slots, const int32_t *__restrict__ key_perm, int K_hi,
            const int32_t *__restrict__ slot, int H, const TIn *__restrict__ q,
            const TIn *__restrict__ k, const TIn *__restrict__ v,
            const float *__restrict__ alpha, const float *__restrict__ beta,
            TOut *__restrict__ out, int32_t *__restrict__ err)
{
    constexpr int CG = DV / 8;            // lanes per row block
    constexpr int LCG = Log2<CG>::v;
    constexpr int NW = (DK / 8) * CG / 64;  // waves per head
    __shared__ float ks[DK], qs[DK], as_[VEC ? DK : 1];
    __shared__ float red_r[NW][DV], red_p[NW][DV], red_qk[NW];
    __shared__ float us[DV];

    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int s = slot ? slot[b] : b;
    if (s < 0) return;
    if (s >= n_slots) {
        if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cg = t & (CG - 1), rg = t >> LCG;
    const int row0 = rg * 8, col0 = cg * 8;
    const int nlo = DK - K_hi;
    const size_t sh = (size_t)s * H + h;
    uint16_t *hrow = hi + (sh * K_hi) * DV + col0;
    int8_t *lrow = lo + (sh * nlo) * DV + col0;
    float *srow = lo_scale + sh * nlo;

    // 1. packed rows of this thread, straight from HBM
    uint32_t raw[8][4];
    float sc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = row0 + m;
        if (r < K_hi) {
            u32x4 w = ld_nt(reinterpret_cast<const u32x4 *>(hrow + (size_t)r * DV));
            raw[m][0] = w.x; raw[m][1] = w.y; raw[m][2] = w.z; raw[m][3] = w.w;
            sc[m] = 1.0f;
        } else {
            u32x2 w = ld_nt(reinterpret_cast<const u32x2 *>(lrow + (size_t)(r - K_hi) * DV));
            raw[m][0] = w.x; raw[m][1] = w.y; raw[m][2] = 0u; raw[m][3] = 0u;
            sc[m] = srow[r - K_hi];
        }
    }
    // 2. k, q (and a vector decay) in packed row order
    if (t < DK) {
        int u = key_perm ? key_perm[h * DK + t] : t;
        if ((unsigned)u >= (unsigned)DK) {
            if (err) atomicOr(err, HLA_DEVERR_PLAN);
            u = t;
        }
        ks[t] = load_one(k + (size_t)bh * DK + u);
        qs[t] = load_one(q + (size_t)bh * DK + u);
        if constexpr (VEC) as_[t] = alpha[(size_t)bh * DK + u];
    }
    const float a_head = VEC ? 0.0f : alpha[bh];
    const float bt = beta[bh];
    __syncthreads();

    // 3. dequantise with the decay folded in; partial column sums
    float x[8][8];
    float pr[8], pp[8], qk = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) pr[c] = pp[c] = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = row0 + m;
        const float a = VEC ? as_[r] : a_head;
        if (r < K_hi)
            decode_fp16(raw[m], a, x[m]);
        else
            decode_int8(raw[m][0], raw[m][1], a * sc[m], x[m]);
        const float kr = ks[r], qr = qs[r];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            pr[c] = fmaf(kr, x[m][c], pr[c]);
            pp[c] = fmaf(qr, x[m][c], pp[c]);
        }
        qk = fmaf(qr, kr, qk);
    }
    // 4. column sums: row blocks inside the wave, then across waves
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        pr[c] = sum_lane_bits<LCG>(pr[c]);
        pp[c] = sum_lane_bits<LCG>(pp[c]);
    }
    qk = sum_lane_bits<LCG>(qk);
    if (lane < CG) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            red_r[wave][col0 + c] = pr[c];
            red_p[wave][col0 + c] = pp[c];
        }
        if (lane == 0) red_qk[wave] = qk;
    }
    __syncthreads();
    if (t < DV) {
        float R = 0.0f, P = 0.0f, QK = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            R += red_r[w][t];
            P += red_p[w][t];
            QK += red_qk[w];
        }
        const float u = bt * (load_one(v + (size_t)bh * DV + t) - R);  // u = beta (v - S'^T k)
        us[t] = u;
        if (out) store_one(out + (size_t)bh * DV + t, fmaf(QK, u, P));  // o = S^T q
    }
    __syncthreads();
    float u8[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) u8[c] = us[col0 + c];

    // 5. rank-1 write, requantise, store
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = row0 + m;
        const float kr = ks[r];
#pragma unroll
        for (int c = 0; c < 8; ++c) x[m][c] = fmaf(kr, u8[c], x[m][c]);
        if (r < K_hi) {
            uint32_t w[4];
            encode_fp16(x[m], w);
            u32x4 t4 = {w[0], w[1], w[2], w[3]};
            st_nt(reinterpret_cast<u32x4 *>(hrow + (size_t)r * DV), t4);
        } else {
            const float amax = max_low_lane_bits<LCG>(row_absmax8(x[m]));
            uint32_t w0, w1;
            const float scale = encode_int8(x[m], amax, w0, w1);
            u32x2 t2 = {w0, w1};
            st_nt(reinterpret_cast<u32x2 *>(lrow + (size_t)(r - K_hi) * DV), t2);
            if (cg == 0) srow[r - K_hi] = scale;
        }
    }
}

// ------------------------------------------------------------------ codec

template <int DK, int DV>
__global__ void __launch_bounds__((DK / 8) * (DV / 8))
k_damp_quantize(const float *__restrict__ state, int H, const int32_t *__restrict__ key_perm,
                int K_hi, uint16_t *__restrict__ hi, int8_t *__restrict__ lo,
                float *__restrict__ lo_scale)
{
    constexpr int CG = DV / 8;
    constexpr int LCG = Log2<CG>::v;
    const size_t sh = blockIdx.x;
    const int h = (int)(sh % H);
    const int t = threadIdx.x, cg = t & (CG - 1), rg = t >> LCG;
    const int nlo = DK - K_hi;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = rg * 8 + m;
        int u = key_perm ? key_perm[h * DK + r] : r;
        if ((unsigned)u >= (unsigned)DK) u = r;  // host-built plans are permutations
        const float *src = state + (sh * DK + u) * DV + cg * 8;
        f32x4 a = reinterpret_cast<const f32x4 *>(src)[0];
        f32x4 c = reinterpret_cast<const f32x4 *>(src)[1];
        float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        if (r < K_hi) {
            uint32_t w[4];
            encode_fp16(x, w);
            u32x4 t4 = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4 *>(hi + (sh * K_hi + r) * DV + cg * 8) = t4;
        } else {
            const float amax = max_low_lane_bits<LCG>(row_absmax8(x));
            uint32_t w0, w1;
            const float scale = encode_int8(x, amax, w0, w1);
            u32x2 t2 = {w0, w1};
            *reinterpret_cast<u32x2 *>(lo + (sh * nlo + (r - K_hi)) * DV + cg * 8) = t2;
            if (cg == 0) lo_scale[sh * nlo + (r - K_hi)] = scale;
        }
    }
}

template <int DK, int DV>
__global__ void __launch_bounds__((DK / 8) * (DV / 8))
k_damp_dequantize(const uint16_t *__restrict__ hi, const int8_t *__restrict__ lo,
                  const float *__restrict__ lo_scale, int H, const int32_t *__restrict__ key_perm,
                  int K_hi, float *__restrict__ state)
{
    constexpr int CG = DV / 8;
    constexpr int LCG = Log2<CG>::v;
    const size_t sh = blockIdx.x;
    const int h = (int)(sh % H);
    const int t = threadIdx.x, cg = t & (CG - 1), rg = t >> LCG;
    const int nlo = DK - K_hi;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = rg * 8 + m;
        int u = key_perm ? key_perm[h * DK + r] : r;
        if ((unsigned)u >= (unsigned)DK) u = r;
        float x[8];
        if (r < K_hi) {
            u32x4 w = *reinterpret_cast<const u32x4 *>(hi + (sh * K_hi + r) * DV + cg * 8);
            uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            decode_fp16(ww, 1.0f, x);
        } else {
            u32x2 w = *reinterpret_cast<const u32x2 *>(lo + (sh * nlo + (r - K_hi)) * DV + cg * 8);
            decode_int8(w.x, w.y, lo_scale[sh * nlo + (r - K_hi)], x);
        }
        float *dst = state + (sh * DK + u) * DV + cg * 8;
        f32x4 a = {x[0], x[1], x[2], x[3]}, c = {x[4], x[5], x[6], x[7]};
        reinterpret_cast<f32x4 *>(dst)[0] = a;
        reinterpret_cast<f32x4 *>(dst)[1] = c;
    }
}

// ------------------------------------------------------------------ dispatch

template <int DK, int DV, typename TIn, typename TOut>
static int launch_damp_typed(const DampArgs &a, int32_t *err, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)a.B * a.H)), block((DK / 8) * (DV / 8));
    if (a.decay == HLA_DECAY_VECTOR)
        hipLaunchKernelGGL((k_damp_step<DK, DV, TIn, TOut, true>), grid, block, 0, st, a.hi, a.lo,
                           a.lo_scale, a.n_slots, a.key_perm, a.K_hi, a.slot, a.H,
                           (const TIn *)a.q, (const TIn *)a.k, (const TIn *)a.v, a.alpha, a.beta,
                           (TOut *)a.out, err);
    else
        hipLaunchKernelGGL((k_damp_step<DK, DV, TIn, TOut, false>), grid, block, 0, st, a.hi,
                           a.lo, a.lo_scale, a.n_slots, a.key_perm, a.K_hi, a.slot, a.H,
                           (const TIn *)a.q, (const TIn *)a.k, (const TIn *)a.v, a.alpha, a.beta,
                           (TOut *)a.out, err);
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

template <int DK, int DV>
static int launch_damp_dtypes(const DampArgs &a, int32_t *err, hipStream_t st)
{
    const bool in16 = a.in_dtype == HLA_BF16, out16 = a.out_dtype == HLA_BF16;
    if (in16)
        return out16 ? launch_damp_typed<DK, DV, uint16_t, uint16_t>(a, err, st)
                     : launch_damp_typed<DK, DV, uint16_t, float>(a, err, st);
    return out16 ? launch_damp_typed<DK, DV, float, uint16_t>(a, err, st)
                 : launch_damp_typed<DK, DV, float, float>(a, err, st);
}

template <int DK, int DV>
static int launch_codec(bool quantize, const float *state_in, float *state_out, int n_slots, int H,
                        const int32_t *key_perm, int K_hi, uint16_t *hi, int8_t *lo,
                        float *lo_scale, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)n_slots * H)), block((DK / 8) * (DV / 8));
    if (quantize)
        hipLaunchKernelGGL((k_damp_quantize<DK, DV>), grid, block, 0, st, state_in, H, key_perm,
                           K_hi, hi, lo, lo_scale);
    else
        hipLaunchKernelGGL((k_damp_dequantize<DK, DV>), grid, block, 0, st, hi, lo, lo_scale, H,
                           key_perm, K_hi, state_out);
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

static int run_codec(bool quantize, const float *state_in, float *state_out, int n_slots, int H,
                     int dk, int dv, const int32_t *key_perm, int K_hi, uint16_t *hi, int8_t *lo,
                     float *lo_scale, void *stream)
{
    const void *st_ptr = quantize ? (const void *)state_in : (const void *)state_out;
    int rc = check_damp_codec(st_ptr, n_slots, H, dk, dv, K_hi, hi, lo, lo_scale);
    if (rc != HLA_OK || n_slots == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
#define HLA_CODEC(DK_, DV_)                                                                   \
    if (dk == DK_ && dv == DV_)                                                               \
        return launch_codec<DK_, DV_>(quantize, state_in, state_out, n_slots, H, key_perm, K_hi, \
                                      hi, lo, lo_scale, st);
    HLA_CODEC(128, 128)
    HLA_CODEC(128, 64)
    HLA_CODEC(64, 128)
    HLA_CODEC(64, 64)
#undef HLA_CODEC
    return HLA_ERR_UNSUPPORTED;
}

} // namespace hla

extern "C" {

int damp_step(uint16_t *hi, int8_t *lo, float *lo_scale, int n_slots, const int32_t *key_perm,
              int K_hi, const int32_t *slot, int B, int H, int dk, int dv, const void *q,
              const void *k, const void *v, int in_dtype, const float *alpha, int decay_kind,
              const float *beta, void *out, int out_dtype, int32_t *err_flag, void *stream)
{
    hla::DampArgs a{hi, lo, lo_scale, n_slots, key_perm, K_hi, slot, B, H, dk, dv, q, k, v,
                    in_dtype, alpha, decay_kind, beta, out, out_dtype};
    int rc = hla::check_damp(a);
    if (rc != HLA_OK || B == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dk == 128 && dv == 128) return hla::launch_damp_dtypes<128, 128>(a, err_flag, st);
    if (dk == 128 && dv == 64) return hla::launch_damp_dtypes<128, 64>(a, err_flag, st);
    if (dk == 64 && dv == 128) return hla::launch_damp_dtypes<64, 128>(a, err_flag, st);
    return hla::launch_damp_dtypes<64, 64>(a, err_flag, st);
}

int damp_quantize(const float *state, int n_slots, int H, int dk, int dv, const int32_t *key_perm,
                  int K_hi, uint16_t *hi, int8_t *lo, float *lo_scale, void *stream)
{
    return hla::run_codec(true, state, nullptr, n_slots, H, dk, dv, key_perm, K_hi, hi, lo,
                          lo_scale, stream);
}

int damp_dequantize(const uint16_t *hi, const int8_t *lo, const float *lo_scale, int n_slots,
                    int H, int dk, int dv, const int32_t *key_perm, int K_hi, float *state,
                    void *stream)
{
    return hla::run_codec(false, nullptr, state, n_slots, H, dk, dv, key_perm, K_hi,
                          const_cast<uint16_t *>(hi), const_cast<int8_t *>(lo),
                          const_cast<float *>(lo_scale), stream);
}

} // extern "C"

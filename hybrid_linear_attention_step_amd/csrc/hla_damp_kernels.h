// gfx950 device code for the mixed-precision recurrent state ("DAMP:
// Decay-Aware Mixed-Precision Recurrent-State Quantization", §3.2-§3.3, §5.2
// and App. A.1-A.4): K_hi key-channel rows per head in FP16, the rest
// symmetric INT8 with one FP32 scale per row or per group of 32 values,
// updated by one fused dequantise -> FP32 update and readout -> requantise
// pass.  Shared by hla_damp.hip (entry points, codec, per-row-scale step
// variants) and hla_damp_sr.hip (group-scale and value-transform variants).
//
// Work decomposition.  The requantisation needs the maximum of each row over
// all dv columns and the update needs column sums over all dk rows, so one
// workgroup owns a whole head: (dk/8) x (dv/8) threads, each holding 8 rows x
// 8 adjacent columns.  A row's dv values are spread over dv/8 consecutive lanes
// (one DPP row for dv = 128), so the row maximum is a 4-step DPP max.  Column
// sums run in-lane over 8 rows, then over the row groups of the wave (permlane
// swaps), then over the waves through a 4 KiB LDS table.  Each INT8 load/store
// instruction covers whole 128-byte rows.
//
// Codec arithmetic (FP32 throughout, as the pages state for the quantiser):
//   see hla_codec.h; dequantise + decay is signed byte -> float (exact) times
//   fl(a * s).
//
// Scale groups ([DAMP] App. A.1 / A.4).  INT8 rows carry one FP32 scale per
// group of 8 << LG consecutive stored values: LG = log2(dv / 8) is one scale per
// row, LG = 2 one per 32 values.  A group is 4 (LG = 2) or dv/8 adjacent lanes,
// so its maximum is a DPP max over the low LG lane bits.
//
// Value transform ([DAMP] App. A.3 Eq. (17)-(18), "SR").  The stored state is
// T = S D^-1 P_V^T: stored column j holds original value index pi(j) divided by
// c'_j.  The update runs on T unchanged except for its two value-side ends:
// v'_j = v_{pi(j)} / c'_j going in and o_{pi(j)} = c'_j (T^T q)_j coming out.
#pragma once

#include <hip/hip_runtime.h>

#include "hla.h"
#include "hla_codec.h"
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

// Sum the lane's column partials (8 columns of S'^T k and of S'^T q) and q.k
// over the row groups of this wave and write the wave's totals to LDS rows
// red_r / red_p (dv floats each) and red_qk.  LCG = log2 of lanes per row
// group: 4 (dv = 128, row groups on lane bits 4-5) or 3 (dv = 64, lane bits
// 3-5; bit 3 is folded first with a DPP butterfly).
template <int LCG>
__device__ __forceinline__ void wave_column_sums(float (&pr)[8], float (&pp)[8], float qk,
                                                 int lane, int col0, float *red_r,
                                                 float *red_p, float *red_qk)
{
    if constexpr (LCG == 3) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            pr[c] = sum_xor8(pr[c]);
            pp[c] = sum_xor8(pp[c]);
        }
    }
    float r2[2], p2[2];
    reduce_scatter_rows4(pr, r2);
    reduce_scatter_rows4(pp, p2);
    qk = sum_lane_bits<LCG>(qk);
    // with dv = 64 the lanes with bit 3 set hold duplicates of their partner's sums
    if (LCG == 4 || ((lane >> 3) & 1) == 0) {
        const int c = col0 + reduce_scatter_rows4_col(lane);
        red_r[c] = r2[0];
        red_r[c + 1] = r2[1];
        red_p[c] = p2[0];
        red_p[c + 1] = p2[1];
    }
    if (lane == 0) *red_qk = qk;
}

// ------------------------------------------------------------------ step
//
// Thread t of the (dk/8) x (dv/8) block: cg = t % (dv/8) picks 8 adjacent
// columns, g = t / (dv/8) a row group, and the thread owns packed rows
// g + (dk/8) m, m = 0..7.  Interleaving the rows this way gives every wave
// the same row index pattern per m, so the FP16 / INT8 choice is uniform
// across the block whenever K_hi is a multiple of dk/8 (K_hi = 16 at dk = 128).
// Each wave stages its own copy of k, q, the decay and the plan row into LDS
// with plain contiguous loads issued together with the state loads (the
// permutation is applied on the LDS read, so there is no dependent global
// gather), and no block barrier is needed before the math.  Two block
// barriers exchange the per-wave column sums and share u.

// MH >= 0: K_hi == MH * (dk/8), so the thread's rows m < MH are the FP16 ones
// and the choice is known at compile time (no branches, no registers held for
// the other format); MH < 0: any K_hi, decided per row at run time.
template <int DK, int DV, typename TIn, typename TOut, bool VEC, int MH, int LG, bool SR>
__global__ void __launch_bounds__((DK / 8) * (DV / 8))
k_damp_step(uint16_t *__restrict__ hi, int8_t *__restrict__ lo, float *__restrict__ lo_scale,
            int n_slots, const int32_t *__restrict__ key_perm, int K_hi,
            const int32_t *__restrict__ val_perm, const float *__restrict__ val_scale,
            const int32_t *__restrict__ slot, int H, const TIn *__restrict__ q,
            const TIn *__restrict__ k, const TIn *__restrict__ v,
            const float *__restrict__ alpha, const float *__restrict__ beta,
            TOut *__restrict__ out, int32_t *__restrict__ err)
{
    constexpr int CG = DV / 8;              // lanes per row group
    constexpr int LCG = Log2<CG>::v;
    constexpr int NRG = DK / 8;             // row groups = row stride between a thread's rows
    constexpr int NW = NRG * CG / 64;       // waves per head
    constexpr int NG = DV / (8 << LG);      // scales per INT8 row (one per 8 << LG values)
    static_assert(LG >= 2 && LG <= LCG, "scale groups of 32 values up to a whole row");
    __shared__ f32x4 kqa[NW][DK];  // {k, q, decay, 0} per original key channel
    __shared__ int pm_[NW][DK];
    __shared__ float red_r[NW][DV], red_p[NW][DV], red_qk[NW];
    __shared__ float us[DV];
    __shared__ float vsh[SR ? DV : 1];  // v by original value index (value permutation)
    __shared__ float csh[SR ? DV : 1];  // c'_j of stored column j
    __shared__ float rsh[SR ? DV : 1];  // 1 / c'_j (v_rcp_f32, within an ulp)
    __shared__ int psh[SR ? DV : 1];    // pi(j) of stored column j

    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int s = slot ? slot[b] : b;
    if (s < 0) return;
    if (s >= n_slots) {
        if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int cg = t & (CG - 1), g = t >> LCG;
    const int col0 = cg * 8;
    if constexpr (MH >= 0) K_hi = MH * NRG;
    const int nlo = DK - K_hi;
    const size_t sh = (size_t)s * H + h;
    uint16_t *hrow = hi + (sh * K_hi) * DV + col0;
    int8_t *lrow = lo + (sh * nlo) * DV + col0;
    float *srow = lo_scale + sh * nlo * NG;
    const int sgrp = cg >> LG;  // this lane's scale group within a row
    auto is_hi = [&](int m, int r) { return MH >= 0 ? (m < MH) : (r < K_hi); };

    // 1. this wave's copy of k, q, the decay and the plan row, read contiguously
    //    (no dependent gather; the permutation is applied when reading LDS).  These
    //    loads are issued first so that their latency hides under the state loads'.
    constexpr int SJ = DK / 64;  // staged channels per lane
    int st_p[SJ];
    float st_k[SJ], st_q[SJ], st_a[SJ];
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
        const int i = lane + 64 * j;
        st_p[j] = key_perm ? key_perm[h * DK + i] : i;
        st_k[j] = load_one(k + (size_t)bh * DK + i);
        st_q[j] = load_one(q + (size_t)bh * DK + i);
        st_a[j] = VEC ? alpha[(size_t)bh * DK + i] : 0.0f;
    }
    // value transform of column t: both loads are unconditional (a missing table reads
    // beta instead and the value is replaced when it is used), so no branch joins the
    // load stream; they land in LDS together with the staged inputs
    float cv_raw = 0.0f, vp_raw = 0.0f;
    if constexpr (SR) {
        const int tv = t & (DV - 1);
        cv_raw = *(val_scale ? val_scale + (size_t)h * DV + tv : beta + bh);
        vp_raw = *(val_perm ? reinterpret_cast<const float *>(val_perm) + (size_t)h * DV + tv
                            : beta + bh);
    }
    // 2. packed rows of this thread, straight from HBM, then their scales, then the
    //    per-head inputs.  All row loads are issued before the first 4-byte scale
    //    load: interleaving the two measured 9% slower even without arithmetic.
    uint32_t raw[8][4];
    float sc[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = g + NRG * m;
        if (is_hi(m, r)) {
            u32x4 w = ld_nt(reinterpret_cast<const u32x4 *>(hrow + (size_t)r * DV));
            raw[m][0] = w.x; raw[m][1] = w.y; raw[m][2] = w.z; raw[m][3] = w.w;
        } else {
            u32x2 w = ld_nt(reinterpret_cast<const u32x2 *>(lrow + (size_t)(r - K_hi) * DV));
            raw[m][0] = w.x; raw[m][1] = w.y; raw[m][2] = 0u; raw[m][3] = 0u;
        }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = g + NRG * m;
        sc[m] = is_hi(m, r) ? 1.0f : srow[(r - K_hi) * NG + sgrp];
    }
    // every thread loads (threads >= dv re-read a valid element and ignore it): a
    // conditional load would end in a wait for all outstanding loads
    const float vt = load_one(v + (size_t)bh * DV + (t & (DV - 1)));
    const float a_head = VEC ? 0.0f : alpha[bh];
    const float bt = beta[bh];
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
        pm_[wave][lane + 64 * j] = st_p[j];
        kqa[wave][lane + 64 * j] = f32x4{st_k[j], st_q[j], st_a[j], 0.0f};
    }
    if constexpr (SR) {
        if (t < DV) {  // whole waves in every instantiated shape
            csh[t] = val_scale ? cv_raw : 1.0f;
            rsh[t] = val_scale ? __builtin_amdgcn_rcpf(cv_raw) : 1.0f;
            psh[t] = val_perm ? __float_as_int(vp_raw) : t;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float kk[8], qq[8], aa[8];  // k, q and decay of each of the thread's packed rows
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        int u = pm_[wave][g + NRG * m];
        if ((unsigned)u >= (unsigned)DK) {
            if (err) atomicOr(err, HLA_DEVERR_PLAN);
            u = g + NRG * m;
        }
        const f32x4 e = kqa[wave][u];
        kk[m] = e.x;
        qq[m] = e.y;
        aa[m] = VEC ? e.z : a_head;
    }

    // 3. dequantise with the decay folded in; partial column sums
    float x[8][8];
    float pr[8], pp[8], qk = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) pr[c] = pp[c] = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = g + NRG * m;
        const float a = aa[m];
        if (is_hi(m, r))
            decode_fp16(raw[m], a, x[m]);
        else
            decode_int8(raw[m][0], raw[m][1], a * sc[m], x[m]);
        const float qr = qq[m];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            pr[c] = fmaf(kk[m], x[m][c], pr[c]);
            pp[c] = fmaf(qr, x[m][c], pp[c]);
        }
        qk = fmaf(qr, kk[m], qk);
    }
    // 4. column sums: row groups inside the wave, then the waves through LDS;
    //    thread j < dv finishes column j and shares u_j
    wave_column_sums<LCG>(pr, pp, qk, lane, col0, red_r[wave], red_p[wave], &red_qk[wave]);
    if constexpr (SR)
        if (t < DV) vsh[t] = vt;
    __syncthreads();
    if (t < DV) {
        float R = red_r[0][t], P = red_p[0][t], QK = red_qk[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            R += red_r[w][t];
            P += red_p[w][t];
            QK += red_qk[w];
        }
        float vv = vt, cv = 1.0f;
        int oj = t;
        if constexpr (SR) {
            // stored column t holds original value index pi(t), scaled by 1 / c'_t:
            // v'_t = v_{pi(t)} / c'_t, and the readout c'_t (T^T q)_t is o_{pi(t)}
            oj = psh[t];
            if ((unsigned)oj >= (unsigned)DV) {
                if (err) atomicOr(err, HLA_DEVERR_PLAN);
                oj = t;
            }
            vv = vsh[oj] * rsh[t];  // v' = v / c', to within two ulps
            cv = csh[t];
        }
        const float u = bt * (vv - R);   // u = beta (v - S'^T k)
        us[t] = u;
        if (out) {
            const float o = fmaf(QK, u, P);  // o = S^T q
            store_one(out + (size_t)bh * DV + oj, SR ? cv * o : o);
        }
    }
    __syncthreads();
    float u8[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) u8[c] = us[col0 + c];

    // 5. rank-1 write, requantise, store the rows, then the scales (as for the
    //    loads, the 4-byte scale stores go after every row store)
    float scale[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = g + NRG * m;
#pragma unroll
        for (int c = 0; c < 8; ++c) x[m][c] = fmaf(kk[m], u8[c], x[m][c]);
        scale[m] = 0.0f;
        if (is_hi(m, r)) {
            uint32_t w[4];
            encode_fp16(x[m], w);
            u32x4 t4 = {w[0], w[1], w[2], w[3]};
            st_nt(reinterpret_cast<u32x4 *>(hrow + (size_t)r * DV), t4);
        } else {
            const float amax = max_low_lane_bits<LG>(row_absmax8(x[m]));
            uint32_t w0, w1;
            scale[m] = encode_int8(x[m], amax, w0, w1);
            u32x2 t2 = {w0, w1};
            st_nt(reinterpret_cast<u32x2 *>(lrow + (size_t)(r - K_hi) * DV), t2);
        }
    }
    if ((cg & ((1 << LG) - 1)) == 0) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int r = g + NRG * m;
            if (!is_hi(m, r)) srow[(r - K_hi) * NG + sgrp] = scale[m];
        }
    }
}

// ------------------------------------------------------------------ codec
//
// Thread (rg, cg) of a head's (dk/8) x (dv/8) block converts packed rows
// rg*8 .. rg*8+7, stored columns cg*8 .. cg*8+7.  Stored column j of a row holds
// the original value index pi(j) = val_perm[h, j] scaled by 1 / val_scale[h, j]
// (identity / 1 when the table is NULL); with a permutation the FP32 side is
// gathered / scattered one value at a time (these kernels run once per request,
// not per token).

template <int DK, int DV, int LG>
__global__ void __launch_bounds__((DK / 8) * (DV / 8))
k_damp_quantize(const float *__restrict__ state, int H, const int32_t *__restrict__ key_perm,
                int K_hi, const int32_t *__restrict__ val_perm,
                const float *__restrict__ val_scale, uint16_t *__restrict__ hi,
                int8_t *__restrict__ lo, float *__restrict__ lo_scale)
{
    constexpr int CG = DV / 8;
    constexpr int LCG = Log2<CG>::v;
    constexpr int NG = DV / (8 << LG);
    const size_t sh = blockIdx.x;
    const int h = (int)(sh % H);
    const int t = threadIdx.x, cg = t & (CG - 1), rg = t >> LCG;
    const int nlo = DK - K_hi;
    int src[8];
    float cdiv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int j = cg * 8 + c;
        const int p = val_perm ? val_perm[(size_t)h * DV + j] : j;
        src[c] = (unsigned)p < (unsigned)DV ? p : j;  // host-built plans are permutations
        cdiv[c] = val_scale ? val_scale[(size_t)h * DV + j] : 1.0f;
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int r = rg * 8 + m;
        int u = key_perm ? key_perm[h * DK + r] : r;
        if ((unsigned)u >= (unsigned)DK) u = r;
        const float *row = state + (sh * DK + u) * DV;
        float x[8];
        if (val_perm) {
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = row[src[c]];
        } else {
            const f32x4 a = reinterpret_cast<const f32x4 *>(row + cg * 8)[0];
            const f32x4 b = reinterpret_cast<const f32x4 *>(row + cg * 8)[1];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
        if (val_scale) {
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = x[c] / cdiv[c];  // T = S / c'
        }
        if (r < K_hi) {
            uint32_t w[4];
            encode_fp16(x, w);
            u32x4 t4 = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4 *>(hi + (sh * K_hi + r) * DV + cg * 8) = t4;
        } else {
            const float amax = max_low_lane_bits<LG>(row_absmax8(x));
            uint32_t w0, w1;
            const float scale = encode_int8(x, amax, w0, w1);
            u32x2 t2 = {w0, w1};
            *reinterpret_cast<u32x2 *>(lo + (sh * nlo + (r - K_hi)) * DV + cg * 8) = t2;
            if ((cg & ((1 << LG) - 1)) == 0)
                lo_scale[(sh * nlo + (r - K_hi)) * NG + (cg >> LG)] = scale;
        }
    }
}

template <int DK, int DV, int LG>
__global__ void __launch_bounds__((DK / 8) * (DV / 8))
k_damp_dequantize(const uint16_t *__restrict__ hi, const int8_t *__restrict__ lo,
                  const float *__restrict__ lo_scale, int H, const int32_t *__restrict__ key_perm,
                  int K_hi, const int32_t *__restrict__ val_perm,
                  const float *__restrict__ val_scale, float *__restrict__ state)
{
    constexpr int CG = DV / 8;
    constexpr int LCG = Log2<CG>::v;
    constexpr int NG = DV / (8 << LG);
    const size_t sh = blockIdx.x;
    const int h = (int)(sh % H);
    const int t = threadIdx.x, cg = t & (CG - 1), rg = t >> LCG;
    const int nlo = DK - K_hi;
    int dst[8];
    float cmul[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int j = cg * 8 + c;
        const int p = val_perm ? val_perm[(size_t)h * DV + j] : j;
        dst[c] = (unsigned)p < (unsigned)DV ? p : j;
        cmul[c] = val_scale ? val_scale[(size_t)h * DV + j] : 1.0f;
    }
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
            decode_int8(w.x, w.y, lo_scale[(sh * nlo + (r - K_hi)) * NG + (cg >> LG)], x);
        }
        if (val_scale) {
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = x[c] * cmul[c];  // S = T c'
        }
        float *row = state + (sh * DK + u) * DV;
        if (val_perm) {
#pragma unroll
            for (int c = 0; c < 8; ++c) row[dst[c]] = x[c];
        } else {
            f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
            reinterpret_cast<f32x4 *>(row + cg * 8)[0] = a;
            reinterpret_cast<f32x4 *>(row + cg * 8)[1] = b;
        }
    }
}

// ------------------------------------------------------------------ launch

template <int DK, int DV, typename TIn, typename TOut, bool VEC, int MH, int LG, bool SR>
inline void launch_damp(const DampArgs &a, int32_t *err, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)a.B * a.H)), block((DK / 8) * (DV / 8));
    hipLaunchKernelGGL((k_damp_step<DK, DV, TIn, TOut, VEC, MH, LG, SR>), grid, block, 0, st,
                       a.hi, a.lo, a.lo_scale, a.n_slots, a.key_perm, a.K_hi, a.val_perm,
                       a.val_scale, a.slot, a.H, (const TIn *)a.q, (const TIn *)a.k,
                       (const TIn *)a.v, a.alpha, a.beta, (TOut *)a.out, err);
}

// Calls F::template run<DK, DV, TIn, TOut, VEC>(a, err, st) for the argument
// shapes and types (validated on the host before this point).
template <class F>
inline void damp_dispatch(const DampArgs &a, int32_t *err, hipStream_t st)
{
    const bool vec = a.decay == HLA_DECAY_VECTOR;
#define HLA_DAMP_T(DK_, DV_, TI_, TO_)                                                        \
    if (vec) F::template run<DK_, DV_, TI_, TO_, true>(a, err, st);                            \
    else F::template run<DK_, DV_, TI_, TO_, false>(a, err, st);
#define HLA_DAMP_O(DK_, DV_, TI_)                                                             \
    if (a.out_dtype == HLA_BF16) { HLA_DAMP_T(DK_, DV_, TI_, uint16_t) }                      \
    else if (a.out_dtype == HLA_F16) { HLA_DAMP_T(DK_, DV_, TI_, f16_t) }                     \
    else { HLA_DAMP_T(DK_, DV_, TI_, float) }
#define HLA_DAMP_S(DK_, DV_)                                                                  \
    if (a.dk == DK_ && a.dv == DV_) {                                                         \
        if (a.in_dtype == HLA_BF16) { HLA_DAMP_O(DK_, DV_, uint16_t) }                        \
        else if (a.in_dtype == HLA_F16) { HLA_DAMP_O(DK_, DV_, f16_t) }                       \
        else { HLA_DAMP_O(DK_, DV_, float) }                                                   \
        return;                                                                               \
    }
    HLA_DAMP_S(128, 128)
    HLA_DAMP_S(128, 64)
    HLA_DAMP_S(64, 128)
    HLA_DAMP_S(64, 64)
#undef HLA_DAMP_S
#undef HLA_DAMP_O
#undef HLA_DAMP_T
}

// Step launchers of the two groups of kernel variants (separate translation
// units, compiled in parallel).  Per-row scales without a value transform:
int launch_damp_rowscale(const DampArgs &a, int32_t *err, hipStream_t st);
// Group-32 scales, and any layout with a value transform:
int launch_damp_grouped_or_sr(const DampArgs &a, int32_t *err, hipStream_t st);

} // namespace hla

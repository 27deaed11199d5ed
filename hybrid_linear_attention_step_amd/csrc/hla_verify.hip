// gfx950 kernel for the verify pass of speculative decoding: the readouts at
// all K draft positions from the committed state, which is only read.
//
// Operation ("Serving recurrent attention", part "Speculative decoding without
// state snapshots"; the per-token update of "DAMP: Decay-Aware Mixed-Precision
// Recurrent-State Quantization", §3.1 Eq. (1)-(2)), per (request, head) with
// state S in dk x dv, for draft t = 1..K:
//     S'_t = Lambda_t S_{t-1},  u_t = beta_t (v_t - S'_t^T k_t),
//     S_t = S'_t + k_t u_t^T,  o_t = S_t^T q_t.
#include <hip/hip_runtime.h>

#include "hla.h"
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

// The verify pass needs the readouts at all K draft positions but never the
// updated state, so it is evaluated in unrolled form instead of token by
// token.  With c_t = prod_{s<=t} a_s (cumulative decay, per key channel) and
// w_st = prod_{s<r<=t} a_r, the recurrence S'_t = Lambda_t S_{t-1},
// u_t = beta_t (v_t - S'_t^T k_t), S_t = S'_t + k_t u_t^T unrolls to
//     S'_t = diag(c_t) S_0 + sum_{s<t} diag(w_st) k_s u_s^T, so
//     u_t = beta_t (v_t - S_0^T (c_t k_t) - sum_{s<t} G_st u_s),
//     o_t = S_t^T q_t = S_0^T (c_t q_t) + sum_{s<t} E_st u_s + E_tt u_t,
// with the scalars G_st = sum_i k_s,i w_st,i k_t,i and E_st = sum_i k_s,i
// w_st,i q_t,i (E_tt = k_t . q_t).  The state then costs two FMAs per
// element per draft (S_0^T (c_t k_t) and S_0^T (c_t q_t)) instead of four
// (decay, two sums, rank-1 write); the corrections are O(K^2 dk) per head
// and the solve O(K^2) per column.  The results equal the token-by-token
// recurrence up to rounding (a different summation order).
//
// Phases per head (workgroup of dv/32 waves, each owning 32 columns):
//   1. stage the K drafts' k, q, decay, v, beta into LDS and form c_t k_t and
//      c_t q_t (one thread per key channel walks the drafts), written straight
//      into the matrix-core operand layout below;
//   2. the pair sums G_st, E_st over chunks of key channels (the products
//      w_st are built incrementally, never as a ratio of cumulative decays, so
//      tiny decays cannot divide by an underflowed product), while the first
//      half of the tile arrives (issued right behind the staged inputs; the
//      second half is issued after the pair sums, which keeps the kernel
//      within five waves per SIMD);
//   3. R = S_0^T [c k | c q], a dk-deep contraction with 2K columns, on the
//      matrix cores: v_mfma_f32_16x16x4f32, FP32 in and FP32 accumulate;
//   4. one thread per column solves the K drafts in order and writes o_t.
//
// Matrix-core layout (16x16x4 FP32, one block): in each instruction lane l
// supplies A[l % 16][l / 16] and B[l / 16][l % 16] and receives
// D[4 (l / 16) + i][l % 16], i = 0..3.  Here A = S_0^T restricted to 16 column
// pairs and 4 rows: lane l = 16 rq + cm holds columns 32 w + 2 cm + {0, 1} of
// rows 4 s + rq (s = 0 .. dk/4 - 1), loaded as one 8-byte pair per row, so
// every load instruction of a wave covers 4 rows x 128 contiguous bytes; the
// two columns of the pair are two M blocks sharing the B operand.  B holds 16
// of the 2K right-hand columns: with KP = 8 NB padded drafts (NB = 1 for
// K <= 8, else 2), right-hand column g is c_t k_t (g = t) or c_t q_t
// (g = KP + t), zero for t >= K.  The output lane l receives columns
// 32 w + 8 rq + 0..7 of right-hand column 16 nb + cm.
constexpr int kPairChunks = 16;  // key-channel chunks of the pair sums

__host__ __device__ constexpr int verify_nb(int K) { return K <= 8 ? 1 : 2; }

// LDS strides chosen against bank conflicts (32 banks of 4 bytes): a staged
// draft row (k, q, per-channel decay) is dk + 16 floats, so the pair sums' 16
// lanes of one draft and the next draft's 16 lanes fall on different halves
// of the banks; an r0 / p0 row is dv + 4 floats, so the matrix-core output
// lanes of different right-hand columns start on different banks; a B-operand
// group (16 key channels, 64 lanes x 16 bytes) is 260 floats, and lane l's 16
// bytes sit in slot l ^ 2 (l / 16), so the writes of the 64 channels of a wave
// (which differ in group and in l / 16) spread over all banks while every
// matrix-core read is still one whole contiguous group.
template <int DK, int DV, bool VEC>
struct VerifyLds {
    static constexpr int KS = DK + 16;   // staged draft row
    static constexpr int RS = DV + 4;    // r0 / p0 row
    static constexpr int XG = 64 * 4 + 4;  // B-operand group of 16 key channels
    // float offsets into the dynamic LDS block for K drafts.  r0 / p0 (phases
    // 3-4) reuse the staging area of k, q and the decay (phases 1-2).
    int k, q, a, r0, p0, v, b, xb, pg, pe;
    int total;  // floats
    __host__ __device__ VerifyLds(int K)
    {
        k = 0;
        q = k + K * KS;
        a = q + K * KS;
        const int staged = a + (VEC ? K * KS : 16);
        r0 = 0;
        p0 = K * RS;
        v = staged > 2 * K * RS ? staged : 2 * K * RS;
        b = v + K * DV;
        xb = b + 16;                                  // 16-byte aligned
        pg = xb + verify_nb(K) * (DK / 16) * XG;
        pe = pg + K * K * kPairChunks;
        total = pe + K * K * kPairChunks;
    }
};

// B-operand slot of matrix-core lane l (see VerifyLds)
__device__ __forceinline__ int xb_slot(int l) { return l ^ ((l >> 4) << 1); }

template <int DK, int DV, typename TIn, typename TOut, bool VEC, int NB>
__global__ void __launch_bounds__(2 * DV) __attribute__((amdgpu_waves_per_eu(5)))
k_verify(const float *__restrict__ state, int n_slots, const int32_t *__restrict__ slot, int H,
         int K, const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
         const float *__restrict__ alpha, const float *__restrict__ beta, TOut *__restrict__ out,
         int32_t *__restrict__ err)
{
    constexpr int NT = 2 * DV, NS = DK / 4, CH = DK / kPairChunks, KP = 8 * NB;
    constexpr int KS = VerifyLds<DK, DV, VEC>::KS, RS = VerifyLds<DK, DV, VEC>::RS;
    constexpr int XG = VerifyLds<DK, DV, VEC>::XG;
    extern __shared__ f32x4 verify_lds[];
    float *L = reinterpret_cast<float *>(verify_lds);
    const VerifyLds<DK, DV, VEC> at(K);
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int s = slot ? slot[b] : b;
    if (s < 0) return;  // uniform over the workgroup
    if (s >= n_slots) {
        if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const size_t tok0 = (size_t)b * K * H + h;  // draft t is token tok0 + t * H
    const int tid = threadIdx.x;

    // 1. stage the drafts' k, q, decay, v and beta (every load issued before the
    //    first LDS write)
    constexpr int JK = KP * DK / NT, JV = KP * DV / NT;  // KP >= K drafts staged
    float rk[JK], rq_[JK], ra[JK], rv[JV];
#pragma unroll
    for (int j = 0; j < JK; ++j) {
        const int e = tid + j * NT, t = e / DK, i = e - t * DK;
        rk[j] = rq_[j] = ra[j] = 0.0f;
        if (t < K) {
            const size_t g = (tok0 + (size_t)t * H) * DK + i;
            rk[j] = load_one(k + g);
            rq_[j] = load_one(q + g);
            if (VEC) ra[j] = alpha[g];
        }
    }
#pragma unroll
    for (int j = 0; j < JV; ++j) {
        const int e = tid + j * NT, t = e / DV, i = e - t * DV;
        rv[j] = t < K ? load_one(v + (tok0 + (size_t)t * H) * DV + i) : 0.0f;
    }
    const float rb = tid < K ? beta[tok0 + (size_t)tid * H] : 0.0f;
    const float rs = !VEC && tid < K ? alpha[tok0 + (size_t)tid * H] : 0.0f;
    // the tile (read only) in the matrix-core layout: the first half is issued
    // right behind the staged inputs, the second once the pair sums are done
    const int lane = tid & 63, wave = tid >> 6;
    const int cm = lane & 15, rq = lane >> 4;
    const float *S = state + ((size_t)s * H + h) * (DK * DV) + (size_t)rq * DV + wave * 32 + 2 * cm;
    constexpr int NS1 = NS / 2;
    float x[NS][2];
#pragma unroll
    for (int m = 0; m < NS1; ++m) {
        const u32x2 t2 = ld_nt(reinterpret_cast<const u32x2 *>(S + (size_t)(4 * m) * DV));
        x[m][0] = __uint_as_float(t2.x);
        x[m][1] = __uint_as_float(t2.y);
    }
#pragma unroll
    for (int j = 0; j < JK; ++j) {
        const int e = tid + j * NT, t = e / DK, i = e - t * DK;
        if (t < K) {
            L[at.k + t * KS + i] = rk[j];
            L[at.q + t * KS + i] = rq_[j];
            if (VEC) L[at.a + t * KS + i] = ra[j];
        }
    }
#pragma unroll
    for (int j = 0; j < JV; ++j) {
        const int e = tid + j * NT;
        if (e < K * DV) L[at.v + e] = rv[j];
    }
    if (tid < K) {
        L[at.b + tid] = rb;
        if (!VEC) L[at.a + tid] = rs;
    }
    __syncthreads();
    // c_t k_t and c_t q_t of key channel i into the B-operand layout: right-hand
    // column g of row i is lane l = 16 (i % 4) + g % 16 of group (g / 16, i / 16),
    // component (i / 4) % 4, stored in slot xb_slot(l)
    for (int i = tid; i < DK; i += NT) {
        float c = 1.0f;
        const int grp = i >> 4, kk = i & 3, comp = (i >> 2) & 3;
        for (int t = 0; t < KP; ++t) {
            float xk = 0.0f, xq = 0.0f;
            if (t < K) {
                c *= VEC ? L[at.a + t * KS + i] : L[at.a + t];
                xk = c * L[at.k + t * KS + i];
                xq = c * L[at.q + t * KS + i];
            }
            const int gk = t, gq = KP + t;
            L[at.xb + ((gk >> 4) * (DK / 16) + grp) * XG + 4 * xb_slot(16 * kk + (gk & 15)) + comp] = xk;
            L[at.xb + ((gq >> 4) * (DK / 16) + grp) * XG + 4 * xb_slot(16 * kk + (gq & 15)) + comp] = xq;
        }
    }

    // 2. the pair sums while the tile arrives
    // (chunk ch takes key channels ch, ch + 16, ch + 32, ...: the 16 lanes of one
    // draft read 16 consecutive floats)
    for (int it = tid; it < K * kPairChunks; it += NT) {
        const int s0 = it / kPairChunks, ch = it - s0 * kPairChunks;
        float ks[CH], w[CH];
        float e_ss = 0.0f;
#pragma unroll
        for (int m = 0; m < CH; ++m) {
            ks[m] = L[at.k + s0 * KS + ch + kPairChunks * m];
            w[m] = 1.0f;
            e_ss = fmaf(ks[m], L[at.q + s0 * KS + ch + kPairChunks * m], e_ss);
        }
        L[at.pe + (s0 * K + s0) * kPairChunks + ch] = e_ss;
        // t runs to the compile-time KP (skipping t <= s0 and t >= K) so that the
        // LDS reads of later drafts can issue ahead of the w products' chain
#pragma unroll
        for (int t = 1; t < KP; ++t) {
            if (t <= s0 || t >= K) continue;
            float g = 0.0f, e2 = 0.0f;
#pragma unroll
            for (int m = 0; m < CH; ++m) {
                const int i = ch + kPairChunks * m;
                w[m] *= VEC ? L[at.a + t * KS + i] : L[at.a + t];
                const float kw = ks[m] * w[m];
                g = fmaf(kw, L[at.k + t * KS + i], g);
                e2 = fmaf(kw, L[at.q + t * KS + i], e2);
            }
            L[at.pg + (s0 * K + t) * kPairChunks + ch] = g;
            L[at.pe + (s0 * K + t) * kPairChunks + ch] = e2;
        }
    }
    // second half of the tile
#pragma unroll
    for (int m = NS1; m < NS; ++m) {
        const u32x2 t2 = ld_nt(reinterpret_cast<const u32x2 *>(S + (size_t)(4 * m) * DV));
        x[m][0] = __uint_as_float(t2.x);
        x[m][1] = __uint_as_float(t2.y);
    }
    __syncthreads();  // the B operand and the pair partials are complete; k, q, decay are dead

    // 3. S_0^T [c k | c q] on the matrix cores, then to LDS (r0 / p0 replace k / q)
    const f32x4 *XB = reinterpret_cast<const f32x4 *>(L + at.xb);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g4 = 0; g4 < DK / 16; ++g4) {
            const f32x4 bq = XB[(nb * (DK / 16) + g4) * (XG / 4) + xb_slot(lane)];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(x[4 * g4 + j][0], bq[j], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(x[4 * g4 + j][1], bq[j], acc1, 0, 0, 0);
            }
        }
        const int g = 16 * nb + cm, typ = g >= KP, t = g - typ * KP;
        if (t < K) {
            float *dst = L + (typ ? at.p0 : at.r0) + t * RS + wave * 32 + 8 * rq;
            reinterpret_cast<f32x4 *>(dst)[0] = f32x4{acc0[0], acc1[0], acc0[1], acc1[1]};
            reinterpret_cast<f32x4 *>(dst)[1] = f32x4{acc0[2], acc1[2], acc0[3], acc1[3]};
        }
    }
    // pair sums: chunk partials -> G_st, E_st (kept in chunk 0's slot)
    for (int it = tid; it < K * K; it += NT) {
        const int s0 = it / K, t = it - s0 * K;
        if (t < s0) continue;
        float g = 0.0f, e2 = 0.0f;
        for (int ch = 0; ch < kPairChunks; ++ch) {
            if (t > s0) g += L[at.pg + it * kPairChunks + ch];
            e2 += L[at.pe + it * kPairChunks + ch];
        }
        L[at.pg + it * kPairChunks] = g;
        L[at.pe + it * kPairChunks] = e2;
    }
    __syncthreads();

    // 4. one thread per column: the drafts in order.  The loops run to the
    //    compile-time KP (drafts t >= K skipped) so that every LDS read, none of
    //    which depends on u, can be issued ahead of the FMA chain.
    if (tid < DV) {
        float r[KP], o[KP], vv[KP], u[KP];
#pragma unroll
        for (int t = 0; t < KP; ++t) {
            r[t] = o[t] = vv[t] = u[t] = 0.0f;
            if (t < K) {
                r[t] = L[at.r0 + t * RS + tid];
                o[t] = L[at.p0 + t * RS + tid];
                vv[t] = L[at.v + t * DV + tid];
            }
        }
#pragma unroll
        for (int t = 0; t < KP; ++t) {
            if (t < K) {
                float rt = r[t], ot = o[t];
#pragma unroll
                for (int s1 = 0; s1 < t; ++s1) {
                    rt = fmaf(L[at.pg + (s1 * K + t) * kPairChunks], u[s1], rt);
                    ot = fmaf(L[at.pe + (s1 * K + t) * kPairChunks], u[s1], ot);
                }
                u[t] = L[at.b + t] * (vv[t] - rt);  // u = beta (v - r)
                ot = fmaf(L[at.pe + (t * K + t) * kPairChunks], u[t], ot);
                store_one(out + (tok0 + (size_t)t * H) * DV + tid, ot);
            }
        }
    }
}

// ----------------------------------------------------------------- dispatch

template <int DK, int DV, typename TIn, typename TOut, bool VEC>
static int launch_verify(const StepArgs &a, int32_t *err, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)a.B * a.H)), block(2 * DV);
    const size_t lds = (size_t)VerifyLds<DK, DV, VEC>(a.K).total * sizeof(float);
    if (verify_nb(a.K) == 1)
        hipLaunchKernelGGL((k_verify<DK, DV, TIn, TOut, VEC, 1>), grid, block, lds, st, a.state,
                           a.n_slots, a.slot, a.H, a.K, (const TIn *)a.q, (const TIn *)a.k,
                           (const TIn *)a.v, a.alpha, a.beta, (TOut *)a.out, err);
    else
        hipLaunchKernelGGL((k_verify<DK, DV, TIn, TOut, VEC, 2>), grid, block, lds, st, a.state,
                           a.n_slots, a.slot, a.H, a.K, (const TIn *)a.q, (const TIn *)a.k,
                           (const TIn *)a.v, a.alpha, a.beta, (TOut *)a.out, err);
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

template <int DK, int DV>
static int verify_dtypes(const StepArgs &a, int32_t *err, hipStream_t st)
{
    const bool vec = a.decay == HLA_DECAY_VECTOR;
#define HLA_VERIFY_T(TI_, TO_)                                                                \
    return vec ? launch_verify<DK, DV, TI_, TO_, true>(a, err, st)                            \
               : launch_verify<DK, DV, TI_, TO_, false>(a, err, st);
#define HLA_VERIFY_OUT(TI_)                                                                   \
    if (a.out_dtype == HLA_BF16) { HLA_VERIFY_T(TI_, uint16_t) }                              \
    if (a.out_dtype == HLA_F16) { HLA_VERIFY_T(TI_, f16_t) }                                  \
    HLA_VERIFY_T(TI_, float)
    if (a.in_dtype == HLA_BF16) { HLA_VERIFY_OUT(uint16_t) }
    if (a.in_dtype == HLA_F16) { HLA_VERIFY_OUT(f16_t) }
    HLA_VERIFY_OUT(float)
#undef HLA_VERIFY_OUT
#undef HLA_VERIFY_T
}

int run_verify(const StepArgs &a, int32_t *err, void *stream)
{
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.dk == 128 && a.dv == 128) return verify_dtypes<128, 128>(a, err, st);
    if (a.dk == 128 && a.dv == 64) return verify_dtypes<128, 64>(a, err, st);
    if (a.dk == 64 && a.dv == 128) return verify_dtypes<64, 128>(a, err, st);
    return verify_dtypes<64, 64>(a, err, st);
}

} // namespace hla

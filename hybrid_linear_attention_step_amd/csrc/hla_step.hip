// gfx950 kernels for the FP32 gated delta-rule step (GDN scalar decay, KDA
// per-key-channel decay) and for several tokens per launch: the replay of
// accepted draft tokens (optionally followed by the bonus token, or preceded by
// the restore of a checkpoint into the state).  The verify pass over all drafts
// has its own kernel (hla_verify.hip).
//
// Operation ("DAMP: Decay-Aware Mixed-Precision Recurrent-State
// Quantization", §3.1 Eq. (1)-(2)), per (request, head), state S in dk x dv:
//     S' = Lambda S,  u = beta (v - S'^T k),  S = S' + k u^T,  o = S^T q.
//
// Work decomposition.  Every column j of the state is independent: r_j =
// (S'^T k)_j and the readout o_j = (S^T q)_j are sums over rows (key
// channels) of column j only.  So one wave64 owns a dk x 32 column slice of
// one head and needs nothing from any other wave:
//   lane = 8 * rg + cg;  cg in 0..7 picks 4 adjacent columns (one 16-byte
//   float4), rg in 0..7 picks a block of dk/8 consecutive rows.
// Each 16-byte load/store instruction of the wave covers 8 rows x 128
// contiguous bytes, so every HBM access is a full 128-byte line.  The tile
// (dk/8 x 4 floats per lane, 64 for dk = 128) stays in registers from the
// load to the store: the state is read once and written once per step.
// Column sums over the 8 row blocks use DPP row_ror:8 and the gfx950
// v_permlane16_swap / v_permlane32_swap (lane bits 3, 4, 5) - no LDS.
// The readout is formed in the same pass: o = S'^T q + (q.k) u, which equals
// S^T q for S = S' + k u^T.
// A workgroup is the dv/32 waves of one head; they share only the small
// q/k/alpha rows, which hit in the CU's caches.
#include <hip/hip_runtime.h>

#include "hla.h"
#include "hla_device.h"
#include "hla_internal.h"

namespace hla {

// The tile is read through a buffer resource over the head (scalar registers:
// base, size) with one 32-bit per-lane byte offset and the row offset in the
// scalar offset operand, so no 64-bit per-lane pointer is kept live across
// the token (registers are what limits waves per SIMD here).  Every read is
// inside the head by construction: the lane offset (row0*dv + col0)*4 plus
// the row offset m*dv*4 plus 16 bytes is at most dk*dv*4.  (The descriptor's
// size is not a guard here: the scalar offset is not part of the hardware
// range check.)  Word 3 of the descriptor is the raw-buffer format used on
// gfx9-family GPUs; cache policy: nontemporal.
// The tile is written back with ordinary global nontemporal stores, whose
// addresses are formed only after the token's arithmetic.  Not the buffer
// form of the store: with the row offset in a scalar register the compiler
// lets the next VALU instruction overwrite the store's 16-byte data registers
// with no wait state (it inserts one for a constant scalar offset and for
// global stores), and that variant wrote wrong values in lanes 12-15 of each
// 16-lane group of some waves, the pattern of a store reading its data after
// it was overwritten.
constexpr int kBufNt = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const float *head, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(head), (short)0, bytes,
                                             0x00020000);
}

template <int RPL>
__device__ __forceinline__ void tile_load(__amdgpu_buffer_rsrc_t rsrc, uint32_t off_bytes, int DV,
                                          float (&x)[RPL][4])
{
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off_bytes, m * DV * 4, kBufNt);
        x[m][0] = __uint_as_float(t[0]); x[m][1] = __uint_as_float(t[1]);
        x[m][2] = __uint_as_float(t[2]); x[m][3] = __uint_as_float(t[3]);
    }
}

template <int RPL>
__device__ __forceinline__ void tile_store(float *head, uint32_t off_bytes, int DV,
                                           const float (&x)[RPL][4])
{
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        f32x4 t = {x[m][0], x[m][1], x[m][2], x[m][3]};
        st_nt(reinterpret_cast<f32x4 *>(head + (size_t)m * DV + off_bytes / 4), t);
    }
}

// One token's per-lane inputs as loaded (raw 16-byte words): rows
// [row0, row0+RPL) of q, k and of a vector decay, the lane's 4 columns of v,
// the scalar decay and beta.  Values are unpacked where they are used, after
// the state loads have been issued.
template <int DK, typename TIn, bool VEC>
struct TokenRaw {
    static constexpr int RPL = DK / 8;
    static constexpr int QW = RPL * (int)sizeof(TIn) / 16;  // 16-byte words per row block
    u32x4 k[QW], q[QW];
    u32x4 a[VEC ? RPL / 4 : 1];
    u32x2 v2;  // 2-byte v (bf16 or binary16)
    u32x4 v4;  // fp32 v
    float a0, b0;
};

// RD: the token's readout is wanted (q is read only then).
template <int DK, int DV, typename TIn, bool VEC, bool RD = true>
__device__ __forceinline__ void token_load(const TIn *q, const TIn *k, const TIn *v,
                                           const float *alpha, const float *beta, size_t tok,
                                           int row0, int col0, TokenRaw<DK, TIn, VEC> &R)
{
    using TR = TokenRaw<DK, TIn, VEC>;
    const u32x4 *kp = reinterpret_cast<const u32x4 *>(k + tok * DK + row0);
    const u32x4 *qp = reinterpret_cast<const u32x4 *>(q + tok * DK + row0);
#pragma unroll
    for (int i = 0; i < TR::QW; ++i) {
        R.k[i] = kp[i];
        if constexpr (RD) R.q[i] = qp[i];
    }
    if constexpr (VEC) {
        const u32x4 *ap = reinterpret_cast<const u32x4 *>(alpha + tok * DK + row0);
#pragma unroll
        for (int i = 0; i < TR::RPL / 4; ++i) R.a[i] = ap[i];
    } else {
        R.a0 = alpha[tok];
    }
    if constexpr (sizeof(TIn) == 2)
        R.v2 = *reinterpret_cast<const u32x2 *>(v + tok * DV + col0);
    else
        R.v4 = *reinterpret_cast<const u32x4 *>(v + tok * DV + col0);
    R.b0 = beta[tok];
}

// The lane's 4 columns of v as floats.
template <typename TIn>
__device__ __forceinline__ void token_v(const u32x2 &v2, const u32x4 &v4, float (&vv)[4])
{
    if constexpr (sizeof(TIn) == 2) {
        vv[0] = lo16<TIn>(v2.x); vv[1] = hi16<TIn>(v2.x);
        vv[2] = lo16<TIn>(v2.y); vv[3] = hi16<TIn>(v2.y);
    } else {
        vv[0] = __uint_as_float(v4.x); vv[1] = __uint_as_float(v4.y);
        vv[2] = __uint_as_float(v4.z); vv[3] = __uint_as_float(v4.w);
    }
}

// Row m of the lane's k or q block as loaded (the 16-byte words of
// TokenRaw), converted at the point of use: a pair of 2-byte inputs shares one
// register until it is needed, which keeps the step's register count low
// enough for five waves per SIMD with bf16 (or binary16) inputs.
template <typename TIn, int QW>
__device__ __forceinline__ float raw_row(const u32x4 (&w)[QW], int m)
{
    if constexpr (sizeof(TIn) == 2) {
        const u32x4 &t = w[m / 8];
        const int c = (m % 8) / 2;
        const uint32_t word = c == 0 ? t.x : c == 1 ? t.y : c == 2 ? t.z : t.w;
        return (m & 1) ? hi16<TIn>(word) : lo16<TIn>(word);
    } else {
        const u32x4 &t = w[m / 4];
        const int c = m % 4;
        return __uint_as_float(c == 0 ? t.x : c == 1 ? t.y : c == 2 ? t.z : t.w);
    }
}

// One token's update of a lane's tile.  x[m][c] is row (rg*RPL + m), column
// (slice + 4*cg + c); k, q and a per-channel decay are read from the token's
// raw words row by row.  Returns the readout for the lane's 4 columns (valid
// in every lane) when RD; without it the readout's terms are not formed at all
// (a third of the token's arithmetic), and the state is the same bits.  Shared
// by the step and the replay kernels so that a replay is bitwise identical to
// the same number of single steps.
template <int DK, typename TIn, bool VEC, bool RD = true>
__device__ __forceinline__ void tile_token_raw(float (&x)[DK / 8][4],
                                               const TokenRaw<DK, TIn, VEC> &R,
                                               const float (&vv)[4], float beta, float (&o)[4])
{
    constexpr int RPL = DK / 8, QW = TokenRaw<DK, TIn, VEC>::QW;
    float r[4] = {0.f, 0.f, 0.f, 0.f};
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        float a = R.a0;
        if constexpr (VEC) a = raw_row<float, RPL / 4>(R.a, m);
        const float km = raw_row<TIn, QW>(R.k, m);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            x[m][c] = x[m][c] * a;             // S' = Lambda S
            r[c] = fmaf(km, x[m][c], r[c]);    // partial (S'^T k)_j
        }
        if constexpr (RD) {
            const float qm = raw_row<TIn, QW>(R.q, m);
#pragma unroll
            for (int c = 0; c < 4; ++c) p[c] = fmaf(qm, x[m][c], p[c]);  // partial (S'^T q)_j
            qk = fmaf(qm, km, qk);
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        r[c] = sum_lane_bits<3>(r[c]);
        if constexpr (RD) p[c] = sum_lane_bits<3>(p[c]);
    }
    if constexpr (RD) qk = sum_lane_bits<3>(qk);
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        u[c] = beta * (vv[c] - r[c]);   // u = beta (v - S'^T k)
        o[c] = RD ? fmaf(qk, u[c], p[c]) : 0.0f;  // o = S'^T q + (q.k) u = S^T q
    }
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        const float km = raw_row<TIn, QW>(R.k, m);
#pragma unroll
        for (int c = 0; c < 4; ++c) x[m][c] = fmaf(km, u[c], x[m][c]);  // S = S' + k u^T
    }
}

// Waves per SIMD the step is compiled for: with bf16 inputs and a scalar
// decay the tile, the raw k / q words and the rest fit 96 VGPRs, i.e. five
// waves per SIMD instead of four (measured faster); otherwise the compiler's
// default (four at 128 x 128).
template <int DK, typename TIn, bool VEC>
struct StepWaves {
    static constexpr int v = (DK == 128 && sizeof(TIn) == 2) ? 5 : 1;
};

template <int DK, int DV, typename TIn, typename TOut, bool VEC>
__global__ void __launch_bounds__(2 * DV)
__attribute__((amdgpu_waves_per_eu(StepWaves<DK, TIn, VEC>::v)))
k_delta_step(float *__restrict__ state, int n_slots, const int32_t *__restrict__ slot, int H,
             const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
             const float *__restrict__ alpha, const float *__restrict__ beta,
             TOut *__restrict__ out, int32_t *__restrict__ err)
{
    constexpr int RPL = DK / 8;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int s = slot ? slot[b] : b;
    if (s < 0) return;  // padding request
    if (s >= n_slots) {
        if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x) >> 6;  // uniform
    const int cg = lane & 7, rg = lane >> 3;
    const int col0 = wave * 32 + cg * 4, row0 = rg * RPL;
    float *head_ptr = state + ((size_t)s * H + h) * (DK * DV);
    const __amdgpu_buffer_rsrc_t head = head_rsrc(head_ptr, DK * DV * 4);
    const uint32_t off = (uint32_t)(row0 * DV + col0) * 4;

    TokenRaw<DK, TIn, VEC> raw;
    token_load<DK, DV, TIn, VEC>(q, k, v, alpha, beta, (size_t)bh, row0, col0, raw);
    float x[RPL][4];
    tile_load<RPL>(head, off, DV, x);
    float vv[4];
    token_v<TIn>(raw.v2, raw.v4, vv);
    float o[4];
    tile_token_raw<DK, TIn, VEC>(x, raw, vv, raw.b0, o);
    tile_store<RPL>(head_ptr, off, DV, x);
    if (out) {
        // the lane index again from the hardware counter rather than kept in a
        // register through the token (registers decide the waves per SIMD)
        const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        if ((ln >> 3) == 0) store_out4(out + (size_t)bh * DV + wave * 32 + (ln & 7) * 4, o);
    }
}

// Draft-token inputs staged in LDS.  A workgroup that replays n_b tokens copies all of
// their inputs into LDS at once, with the direct global-to-LDS load (global_load_lds,
// 16 bytes per lane; a wave's 64 lanes fill 1 KiB of LDS in lane order), issued together
// with the state tile's loads; the token loop then reads each token from LDS.  So the
// tokens cost one memory round trip per workgroup instead of one each, which matters
// most for a head that starts from zero (no state read to hide the token loads behind).
// Token t takes WG consecutive 16-byte words: q (only when readouts are wanted), k, v and
// (per-channel decay) alpha, as stored; the scalar decay and beta sit in one float2 per
// token after the K tokens.
// The staging costs a workgroup barrier, which ties the head's waves together (each
// otherwise streams its column slice on its own): with a state read to hide the token
// loads behind, it pays from about 7 accepted tokens on (measured over 1-8), so fewer
// are loaded token by token as in the step.
constexpr int kStageMinTokens = 7;

template <int DK, int DV, typename TIn, bool VEC, bool RD>
struct TokenLds {
    static constexpr int QB = DK * (int)sizeof(TIn) / 16;  // words of k (and of q)
    static constexpr int Q0 = RD ? QB : 0;                 // words of q staged
    static constexpr int VB = DV * (int)sizeof(TIn) / 16;  // words of v
    static constexpr int AB = VEC ? DK * 4 / 16 : 0;        // words of a vector decay
    static constexpr int WG = Q0 + QB + VB + AB;           // words per token
    static size_t bytes(int K) { return (size_t)K * (WG * 16 + sizeof(float2)); }
};

// An LDS address as the direct global-to-LDS load takes it.
typedef __attribute__((address_space(3))) void lds_void_t;

// Issue the staging copies of tokens [0, nb) of workgroup (ln, h); every wave of the
// workgroup takes 64 words per pass.  The LDS address of a wave's copy is wave-uniform.
template <int DK, int DV, typename TIn, bool VEC, bool RD>
__device__ __forceinline__ void stage_tokens(uint8_t *lds, int nb, size_t tok0, int H,
                                             const TIn *q, const TIn *k, const TIn *v,
                                             const float *alpha, const float *beta, int K)
{
    using T = TokenLds<DK, DV, TIn, VEC, RD>;
    constexpr int NW = 2 * DV / 64;  // waves per workgroup
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int total = nb * T::WG;
    for (int w0 = wave * 64; w0 < total; w0 += NW * 64) {
        const int f = w0 + lane;
        if (f < total) {
            const int t = f / T::WG, i = f - t * T::WG;
            const size_t tok = tok0 + (size_t)t * H;
            const uint8_t *src;
            if (i < T::Q0)
                src = reinterpret_cast<const uint8_t *>(q + tok * DK) + i * 16;
            else if (i < T::Q0 + T::QB)
                src = reinterpret_cast<const uint8_t *>(k + tok * DK) + (i - T::Q0) * 16;
            else if (i < T::Q0 + T::QB + T::VB)
                src = reinterpret_cast<const uint8_t *>(v + tok * DV) + (i - T::Q0 - T::QB) * 16;
            else
                src = reinterpret_cast<const uint8_t *>(alpha + tok * DK) +
                      (i - T::Q0 - T::QB - T::VB) * 16;
            __builtin_amdgcn_global_load_lds(src, (lds_void_t *)(lds + (size_t)w0 * 16), 16, 0,
                                             0);
        }
    }
    float2 *ab = reinterpret_cast<float2 *>(lds + (size_t)K * T::WG * 16);
    if ((int)threadIdx.x < nb) {
        const size_t tok = tok0 + (size_t)threadIdx.x * H;
        ab[threadIdx.x] = make_float2(VEC ? 0.0f : alpha[tok], beta[tok]);
    }
}

// Token t's per-lane inputs from LDS, in the layout token_load gives.
template <int DK, int DV, typename TIn, bool VEC, bool RD>
__device__ __forceinline__ void token_from_lds(const uint8_t *lds, int t, int K, int row0,
                                               int col0, TokenRaw<DK, TIn, VEC> &R)
{
    using T = TokenLds<DK, DV, TIn, VEC, RD>;
    using TR = TokenRaw<DK, TIn, VEC>;
    constexpr int K0 = T::Q0, V0 = T::Q0 + T::QB, A0 = V0 + T::VB;  // first words of k, v, a
    const u32x4 *w = reinterpret_cast<const u32x4 *>(lds) + (size_t)t * T::WG;
    const int r = row0 * (int)sizeof(TIn) / 16;
#pragma unroll
    for (int i = 0; i < TR::QW; ++i) {
        if constexpr (RD) R.q[i] = w[r + i];
        R.k[i] = w[K0 + r + i];
    }
    if constexpr (VEC) {
#pragma unroll
        for (int i = 0; i < TR::RPL / 4; ++i) R.a[i] = w[A0 + row0 / 4 + i];
    }
    if constexpr (sizeof(TIn) == 2)
        R.v2 = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint8_t *>(w + V0) +
                                                col0 * 2);
    else
        R.v4 = w[V0 + col0 / 4];
    const float2 ab = reinterpret_cast<const float2 *>(lds + (size_t)K * T::WG * 16)[t];
    R.a0 = ab.x;
    R.b0 = ab.y;
}

// Several tokens per (request, head) with the tile held in registers
// throughout ("Serving recurrent attention", part "Speculative decoding
// without state snapshots"):
//   MODE_REPLAY  the first n_b of K cached draft projections (inputs staged
//                in LDS from kStageMinTokens tokens on); the state is read once
//                and written once, and not touched when n_b = 0;
//   MODE_BONUS   the same, then the target model's bonus token ([B, H, .]
//                inputs, applied also when n_b = 0), then one write.
template <int DK, int DV, typename TIn, typename TOut, bool VEC, int MODE, bool RD>
__global__ void __launch_bounds__(2 * DV)
k_tokens(float *__restrict__ state, int n_slots, const int32_t *__restrict__ slot, int H, int K,
         const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
         const float *__restrict__ alpha, const float *__restrict__ beta,
         const int32_t *__restrict__ n_accept, TOut *__restrict__ out,
         const TIn *__restrict__ qb, const TIn *__restrict__ kb, const TIn *__restrict__ vb,
         const float *__restrict__ alpha_b, const float *__restrict__ beta_b,
         TOut *__restrict__ out_b, int32_t *__restrict__ err)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t tok_lds[];
    constexpr int RPL = DK / 8;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int s = slot ? slot[b] : b;
    if (s < 0) return;
    if (s >= n_slots) {
        if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    int n = n_accept[b];
    if (n < 0 || n > K) {
        if (err && threadIdx.x == 0 && h == 0) atomicOr(err, HLA_DEVERR_ACCEPT);
        n = n < 0 ? 0 : K;
    }
    if (MODE == MODE_REPLAY && n == 0) return;  // nothing accepted: the state is not touched
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 7, rg = lane >> 3;
    const int col0 = wave * 32 + cg * 4, row0 = rg * RPL;
    float *head_ptr = state + ((size_t)s * H + h) * (DK * DV);
    const __amdgpu_buffer_rsrc_t head = head_rsrc(head_ptr, DK * DV * 4);
    const uint32_t off = (uint32_t)(row0 * DV + col0) * 4;

    float x[RPL][4];
    tile_load<RPL>(head, off, DV, x);
    const size_t tok0 = (size_t)b * K * H + h;  // token t of (b, h) is tok0 + t * H
    const bool staged = n >= kStageMinTokens;  // uniform over the workgroup
    if (staged) {
        stage_tokens<DK, DV, TIn, VEC, RD>(tok_lds, n, tok0, H, q, k, v, alpha, beta, K);
        __builtin_amdgcn_s_waitcnt(0);  // the copies into LDS (and the tile) have landed
        __syncthreads();
    }
    for (int t = 0; t < n; ++t) {
        TokenRaw<DK, TIn, VEC> raw;
        if (staged)
            token_from_lds<DK, DV, TIn, VEC, RD>(tok_lds, t, K, row0, col0, raw);
        else
            token_load<DK, DV, TIn, VEC, RD>(q, k, v, alpha, beta, tok0 + (size_t)t * H, row0,
                                             col0, raw);
        float vv[4];
        token_v<TIn>(raw.v2, raw.v4, vv);
        float o[4];
        tile_token_raw<DK, TIn, VEC, RD>(x, raw, vv, raw.b0, o);
        if (RD && out && rg == 0) store_out4(out + (tok0 + (size_t)t * H) * DV + col0, o);
    }
    if constexpr (MODE == MODE_BONUS) {
        TokenRaw<DK, TIn, VEC> raw;
        token_load<DK, DV, TIn, VEC>(qb, kb, vb, alpha_b, beta_b, (size_t)bh, row0, col0, raw);
        float vv[4];
        token_v<TIn>(raw.v2, raw.v4, vv);
        float o[4];
        tile_token_raw<DK, TIn, VEC>(x, raw, vv, raw.b0, o);
        if (out_b && rg == 0) store_out4(out_b + (size_t)bh * DV + col0, o);
    }
    tile_store<RPL>(head_ptr, off, DV, x);
}

// A checkpoint restored into private slots with each request's accepted drafts replayed
// on the way ("dasc: Decay-Aware State Compression for Hybrid Linear-Attention Serving",
// §4.2 dasc-nr; "Serving recurrent attention", part "Speculative decoding without state
// snapshots").  Workgroup (l, n, h): each unit of the head (HU: the whole head, one
// buffer descriptor; otherwise 2^log2_ur rows, each lane looking up the unit of each of
// its rows) starts as its packed copy from checkpoint slot src_slot[n], or as zero when
// it is not retained; the head takes the first n_b draft tokens of layer l in registers
// and is written once into private slot dst_slot[n].  The tokens' inputs are staged in
// LDS for every head with n_b > 0: many heads start from zero, with no state read to hide
// token loads behind, and over the whole workload staging all of them measured fastest.
// Same lane layout and per-token function as the step, so the result is bitwise that of
// dasc_restore (Q8: dasc_restore_int8, each retained row code x scale in FP32) followed
// by replay_accepted.  RD: readouts are written (otherwise their terms are not formed).
// With n_accept NULL it is the restore alone (restore_int8_by_blocks).
template <int DK, int DV, typename TIn, typename TOut, bool VEC, bool HU, bool Q8, bool RD>
__global__ void __launch_bounds__(2 * DV)
k_restore_tokens(const void *__restrict__ packed, const float *__restrict__ scales, int S_ckpt,
                 int R_total, const int32_t *__restrict__ unit_pos, int log2_ur, int N,
                 const int32_t *__restrict__ src_slot, const int32_t *__restrict__ dst_slot,
                 float *__restrict__ active_out, int64_t layer_stride_floats, int S_dst, int H,
                 int K, const TIn *__restrict__ q, const TIn *__restrict__ k,
                 const TIn *__restrict__ v, const float *__restrict__ alpha,
                 const float *__restrict__ beta, const int32_t *__restrict__ n_accept,
                 TOut *__restrict__ out, int32_t *__restrict__ err)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t tok_lds[];
    constexpr int RPL = DK / 8;
    const int g = blockIdx.x;  // (l * N + n) * H + h
    const int ln = g / H, h = g - ln * H;
    const int l = ln / N, n = ln - l * N;
    const int src = src_slot[n], dst = dst_slot[n];
    if (src < 0 || src >= S_ckpt || dst < 0 || dst >= S_dst) {
        if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_SLOT);
        return;
    }
    int nb = n_accept ? n_accept[n] : 0;  // no accepted counts: a restore only
    if (nb < 0 || nb > K) {
        if (err && threadIdx.x == 0 && h == 0 && l == 0) atomicOr(err, HLA_DEVERR_ACCEPT);
        nb = nb < 0 ? 0 : K;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cg = lane & 7, rg = lane >> 3;
    const int col0 = wave * 32 + cg * 4, row0 = rg * RPL;
    const uint32_t off = (uint32_t)(row0 * DV + col0) * 4;

    float x[RPL][4];
    if constexpr (HU) {
        int pos = unit_pos[l * H + h];
        if (pos >= R_total) {  // a bad plan entry: the head starts from zero, as restored
            if (err && threadIdx.x == 0) atomicOr(err, HLA_DEVERR_PLAN);
            pos = -1;
        }
        if (pos >= 0 && Q8) {  // codes of the head's rows, then their scales
            const size_t u0 = (size_t)src * R_total + pos;
            const int8_t *cb = static_cast<const int8_t *>(packed) + u0 * (DK * DV) + col0;
            // cached loads: a row's 128 code bytes are read 32 at a time by the head's four
            // waves, which must find the line in L2 (nontemporal loads fetched it 4 times)
            uint32_t w[RPL];
#pragma unroll
            for (int m = 0; m < RPL; ++m)
                w[m] = *reinterpret_cast<const uint32_t *>(cb + (size_t)(row0 + m) * DV);
            float sc[RPL];
#pragma unroll
            for (int i = 0; i < RPL / 4; ++i) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(scales + u0 * DK + row0 + 4 * i);
                sc[4 * i] = t.x; sc[4 * i + 1] = t.y; sc[4 * i + 2] = t.z; sc[4 * i + 3] = t.w;
            }
#pragma unroll
            for (int m = 0; m < RPL; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    x[m][c] = (float)(int)(int8_t)(w[m] >> (8 * c)) * sc[m];  // code * scale
        } else if (pos >= 0) {
            const float *ck =
                static_cast<const float *>(packed) + ((size_t)src * R_total + pos) * (DK * DV);
            tile_load<RPL>(head_rsrc(ck, DK * DV * 4), off, DV, x);
        } else {
#pragma unroll
            for (int m = 0; m < RPL; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) x[m][c] = 0.0f;
        }
    } else {
        // units of 2^log2_ur rows: every lookup first, then every retained row's load
        const int upt = DK >> log2_ur;  // units per head
        const int32_t *up = unit_pos + ((size_t)l * H + h) * upt;
        const uint32_t rmask = (1u << log2_ur) - 1u;
        int pr[RPL];
        if (log2_ur == 0) {  // one unit per row: the lane's RPL entries are contiguous
#pragma unroll
            for (int i = 0; i < RPL / 4; ++i) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(up + row0 + 4 * i);
                pr[4 * i] = (int)w.x; pr[4 * i + 1] = (int)w.y;
                pr[4 * i + 2] = (int)w.z; pr[4 * i + 3] = (int)w.w;
            }
        } else {
#pragma unroll
            for (int m = 0; m < RPL; ++m) pr[m] = up[(row0 + m) >> log2_ur];
        }
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            if (pr[m] >= R_total) {  // a bad plan entry: that unit starts from zero
                if (err) atomicOr(err, HLA_DEVERR_PLAN);
                pr[m] = -1;
            }
        }
        const size_t unit0 = (size_t)src * R_total;  // the source slot's first unit
        if constexpr (Q8) {  // every retained row's codes, then its scale
            uint32_t w[RPL];
            float sc[RPL];
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                w[m] = 0u;
                if (pr[m] >= 0) {
                    const size_t row = ((unit0 + pr[m]) << log2_ur) + ((row0 + m) & rmask);
                    w[m] = *reinterpret_cast<const uint32_t *>(  // cached, as above
                        static_cast<const int8_t *>(packed) + row * DV + col0);
                }
            }
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                sc[m] = 0.0f;
                if (pr[m] >= 0)
                    sc[m] = scales[((unit0 + pr[m]) << log2_ur) + ((row0 + m) & rmask)];
            }
#pragma unroll
            for (int m = 0; m < RPL; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    x[m][c] = (float)(int)(int8_t)(w[m] >> (8 * c)) * sc[m];  // 0 when omitted
        } else {
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
                if (pr[m] >= 0) {
                    const size_t row = ((unit0 + pr[m]) << log2_ur) + ((row0 + m) & rmask);
                    t = ld_nt(reinterpret_cast<const f32x4 *>(
                        static_cast<const float *>(packed) + row * DV + col0));
                }
                x[m][0] = t.x; x[m][1] = t.y; x[m][2] = t.z; x[m][3] = t.w;
            }
        }
    }
    const size_t tok0 = (size_t)ln * K * H + h;  // token t of (l, n, h) is tok0 + t * H
    if (nb > 0) {  // uniform over the workgroup
        stage_tokens<DK, DV, TIn, VEC, RD>(tok_lds, nb, tok0, H, q, k, v, alpha, beta, K);
        __builtin_amdgcn_s_waitcnt(0);  // the copies into LDS (and the tile) have landed
        __syncthreads();
    }
    for (int t = 0; t < nb; ++t) {
        TokenRaw<DK, TIn, VEC> raw;
        token_from_lds<DK, DV, TIn, VEC, RD>(tok_lds, t, K, row0, col0, raw);
        float vv[4];
        token_v<TIn>(raw.v2, raw.v4, vv);
        float o[4];
        tile_token_raw<DK, TIn, VEC, RD>(x, raw, vv, raw.b0, o);
        if (RD && out && rg == 0) store_out4(out + (tok0 + (size_t)t * H) * DV + col0, o);
    }
    float *head_ptr = active_out + l * layer_stride_floats + ((size_t)dst * H + h) * (DK * DV);
    tile_store<RPL>(head_ptr, off, DV, x);
}

// ----------------------------------------------------------------- dispatch

template <int DK, int DV, typename TIn, typename TOut, bool VEC, int MODE, bool RD>
static void launch_tokens_rd(const StepArgs &a, int32_t *err, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)a.B * a.H)), block(2 * DV);
    // no request can reach the staging threshold when K is below it: no LDS then
    const size_t lds = a.K >= kStageMinTokens ? TokenLds<DK, DV, TIn, VEC, RD>::bytes(a.K) : 0;
    hipLaunchKernelGGL((k_tokens<DK, DV, TIn, TOut, VEC, MODE, RD>), grid, block, lds, st,
                       a.state, a.n_slots, a.slot, a.H, a.K, (const TIn *)a.q, (const TIn *)a.k,
                       (const TIn *)a.v, a.alpha, a.beta, a.n_accept, (TOut *)a.out,
                       (const TIn *)a.qb, (const TIn *)a.kb, (const TIn *)a.vb, a.alpha_b,
                       a.beta_b, (TOut *)a.out_b, err);
}

// A replay without readouts (a NULL out) forms no readout terms and reads no q, and
// writes nothing of its output type.  The replay + bonus keeps the drafts' terms either
// way: without them it measured 3% slower (381 against 371 us on the checkpoint
// workload's 512 requests), the bonus token's loads then being exposed later.
template <int DK, int DV, typename TIn, typename TOut, bool VEC, int MODE>
static void launch_tokens(const StepArgs &a, int32_t *err, hipStream_t st)
{
    if constexpr (MODE == MODE_REPLAY) {
        if (!a.out) return launch_tokens_rd<DK, DV, TIn, float, VEC, MODE, false>(a, err, st);
    }
    launch_tokens_rd<DK, DV, TIn, TOut, VEC, MODE, true>(a, err, st);
}

template <int DK, int DV, typename TIn, typename TOut, bool VEC>
static int launch_typed(const StepArgs &a, int32_t *err, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)a.B * a.H)), block(2 * DV);
    switch (a.mode) {
    case MODE_STEP:
        hipLaunchKernelGGL((k_delta_step<DK, DV, TIn, TOut, VEC>), grid, block, 0, st, a.state,
                           a.n_slots, a.slot, a.H, (const TIn *)a.q, (const TIn *)a.k,
                           (const TIn *)a.v, a.alpha, a.beta, (TOut *)a.out, err);
        break;
    case MODE_REPLAY: launch_tokens<DK, DV, TIn, TOut, VEC, MODE_REPLAY>(a, err, st); break;
    case MODE_BONUS: launch_tokens<DK, DV, TIn, TOut, VEC, MODE_BONUS>(a, err, st); break;
    default: break;  // MODE_VERIFY runs in its own translation unit
    }
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

template <int DK, int DV, typename TIn, typename TOut>
static int launch_decay(const StepArgs &a, int32_t *err, hipStream_t st)
{
    return a.decay == HLA_DECAY_VECTOR ? launch_typed<DK, DV, TIn, TOut, true>(a, err, st)
                                       : launch_typed<DK, DV, TIn, TOut, false>(a, err, st);
}

template <int DK, int DV>
static int launch_dtypes(const StepArgs &a, int32_t *err, hipStream_t st)
{
    // element types: float (HLA_F32), uint16_t bf16 bits (HLA_BF16), f16_t (HLA_F16)
#define HLA_STEP_OUT(TI_)                                                                     \
    return a.out_dtype == HLA_BF16  ? launch_decay<DK, DV, TI_, uint16_t>(a, err, st)        \
           : a.out_dtype == HLA_F16 ? launch_decay<DK, DV, TI_, f16_t>(a, err, st)           \
                                    : launch_decay<DK, DV, TI_, float>(a, err, st);
    if (a.in_dtype == HLA_BF16) { HLA_STEP_OUT(uint16_t) }
    if (a.in_dtype == HLA_F16) { HLA_STEP_OUT(f16_t) }
    HLA_STEP_OUT(float)
#undef HLA_STEP_OUT
}

template <int DK, int DV, typename TIn, typename TOut, bool VEC, bool RD>
static void launch_restore_tokens_rd(const RestoreReplayArgs &a, int32_t *err, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)a.L * a.N * a.H)), block(2 * DV);
    const size_t lds = TokenLds<DK, DV, TIn, VEC, RD>::bytes(a.K);
    const int lr = log2_exact(a.unit_rows);
#define HLA_RT_LAUNCH(HU_, Q8_)                                                               \
    hipLaunchKernelGGL((k_restore_tokens<DK, DV, TIn, TOut, VEC, HU_, Q8_, RD>), grid, block,  \
                       lds, st, a.packed, a.scales, a.S_ckpt, a.R_total, a.unit_pos, lr, a.N,   \
                       a.src_slot, a.dst_slot, a.active_out, a.layer_stride_bytes / 4, a.S_dst, \
                       a.H, a.K, (const TIn *)a.q, (const TIn *)a.k, (const TIn *)a.v, a.alpha, \
                       a.beta, a.n_accept, (TOut *)a.out, err)
    const bool hu = a.unit_rows == DK;
    if (a.q8) {
        if (hu) HLA_RT_LAUNCH(true, true);
        else HLA_RT_LAUNCH(false, true);
    } else {
        if (hu) HLA_RT_LAUNCH(true, false);
        else HLA_RT_LAUNCH(false, false);
    }
#undef HLA_RT_LAUNCH
}

// With readouts, or without (a NULL out: their terms are never formed, nothing of the
// output type is written).
template <int DK, int DV, typename TIn, typename TOut, bool VEC>
static void launch_restore_tokens(const RestoreReplayArgs &a, int32_t *err, hipStream_t st)
{
    if (a.out) launch_restore_tokens_rd<DK, DV, TIn, TOut, VEC, true>(a, err, st);
    else launch_restore_tokens_rd<DK, DV, TIn, float, VEC, false>(a, err, st);
}

// The INT8 checkpoint restore through the fused kernel with no tokens: workgroups of 128
// consecutive rows of a slot's layer (H counting such blocks), a lane holding 16 of them.
// Units of 2-8 rows with up to half of them retained restore 5-13% faster this way than
// by the restore kernel (checkpoints read cold); single rows and larger units do not
// gain.  Same decode, so the same bits.  Returns false, with nothing launched, when the
// geometry or the alignment does not fit.
bool restore_int8_by_blocks(const int8_t *codes, const float *scales, int S_ckpt, int R_total,
                            const int32_t *unit_pos, int L, int n_units, int unit_rows, int dv,
                            const int32_t *src_slot, const int32_t *dst_slot, int N,
                            float *active_out, int64_t layer_stride_bytes, int S_dst,
                            int32_t *err, void *stream)
{
    constexpr int DK = 128;
    const int64_t rows = (int64_t)n_units * unit_rows;  // per slot and layer
    if ((dv != 64 && dv != 128) || unit_rows > DK || rows % DK != 0) return false;
    const auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if (!a16(codes) || !a16(scales) || !a16(unit_pos) || !a16(active_out) ||
        layer_stride_bytes % 16 != 0)
        return false;
    const int64_t blocks = rows / DK;
    if ((int64_t)L * N * blocks > (int64_t)INT_MAX) return false;
    RestoreReplayArgs a{true,     codes,     scales,   S_ckpt,  R_total, unit_pos,
                        L,        unit_rows, src_slot, dst_slot, N,      active_out,
                        layer_stride_bytes,  S_dst,    (int)blocks, DK,  dv,
                        1,        nullptr,   nullptr,  nullptr, HLA_F32, nullptr,
                        HLA_DECAY_SCALAR,    nullptr,  nullptr, nullptr, HLA_F32};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dv == 128) launch_restore_tokens<DK, 128, float, float, false>(a, err, st);
    else launch_restore_tokens<DK, 64, float, float, false>(a, err, st);
    return true;
}

template <int DK, int DV>
static void restore_tokens_dtypes(const RestoreReplayArgs &a, int32_t *err, hipStream_t st)
{
    const bool vec = a.decay == HLA_DECAY_VECTOR;
#define HLA_RT_DECAY(TI_, TO_)                                                                \
    if (vec) launch_restore_tokens<DK, DV, TI_, TO_, true>(a, err, st);                       \
    else launch_restore_tokens<DK, DV, TI_, TO_, false>(a, err, st);
#define HLA_RT_OUT(TI_)                                                                       \
    if (a.out_dtype == HLA_BF16) { HLA_RT_DECAY(TI_, uint16_t) }                              \
    else if (a.out_dtype == HLA_F16) { HLA_RT_DECAY(TI_, f16_t) }                             \
    else { HLA_RT_DECAY(TI_, float) }
    if (a.in_dtype == HLA_BF16) { HLA_RT_OUT(uint16_t) }
    else if (a.in_dtype == HLA_F16) { HLA_RT_OUT(f16_t) }
    else { HLA_RT_OUT(float) }
#undef HLA_RT_OUT
#undef HLA_RT_DECAY
}

static int run_restore_replay(const RestoreReplayArgs &a, int32_t *err, void *stream)
{
    int rc = check_restore_replay(a);
    if (rc != HLA_OK || a.N == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.dk == 128 && a.dv == 128) restore_tokens_dtypes<128, 128>(a, err, st);
    else if (a.dk == 128 && a.dv == 64) restore_tokens_dtypes<128, 64>(a, err, st);
    else if (a.dk == 64 && a.dv == 128) restore_tokens_dtypes<64, 128>(a, err, st);
    else restore_tokens_dtypes<64, 64>(a, err, st);
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

static int run_step(const StepArgs &a, int32_t *err, void *stream)
{
    int rc = check_step(a);
    if (rc != HLA_OK || a.B == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.mode == MODE_VERIFY) return run_verify(a, err, stream);
    if (a.dk == 128 && a.dv == 128) return launch_dtypes<128, 128>(a, err, st);
    if (a.dk == 128 && a.dv == 64) return launch_dtypes<128, 64>(a, err, st);
    if (a.dk == 64 && a.dv == 128) return launch_dtypes<64, 128>(a, err, st);
    return launch_dtypes<64, 64>(a, err, st);
}

} // namespace hla

extern "C" {

int gdn_step(float *state, int n_slots, const int32_t *slot, int B, int H, int dk, int dv,
             const void *q, const void *k, const void *v, int in_dtype, const float *alpha,
             const float *beta, void *out, int out_dtype, int32_t *err_flag, void *stream)
{
    hla::StepArgs a{state, n_slots, slot, B, H, dk, dv, 1, q, k, v, in_dtype, alpha,
                    HLA_DECAY_SCALAR, beta, nullptr, out, out_dtype, hla::MODE_STEP};
    return hla::run_step(a, err_flag, stream);
}

int kda_step(float *state, int n_slots, const int32_t *slot, int B, int H, int dk, int dv,
             const void *q, const void *k, const void *v, int in_dtype, const float *alpha,
             const float *beta, void *out, int out_dtype, int32_t *err_flag, void *stream)
{
    hla::StepArgs a{state, n_slots, slot, B, H, dk, dv, 1, q, k, v, in_dtype, alpha,
                    HLA_DECAY_VECTOR, beta, nullptr, out, out_dtype, hla::MODE_STEP};
    return hla::run_step(a, err_flag, stream);
}

int replay_accepted(float *state, int n_slots, const int32_t *slot, int B, int H, int dk, int dv,
                    int K, const void *q, const void *k, const void *v, int in_dtype,
                    const float *alpha, int decay_kind, const float *beta,
                    const int32_t *n_accept, void *out, int out_dtype, int32_t *err_flag,
                    void *stream)
{
    hla::StepArgs a{state, n_slots, slot, B, H, dk, dv, K, q, k, v, in_dtype, alpha,
                    decay_kind, beta, n_accept, out, out_dtype, hla::MODE_REPLAY};
    return hla::run_step(a, err_flag, stream);
}

int replay_accepted_bonus(float *state, int n_slots, const int32_t *slot, int B, int H, int dk,
                          int dv, int K, const void *q, const void *k, const void *v,
                          int in_dtype, const float *alpha, int decay_kind, const float *beta,
                          const int32_t *n_accept, void *out, const void *q_bonus,
                          const void *k_bonus, const void *v_bonus, const float *alpha_bonus,
                          const float *beta_bonus, void *out_bonus, int out_dtype,
                          int32_t *err_flag, void *stream)
{
    hla::StepArgs a{state,     n_slots,  slot,    B,       H,          dk,          dv,
                    K,         q,        k,       v,       in_dtype,   alpha,       decay_kind,
                    beta,      n_accept, out,     out_dtype, hla::MODE_BONUS, q_bonus, k_bonus,
                    v_bonus,   alpha_bonus, beta_bonus, out_bonus};
    return hla::run_step(a, err_flag, stream);
}

int dasc_restore_replay(const float *packed, int S_ckpt, int R_total, const int32_t *unit_pos,
                        int L, int unit_rows, const int32_t *src_slot, const int32_t *dst_slot,
                        int N, float *active_out, int64_t layer_stride_bytes, int S_dst, int H,
                        int dk, int dv, int K, const void *q, const void *k, const void *v,
                        int in_dtype, const float *alpha, int decay_kind, const float *beta,
                        const int32_t *n_accept, void *out, int out_dtype, int32_t *err_flag,
                        void *stream)
{
    hla::RestoreReplayArgs a{false,    packed,     nullptr,    S_ckpt,   R_total, unit_pos,
                             L,        unit_rows,  src_slot,   dst_slot, N,       active_out,
                             layer_stride_bytes,   S_dst,      H,        dk,      dv,
                             K,        q,          k,          v,        in_dtype,
                             alpha,    decay_kind, beta,       n_accept, out,     out_dtype};
    return hla::run_restore_replay(a, err_flag, stream);
}

int dasc_restore_int8_replay(const int8_t *codes, const float *scales, int S_ckpt, int R_total,
                             const int32_t *unit_pos, int L, int unit_rows,
                             const int32_t *src_slot, const int32_t *dst_slot, int N,
                             float *active_out, int64_t layer_stride_bytes, int S_dst, int H,
                             int dk, int dv, int K, const void *q, const void *k, const void *v,
                             int in_dtype, const float *alpha, int decay_kind, const float *beta,
                             const int32_t *n_accept, void *out, int out_dtype,
                             int32_t *err_flag, void *stream)
{
    hla::RestoreReplayArgs a{true,     codes,      scales,     S_ckpt,   R_total, unit_pos,
                             L,        unit_rows,  src_slot,   dst_slot, N,       active_out,
                             layer_stride_bytes,   S_dst,      H,        dk,      dv,
                             K,        q,          k,          v,        in_dtype,
                             alpha,    decay_kind, beta,       n_accept, out,     out_dtype};
    return hla::run_restore_replay(a, err_flag, stream);
}

int verify_drafts(const float *state, int n_slots, const int32_t *slot, int B, int H, int dk,
                  int dv, int K, const void *q, const void *k, const void *v, int in_dtype,
                  const float *alpha, int decay_kind, const float *beta, void *out,
                  int out_dtype, int32_t *err_flag, void *stream)
{
    // the kernel never writes the state in this mode
    hla::StepArgs a{const_cast<float *>(state), n_slots, slot, B, H, dk, dv, K, q, k, v,
                    in_dtype, alpha, decay_kind, beta, nullptr, out, out_dtype,
                    hla::MODE_VERIFY};
    return hla::run_step(a, err_flag, stream);
}

} // extern "C"

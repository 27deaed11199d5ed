// Entry points of the mixed-precision state ("DAMP: Decay-Aware Mixed-Precision
// Recurrent-State Quantization", §3.3 Eq. (7), §5.2 and App. A.1-A.4), the
// codec launches and the step variants with one scale per INT8 row and no
// value transform.  The device code is in hla_damp_kernels.h.
#include "hla_damp_kernels.h"

namespace hla {

namespace {

// Per-row scales, no value transform: compile-time FP16 row counts for
// K_hi = 0, dk/8 and dk/4 (K_hi = 16 and 32 at dk = 128); every other K_hi
// takes the run-time variant.
struct RowScale {
    template <int DK, int DV, typename TIn, typename TOut, bool VEC>
    static void run(const DampArgs &a, int32_t *err, hipStream_t st)
    {
        constexpr int NRG = DK / 8, LG = Log2<DV / 8>::v;
        if (a.K_hi == 0)
            launch_damp<DK, DV, TIn, TOut, VEC, 0, LG, false>(a, err, st);
        else if (a.K_hi == NRG)
            launch_damp<DK, DV, TIn, TOut, VEC, 1, LG, false>(a, err, st);
        else if (a.K_hi == 2 * NRG)
            launch_damp<DK, DV, TIn, TOut, VEC, 2, LG, false>(a, err, st);
        else
            launch_damp<DK, DV, TIn, TOut, VEC, -1, LG, false>(a, err, st);
    }
};

template <int DK, int DV, int LG>
void launch_codec(bool quantize, const CodecArgs &c, hipStream_t st)
{
    const dim3 grid((unsigned)((size_t)c.n_slots * c.H)), block((DK / 8) * (DV / 8));
    if (quantize)
        hipLaunchKernelGGL((k_damp_quantize<DK, DV, LG>), grid, block, 0, st, c.state_in, c.H,
                           c.key_perm, c.K_hi, c.val_perm, c.val_scale, c.hi, c.lo, c.lo_scale);
    else
        hipLaunchKernelGGL((k_damp_dequantize<DK, DV, LG>), grid, block, 0, st, c.hi, c.lo,
                           c.lo_scale, c.H, c.key_perm, c.K_hi, c.val_perm, c.val_scale,
                           c.state_out);
}

int run_codec(bool quantize, const CodecArgs &c, void *stream)
{
    int rc = check_damp_codec(c);
    if (rc != HLA_OK || c.n_slots == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool row = c.group == c.dv;
#define HLA_CODEC(DK_, DV_)                                                                   \
    if (c.dk == DK_ && c.dv == DV_) {                                                         \
        if (row) launch_codec<DK_, DV_, Log2<DV_ / 8>::v>(quantize, c, st);                    \
        else launch_codec<DK_, DV_, 2>(quantize, c, st);                                      \
    }
    HLA_CODEC(128, 128)
    HLA_CODEC(128, 64)
    HLA_CODEC(64, 128)
    HLA_CODEC(64, 64)
#undef HLA_CODEC
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

} // namespace

int launch_damp_rowscale(const DampArgs &a, int32_t *err, hipStream_t st)
{
    damp_dispatch<RowScale>(a, err, st);
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

} // namespace hla

extern "C" {

int damp_step(uint16_t *hi, int8_t *lo, float *lo_scale, int n_slots, const int32_t *key_perm,
              int K_hi, int group, const int32_t *val_perm, const float *val_scale,
              const int32_t *slot, int B, int H, int dk, int dv, const void *q, const void *k,
              const void *v, int in_dtype, const float *alpha, int decay_kind, const float *beta,
              void *out, int out_dtype, int32_t *err_flag, void *stream)
{
    hla::DampArgs a{hi,    lo,        lo_scale, n_slots, key_perm, K_hi,      group,
                    val_perm, val_scale, slot,  B,       H,        dk,        dv,
                    q,     k,         v,        in_dtype, alpha,   decay_kind, beta,
                    out,   out_dtype};
    int rc = hla::check_damp(a);
    if (rc != HLA_OK || B == 0) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (group == dv && !val_perm && !val_scale) return hla::launch_damp_rowscale(a, err_flag, st);
    return hla::launch_damp_grouped_or_sr(a, err_flag, st);
}

int damp_quantize(const float *state, int n_slots, int H, int dk, int dv, const int32_t *key_perm,
                  int K_hi, int group, const int32_t *val_perm, const float *val_scale,
                  uint16_t *hi, int8_t *lo, float *lo_scale, void *stream)
{
    hla::CodecArgs c{state, nullptr, n_slots, H, dk, dv, key_perm, K_hi, group, val_perm,
                     val_scale, hi, lo, lo_scale};
    return hla::run_codec(true, c, stream);
}

int damp_dequantize(const uint16_t *hi, const int8_t *lo, const float *lo_scale, int n_slots,
                    int H, int dk, int dv, const int32_t *key_perm, int K_hi, int group,
                    const int32_t *val_perm, const float *val_scale, float *state, void *stream)
{
    hla::CodecArgs c{nullptr, state, n_slots, H, dk, dv, key_perm, K_hi, group, val_perm,
                     val_scale, const_cast<uint16_t *>(hi), const_cast<int8_t *>(lo),
                     const_cast<float *>(lo_scale)};
    return hla::run_codec(false, c, stream);
}

} // extern "C"

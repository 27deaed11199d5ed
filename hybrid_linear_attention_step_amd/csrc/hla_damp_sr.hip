// Step variants of the mixed-precision state with one FP32 scale per group of
// 32 INT8 values ("DAMP: Decay-Aware Mixed-Precision Recurrent-State
// Quantization", App. A.1 and A.4) and with the value scaling and reordering of
// App. A.3 Eq. (17)-(18).  The device code is in hla_damp_kernels.h.
#include "hla_damp_kernels.h"

namespace hla {

namespace {

// Group-32 scales: compile-time FP16 row count for K_hi = dk/8 (the pages'
// K_hi = 16 at dk = 128), run-time otherwise; the value transform is a
// compile-time switch.  Per-row scales reach this file only with a transform.
struct GroupedOrSr {
    template <int DK, int DV, typename TIn, typename TOut, bool VEC>
    static void run(const DampArgs &a, int32_t *err, hipStream_t st)
    {
        constexpr int NRG = DK / 8, LG_ROW = Log2<DV / 8>::v;
        const bool sr = a.val_perm || a.val_scale;
        if (a.group == DV) {
            launch_damp<DK, DV, TIn, TOut, VEC, -1, LG_ROW, true>(a, err, st);
        } else if (sr) {
            if (a.K_hi == NRG)
                launch_damp<DK, DV, TIn, TOut, VEC, 1, 2, true>(a, err, st);
            else
                launch_damp<DK, DV, TIn, TOut, VEC, -1, 2, true>(a, err, st);
        } else {
            if (a.K_hi == NRG)
                launch_damp<DK, DV, TIn, TOut, VEC, 1, 2, false>(a, err, st);
            else
                launch_damp<DK, DV, TIn, TOut, VEC, -1, 2, false>(a, err, st);
        }
    }
};

} // namespace

int launch_damp_grouped_or_sr(const DampArgs &a, int32_t *err, hipStream_t st)
{
    damp_dispatch<GroupedOrSr>(a, err, st);
    return hipGetLastError() == hipSuccess ? HLA_OK : HLA_ERR_LAUNCH;
}

} // namespace hla

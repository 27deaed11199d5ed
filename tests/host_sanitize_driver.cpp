// Drives the library's host-only code (argument checks, ragged plans, static
// horizons, replay windows) with ordinary and adversarial arguments.  Built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitized.py
// (no GPU code involved); any sanitizer report aborts the run.  Exit code 0 and
// "ok" on stdout when every invariant below holds.
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "hla.h"
#include "hla_internal.h"

static int failures = 0;
#define EXPECT(c)                                                              \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32()
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

// fake, 16-byte aligned, non-overlapping device addresses (never dereferenced)
static const void *fake(uint64_t gib) { return reinterpret_cast<const void *>((gib + 1) << 40); }

static void plans()
{
    for (int trial = 0; trial < 300; ++trial) {
        const int L = 1 + (int)(next_u32() % 6), n = 1 + (int)(next_u32() % 300);
        const int keep = (int)(next_u32() % 101);
        std::vector<uint8_t> mask((size_t)L * n);
        int total = 0;
        for (auto &m : mask) total += (m = (int)(next_u32() % 100) < keep);
        std::vector<int32_t> offs(L + 1), pos((size_t)L * n);
        // exact capacity (heap buffer of exactly `total` entries)
        int32_t *idx = total ? (int32_t *)malloc(sizeof(int32_t) * total) : nullptr;
        int32_t R = -1;
        EXPECT(dasc_plan(mask.data(), L, n, offs.data(), idx, total, pos.data(), &R) == HLA_OK);
        EXPECT(R == total && offs[0] == 0 && offs[L] == total);
        for (int l = 0; l < L; ++l)
            for (int p = offs[l]; p < offs[l + 1]; ++p) {
                EXPECT(idx[p] >= 0 && idx[p] < n && mask[(size_t)l * n + idx[p]]);
                EXPECT(pos[(size_t)l * n + idx[p]] == p);
                if (p > offs[l]) EXPECT(idx[p] > idx[p - 1]);
            }
        if (total > 0) {  // one entry short: refused before anything is written
            EXPECT(dasc_plan(mask.data(), L, n, offs.data(), idx, total - 1, nullptr, &R) ==
                   HLA_ERR_PLAN);
        }
        free(idx);
    }
    int32_t o[2], R;
    uint8_t m = 1;
    EXPECT(dasc_plan(&m, 0, 1, o, nullptr, 0, nullptr, &R) == HLA_ERR_SHAPE);
    EXPECT(dasc_plan(&m, INT_MAX, INT_MAX, o, nullptr, 0, nullptr, &R) == HLA_ERR_SHAPE);
    EXPECT(dasc_plan(nullptr, 1, 1, o, nullptr, 0, nullptr, &R) == HLA_ERR_NULL);
}

static void horizons()
{
    const float special[] = {0.0f, -0.0f, 1e-30f, -1e-30f, 1e30f, -1e30f, 88.0f, -88.0f,
                             INFINITY, -INFINITY, NAN};
    const int n = (int)(sizeof(special) / sizeof(special[0]));
    std::vector<float> A(n * n), d(n * n);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) A[i * n + j] = special[i], d[i * n + j] = special[j];
    std::vector<double> H(n * n);
    std::vector<uint8_t> mk(n * n);
    for (int gate : {HLA_GATE_SOFTPLUS, HLA_GATE_BOUNDED})
        for (double eps : {1e-300, 1e-3, 0.5, 1.0 - 1e-16}) {
            EXPECT(dasc_static_horizon(A.data(), d.data(), n * n, gate, -0.3, eps, 16.0,
                                       H.data(), mk.data()) == HLA_OK);
            EXPECT(dasc_static_horizon(A.data(), d.data(), n * n, gate, 1e300, eps, 16.0,
                                       nullptr, mk.data()) == HLA_OK);
        }
    EXPECT(dasc_static_horizon(A.data(), d.data(), 4, 7, 0.0, 0.5, 16.0, H.data(), nullptr) ==
           HLA_ERR_UNSUPPORTED);
    EXPECT(dasc_static_horizon(A.data(), d.data(), 4, HLA_GATE_SOFTPLUS, 0.0, 1.0, 16.0,
                               H.data(), nullptr) == HLA_ERR_SHAPE);
    // replay windows over extreme horizons and every W_max class
    const double hs[] = {0.0, -1.0, 1e-300, 0.5, 1.0, 3.0, 4.0, 4.0000001, 1e9, 1e300,
                         INFINITY, -INFINITY, NAN};
    const int m = (int)(sizeof(hs) / sizeof(hs[0]));
    std::vector<uint8_t> msk(m);
    std::vector<int32_t> W(m);
    for (int W_max : {4, 5, 16, 1 << 20, INT_MAX})
        for (int pre : {0, 1, 7, INT_MAX}) {
            for (int i = 0; i < m; ++i) msk[i] = (uint8_t)(next_u32() & 1);
            int32_t Wr = -1;
            EXPECT(dasc_replay_window(hs, msk.data(), m, pre, W_max, W.data(), &Wr) == HLA_OK);
            for (int i = 0; i < m; ++i) EXPECT(W[i] >= 4 && W[i] <= W_max);
            EXPECT(Wr >= 0 && Wr <= pre);
        }
    int32_t Wr;
    EXPECT(dasc_replay_window(hs, msk.data(), m, 0, 3, nullptr, &Wr) == HLA_ERR_SHAPE);
}

static void checks()
{
    using namespace hla;
    const int big[] = {0, 1, 2, 255, 256, 4096, 1 << 20, INT_MAX - 1, INT_MAX};
    // the step family: any sizes give a status, never undefined arithmetic
    for (int B : big)
        for (int H : big)
            for (int S : big) {
                StepArgs a{};
                a.state = (float *)fake(1);
                a.n_slots = S;
                a.B = B, a.H = H, a.dk = 128, a.dv = 128, a.K = 16;
                a.q = fake(2), a.k = fake(3), a.v = fake(4);
                a.alpha = (const float *)fake(5), a.beta = (const float *)fake(6);
                a.n_accept = (const int32_t *)fake(7);
                a.out = (void *)fake(8);
                a.in_dtype = a.out_dtype = HLA_F32;
                a.decay = HLA_DECAY_VECTOR;
                for (int mode : {MODE_STEP, MODE_REPLAY, MODE_VERIFY}) {
                    a.mode = mode;
                    (void)check_step(a);
                }
                DampArgs dm{};
                dm.hi = (uint16_t *)fake(1), dm.lo = (int8_t *)fake(2);
                dm.lo_scale = (float *)fake(3), dm.n_slots = S, dm.K_hi = 16, dm.group = 128;
                dm.B = B, dm.H = H, dm.dk = 128, dm.dv = 128;
                dm.q = fake(4), dm.k = fake(5), dm.v = fake(6);
                dm.alpha = (const float *)fake(7), dm.beta = (const float *)fake(8);
                dm.in_dtype = dm.out_dtype = HLA_F32, dm.decay = HLA_DECAY_VECTOR;
                (void)check_damp(dm);
                CodecArgs c{};
                c.state_in = (const float *)fake(1), c.n_slots = S, c.H = H, c.dk = 128;
                c.dv = 128, c.K_hi = 16, c.group = 32;
                c.hi = (uint16_t *)fake(2), c.lo = (int8_t *)fake(3), c.lo_scale = (float *)fake(4);
                (void)check_damp_codec(c);
            }
    // the checkpoint family, including sizes whose products exceed 64 bits
    const int64_t strides[] = {0, 16, (int64_t)1 << 40, INT64_MAX - 15};
    const int64_t units[] = {16, 65536, (int64_t)1 << 40, INT64_MAX - 15};
    for (int S : big)
        for (int L : {1, 2, 1 << 16, INT_MAX})
            for (int n : {1, 4096, INT_MAX})
                for (int64_t st : strides)
                    for (int64_t ub : units)
                        for (int R : {0, 1, INT_MAX}) {
                            (void)check_dasc(fake(1), st, S, L, n, ub, fake(2), fake(3), R,
                                             (const int32_t *)fake(4), (const int32_t *)fake(5),
                                             1, fake(6), S);
                        }
    for (int S : big)
        for (int L : {1, 3, INT_MAX})
            for (int n : {1, 4096, INT_MAX})
                for (int rows : {1, 128, 256})
                    for (int R : {0, 7, INT_MAX})
                        for (int64_t st : strides)
                            (void)check_dasc_int8(fake(1), st, S, L, n, rows, 128, fake(2),
                                                  fake(3), R, (const int32_t *)fake(4),
                                                  (const int32_t *)fake(5), 1, fake(6),
                                                  fake(7), S);
    // the fused restore + replay: both halves' sizes at once
    for (int S : big)
        for (int L : {1, 4, 1 << 16, INT_MAX})
            for (int N : {0, 1, 512, INT_MAX})
                for (int H : {1, 32, INT_MAX})
                    for (int R : {0, 64, INT_MAX})
                        for (int64_t st : strides)
                        for (int ur : {1, 16, 128})
                        for (bool q8 : {false, true}) {
                            RestoreReplayArgs rr{};
                            rr.q8 = q8, rr.unit_rows = ur;
                            rr.packed = fake(1), rr.S_ckpt = S, rr.R_total = R;
                            rr.scales = q8 ? (const float *)fake(13) : nullptr;
                            rr.unit_pos = (const int32_t *)fake(2), rr.L = L;
                            rr.src_slot = (const int32_t *)fake(3);
                            rr.dst_slot = (const int32_t *)fake(4), rr.N = N;
                            rr.active_out = (float *)fake(5), rr.layer_stride_bytes = st;
                            rr.S_dst = S, rr.H = H, rr.dk = 128, rr.dv = 128, rr.K = 16;
                            rr.q = fake(6), rr.k = fake(7), rr.v = fake(8);
                            rr.in_dtype = rr.out_dtype = HLA_F32;
                            rr.alpha = (const float *)fake(9), rr.decay = HLA_DECAY_VECTOR;
                            rr.beta = (const float *)fake(10);
                            rr.n_accept = (const int32_t *)fake(11), rr.out = (void *)fake(12);
                            (void)check_restore_replay(rr);
                        }
    for (int s = -3; s < 16; ++s) EXPECT(hla_status_str(s) != nullptr);
}

int main()
{
    plans();
    horizons();
    checks();
    if (failures) return 1;
    printf("ok\n");
    return 0;
}

// Calls every entry point of the float64 oracle (oracle/oracle.c) on small ragged
// shapes with exactly sized heap buffers, padding requests, every accepted count, both
// decay kinds, FP16 budgets 0 < K_hi < dk and K_hi = dk, both scale groups, the value
// transform, empty and full checkpoint masks.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py; any report aborts the
// run.  Prints "ok" and exits 0 when every call returned.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

extern "C" {
void orc_gdn_step(double *, int, const int32_t *, int, int, int, int, const double *,
                  const double *, const double *, const double *, const double *, double *);
void orc_kda_step(double *, int, const int32_t *, int, int, int, int, const double *,
                  const double *, const double *, const double *, const double *, double *);
void orc_replay(double *, int, const int32_t *, int, int, int, int, int, const double *,
                const double *, const double *, const double *, int, const double *,
                const int32_t *, double *);
void orc_verify(const double *, int, const int32_t *, int, int, int, int, int, const double *,
                const double *, const double *, const double *, int, const double *, double *);
void orc_replay_bonus(double *, int, const int32_t *, int, int, int, int, int, const double *,
                      const double *, const double *, const double *, int, const double *,
                      const int32_t *, double *, const double *, const double *,
                      const double *, const double *, const double *, double *);
void orc_sr_step(double *, int, const int32_t *, int, int, int, int, const double *,
                 const double *, const double *, const double *, int, const double *,
                 const int32_t *, const float *, double *);
void orc_damp_quantize(const double *, int, int, int, int, const int32_t *, int, int,
                       const int32_t *, const float *, uint16_t *, int8_t *, float *);
void orc_damp_dequantize(const uint16_t *, const int8_t *, const float *, int, int, int, int,
                         const int32_t *, int, int, const int32_t *, const float *, double *);
void orc_damp_step(uint16_t *, int8_t *, float *, int, const int32_t *, int, int,
                   const int32_t *, const float *, const int32_t *, int, int, int, int,
                   const double *, const double *, const double *, const double *, int,
                   const double *, double *);
int orc_dasc_plan(const uint8_t *, int, int, int32_t *, int32_t *);
void orc_dasc_pack(const uint8_t *, long, int, int, int, long, const int32_t *,
                   const int32_t *, int, const int32_t *, const int32_t *, int, uint8_t *, int);
void orc_dasc_restore(const uint8_t *, int, int, const int32_t *, const int32_t *, int, int,
                      long, const int32_t *, const int32_t *, int, uint8_t *, long, int);
void orc_static_horizon(const double *, const double *, int, int, double, double, double *);
void orc_static_mask(const double *, int, double, uint8_t *);
int orc_replay_window(const double *, const uint8_t *, int, int, int, int32_t *);
void orc_dasc_pack_int8(const uint8_t *, long, int, int, int, int, const int32_t *,
                        const int32_t *, int, const int32_t *, const int32_t *, int, int8_t *,
                        float *);
void orc_dasc_restore_int8(const int8_t *, const float *, int, const int32_t *,
                           const int32_t *, int, int, int, int, const int32_t *,
                           const int32_t *, int, uint8_t *, long);
void orc_dasc_refresh_local(const uint8_t *, long, uint8_t *, long, int, int, long,
                            const uint8_t *, const int32_t *, const int32_t *, int);
}

static uint64_t rng = 0x243F6A8885A308D3ull;
static double uni()
{
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}
template <class T> static T *buf(size_t n, double lo = -0.5, double hi = 0.5)
{
    T *p = (T *)malloc(sizeof(T) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (T)(lo + (hi - lo) * uni());
    return p;
}

static void fp32_paths(int dk, int dv)
{
    const int B = 3, H = 2, S = 5, K = 4;
    int32_t slot[B] = {4, -1, 1};
    int32_t nacc[B] = {0, 4, 2};
    for (int per = 0; per < 2; ++per) {
        double *st = buf<double>((size_t)S * H * dk * dv);
        double *q = buf<double>((size_t)B * K * H * dk), *k = buf<double>((size_t)B * K * H * dk);
        double *v = buf<double>((size_t)B * K * H * dv);
        double *a = buf<double>((size_t)B * K * H * (per ? dk : 1), 0.5, 1.0);
        double *be = buf<double>((size_t)B * K * H, 0.0, 1.0);
        double *o = buf<double>((size_t)B * K * H * dv);
        double *o1 = buf<double>((size_t)B * H * dv);
        (per ? orc_kda_step : orc_gdn_step)(st, S, slot, B, H, dk, dv, q, k, v, a, be, o1);
        orc_replay(st, S, slot, B, H, dk, dv, K, q, k, v, a, per, be, nacc, o);
        orc_verify(st, S, slot, B, H, dk, dv, K, q, k, v, a, per, be, o);
        orc_replay_bonus(st, S, slot, B, H, dk, dv, K, q, k, v, a, per, be, nacc, o, q, k, v, a,
                         be, o1);
        int32_t *vp = (int32_t *)malloc(sizeof(int32_t) * H * dv);
        for (int h = 0; h < H; ++h)
            for (int j = 0; j < dv; ++j) vp[h * dv + j] = (j * 7 + h) % dv;  // a permutation
        float *vs = buf<float>((size_t)H * dv, 0.5, 2.0);
        orc_sr_step(st, S, slot, B, H, dk, dv, q, k, v, a, per, be, vp, vs, o1);
        for (double *p : {st, q, k, v, a, be, o, o1}) free(p);
        free(vp);
        free(vs);
    }
}

static void damp_paths(int dk, int dv)
{
    const int B = 3, H = 2, S = 4;
    int32_t slot[B] = {3, -1, 0};
    for (int K_hi : {0, 5, dk})
        for (int group : {32, dv}) {
            const int nlo = dk - K_hi, ng = dv / group;
            double *st = buf<double>((size_t)S * H * dk * dv);
            int32_t *kp = (int32_t *)malloc(sizeof(int32_t) * H * dk);
            for (int h = 0; h < H; ++h)
                for (int r = 0; r < dk; ++r) kp[h * dk + r] = (r * 5 + h) % dk;
            uint16_t *hi = (uint16_t *)malloc(sizeof(uint16_t) * ((size_t)S * H * K_hi * dv + 1));
            int8_t *lo = (int8_t *)malloc((size_t)S * H * nlo * dv + 1);
            float *sc = (float *)malloc(sizeof(float) * ((size_t)S * H * nlo * ng + 1));
            orc_damp_quantize(st, S, H, dk, dv, kp, K_hi, group, nullptr, nullptr, hi, lo, sc);
            orc_damp_dequantize(hi, lo, sc, S, H, dk, dv, kp, K_hi, group, nullptr, nullptr, st);
            double *q = buf<double>((size_t)B * H * dk), *k = buf<double>((size_t)B * H * dk);
            double *v = buf<double>((size_t)B * H * dv), *a = buf<double>((size_t)B * H * dk, .5, 1);
            double *be = buf<double>((size_t)B * H, 0, 1), *o = buf<double>((size_t)B * H * dv);
            for (int per = 0; per < 2; ++per)
                orc_damp_step(hi, lo, sc, S, kp, K_hi, group, nullptr, nullptr, slot, B, H, dk,
                              dv, q, k, v, a, per, be, o);
            for (double *p : {st, q, k, v, a, be, o}) free(p);
            free(kp), free(hi), free(lo), free(sc);
        }
}

static void dasc_paths()
{
    for (int trial = 0; trial < 40; ++trial) {
        const int L = 1 + trial % 4, n = 1 + (trial * 7) % 23, S = 1 + trial % 3;
        const long ub = 16 * (1 + trial % 5);
        const double keep = trial % 10 == 0 ? 0.0 : trial % 10 == 1 ? 1.0 : uni();
        std::vector<uint8_t> mask((size_t)L * n), local((size_t)L * n);
        for (size_t i = 0; i < mask.size(); ++i) local[i] = !(mask[i] = uni() < keep);
        std::vector<int32_t> offs(L + 1), idx(mask.size() + 1);
        const int R = orc_dasc_plan(mask.data(), L, n, offs.data(), idx.data());
        uint8_t *act = buf<uint8_t>((size_t)L * S * n * ub, 0, 255);
        uint8_t *pk = (uint8_t *)malloc((size_t)S * R * ub + 1);
        int32_t src[2] = {0, S - 1}, dst[2] = {S - 1, 0};
        const int N = S > 1 ? 2 : 1;
        orc_dasc_pack(act, (long)S * n * ub, S, L, n, ub, offs.data(), idx.data(), R, src, dst,
                      N, pk, S);
        orc_dasc_restore(pk, S, R, offs.data(), idx.data(), L, n, ub, src, dst, N, act,
                         (long)S * n * ub, S);
        orc_dasc_refresh_local(act, (long)S * n * ub, act, (long)S * n * ub, L, n, ub,
                               local.data(), src, dst, N);
        const int rows = 1 + trial % 3, dv = trial % 2 ? 64 : 128;
        const long ub8 = (long)rows * dv * 4;
        float *f = buf<float>((size_t)L * S * n * rows * dv);
        int8_t *codes = (int8_t *)malloc((size_t)S * R * rows * dv + 1);
        float *scales = (float *)malloc(sizeof(float) * ((size_t)S * R * rows + 1));
        orc_dasc_pack_int8((const uint8_t *)f, (long)S * n * ub8, L, n, rows, dv, offs.data(),
                           idx.data(), R, src, dst, N, codes, scales);
        orc_dasc_restore_int8(codes, scales, R, offs.data(), idx.data(), L, n, rows, dv, src, dst,
                              N, (uint8_t *)f, (long)S * n * ub8);
        free(act), free(pk), free(f), free(codes), free(scales);
    }
    double A[6] = {-3, -1, 0, 0.5, 2, 8}, d[6] = {-9, -1, 0, 1, 3, 40}, Hh[6];
    uint8_t m[6];
    int32_t W[6];
    for (int gate = 0; gate < 2; ++gate) {
        orc_static_horizon(A, d, 6, gate, -0.3, 1e-3, Hh);
        orc_static_mask(Hh, 6, 16.0, m);
        (void)orc_replay_window(Hh, m, 6, 9, 16, W);
    }
}

int main()
{
    for (int dk : {64, 128})
        for (int dv : {64, 128}) {
            fp32_paths(dk, dv);
            damp_paths(dk, dv);
        }
    dasc_paths();
    printf("ok\n");
    return 0;
}

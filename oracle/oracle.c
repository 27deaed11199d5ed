/*
 * Reference oracle for the gated delta-rule recurrent-state step and the state
 * formats around it.  TEST INFRASTRUCTURE ONLY: the product path (the HIP
 * library) never links, loads or calls this file.  Only the test-suite, the
 * smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * Rules this file keeps:
 *   - plain sequential C, float64 for all recurrence arithmetic, sums taken in
 *     increasing index order, built without fast-math and without FP
 *     contraction (-ffp-contract=off), so every line can be checked by eye
 *     against the equation it cites;
 *   - where the pages fix a narrower precision (the INT8 quantiser's maximum,
 *     division and rounding are FP32; the stored scale is FP32; the
 *     high-precision rows are FP16), that precision is used here too;
 *   - no blocking, fusion or reordering beyond what the cited definition says.
 *
 * Sources (page title, section / equation):
 *   [DAMP]  "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization"
 *   [dasc]  "dasc: Decay-Aware State Compression for Hybrid Linear-Attention
 *            Serving"
 *   [K3]    "Serving recurrent attention" (long-form explainer on Kimi K3),
 *           part "Speculative decoding without state snapshots"
 *
 * State orientation: one head's state is S in R^{dk x dv}, row u = key channel
 * u, as in [DAMP] §3.1.  [dasc] §3.1 Eq. (1) writes the transpose (dv x dk);
 * transposing that equation gives [DAMP] Eq. (2) exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* One head, one token: [DAMP] §3.1 Eq. (1)-(2).                              */
/*                                                                            */
/*   S_t = (I - beta k k^T) Lambda S_{t-1} + beta k v^T ,   o_t = S_t^T q      */
/*                                                                            */
/* Lambda = diag(a_0 .. a_{dk-1}); GDN passes the same a for every channel,   */
/* KDA one a per key channel ([DAMP] §3.1, [dasc] §3.1 Eq. (1)).             */
/* Expanding the product: with S' = Lambda S_{t-1},                          */
/*   (I - beta k k^T) S' + beta k v^T = S' + k (beta (v - S'^T k))^T,         */
/* so the step is: decay, delta r = S'^T k, u = beta (v - r), rank-1 write    */
/* S = S' + k u^T, and the readout of the UPDATED state ([DAMP] Eq. (1)).    */
/* ------------------------------------------------------------------------ */
static void orc_step_head(double *S, int dk, int dv, const double *q,
                          const double *k, const double *v, const double *a,
                          double beta, double *o /* may be NULL */)
{
    /* decay: S'[i][j] = a_i * S[i][j] */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(long)i * dv + j] = a[i] * S[(long)i * dv + j];

    /* delta correction and rank-1 write, one value column j at a time:
       r_j = sum_i k_i S'[i][j]  (increasing i);  u_j = beta (v_j - r_j);
       S[i][j] = S'[i][j] + k_i u_j */
    for (int j = 0; j < dv; ++j) {
        double r = 0.0;
        for (int i = 0; i < dk; ++i)
            r = r + k[i] * S[(long)i * dv + j];
        double u = beta * (v[j] - r);
        for (int i = 0; i < dk; ++i)
            S[(long)i * dv + j] = S[(long)i * dv + j] + k[i] * u;
    }

    /* readout from the updated state: o_j = sum_i q_i S[i][j] */
    if (o) {
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc = acc + q[i] * S[(long)i * dv + j];
            o[j] = acc;
        }
    }
}

/* Map request b to its state slot: identity when slot == NULL; a negative or
   out-of-range entry means "padding request, skip". */
static long orc_slot(const int32_t *slot, int b, int n_slots)
{
    long s = slot ? (long)slot[b] : (long)b;
    if (s < 0 || s >= n_slots) return -1;
    return s;
}

/* GDN decode step over a batch ([DAMP] §3.1 Eq. (2), scalar decay per head).
   state  [n_slots, H, dk, dv];  q, k [B, H, dk];  v [B, H, dv];
   alpha  [B, H];  beta [B, H];  out [B, H, dv] (rows of skipped requests are
   left untouched; out may be NULL). */
ORC_API void orc_gdn_step(double *state, int n_slots, const int32_t *slot, int B,
                          int H, int dk, int dv, const double *q, const double *k,
                          const double *v, const double *alpha, const double *beta,
                          double *out)
{
    double *a = (double *)malloc(sizeof(double) * dk);
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        for (int h = 0; h < H; ++h) {
            long bh = (long)b * H + h;
            for (int i = 0; i < dk; ++i) a[i] = alpha[bh];
            orc_step_head(state + (s * H + h) * (long)dk * dv, dk, dv, q + bh * dk,
                          k + bh * dk, v + bh * dv, a, beta[bh],
                          out ? out + bh * dv : NULL);
        }
    }
    free(a);
}

/* KDA decode step over a batch ([DAMP] §3.1 Eq. (2) with
   Lambda = diag(exp g) = diag(alpha); [dasc] §3.1 Eq. (1)).
   Same layout as orc_gdn_step except alpha [B, H, dk]. */
ORC_API void orc_kda_step(double *state, int n_slots, const int32_t *slot, int B,
                          int H, int dk, int dv, const double *q, const double *k,
                          const double *v, const double *alpha, const double *beta,
                          double *out)
{
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        for (int h = 0; h < H; ++h) {
            long bh = (long)b * H + h;
            orc_step_head(state + (s * H + h) * (long)dk * dv, dk, dv, q + bh * dk,
                          k + bh * dk, v + bh * dv, alpha + bh * dk, beta[bh],
                          out ? out + bh * dv : NULL);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Replay of accepted draft projections ([K3], "Speculative decoding without  */
/* state snapshots"): the verify pass cached the projected inputs of K draft  */
/* tokens; once n_b of them are accepted, the state is advanced by exactly    */
/* those n_b tokens, in draft order, with the ordinary step.  n_b is clamped  */
/* to [0, K].                                                                 */
/*   q, k [B, K, H, dk];  v [B, K, H, dv];  alpha [B, K, H] (GDN) or         */
/*   [B, K, H, dk] (KDA, per_channel != 0);  beta [B, K, H];                 */
/*   out [B, K, H, dv] or NULL; rows t >= n_b are left untouched.            */
/* ------------------------------------------------------------------------ */
ORC_API void orc_replay(double *state, int n_slots, const int32_t *slot, int B,
                        int H, int dk, int dv, int K, const double *q,
                        const double *k, const double *v, const double *alpha,
                        int per_channel, const double *beta,
                        const int32_t *n_accept, double *out)
{
    double *a = (double *)malloc(sizeof(double) * dk);
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        int n = n_accept[b];
        if (n < 0) n = 0;
        if (n > K) n = K;
        for (int t = 0; t < n; ++t) {
            for (int h = 0; h < H; ++h) {
                long bth = ((long)b * K + t) * H + h;
                for (int i = 0; i < dk; ++i)
                    a[i] = per_channel ? alpha[bth * dk + i] : alpha[bth];
                orc_step_head(state + (s * H + h) * (long)dk * dv, dk, dv,
                              q + bth * dk, k + bth * dk, v + bth * dv, a,
                              beta[bth], out ? out + bth * dv : NULL);
            }
        }
    }
    free(a);
}


/* Verify pass over K draft tokens ([K3], same section): the target model
   needs the readout at every draft position, computed from the committed
   state advanced through the drafts in order, while the committed state
   itself is not changed (a rejected draft must leave no trace).  The state
   of each (request, head) is copied, advanced through all K tokens with the
   ordinary step, and the copy is dropped.
   out [B, K, H, dv] (every t < K is written); layouts as orc_replay. */
ORC_API void orc_verify(const double *state, int n_slots, const int32_t *slot, int B,
                        int H, int dk, int dv, int K, const double *q,
                        const double *k, const double *v, const double *alpha,
                        int per_channel, const double *beta, double *out)
{
    double *a = (double *)malloc(sizeof(double) * dk);
    double *S = (double *)malloc(sizeof(double) * dk * dv);
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        for (int h = 0; h < H; ++h) {
            memcpy(S, state + (s * H + h) * (long)dk * dv, sizeof(double) * dk * dv);
            for (int t = 0; t < K; ++t) {
                long bth = ((long)b * K + t) * H + h;
                for (int i = 0; i < dk; ++i)
                    a[i] = per_channel ? alpha[bth * dk + i] : alpha[bth];
                orc_step_head(S, dk, dv, q + bth * dk, k + bth * dk, v + bth * dv, a,
                              beta[bth], out + bth * dv);
            }
        }
    }
    free(S);
    free(a);
}

/* After verification ([K3], same section): replay the n_b accepted draft
   projections, then apply the target model's bonus token (its own
   projections, [B, H, .] like an ordinary step) and read it out.  The
   bonus token is applied for every live request, also when n_b = 0.
   out [B, K, H, dv] or NULL for the replayed tokens (rows t >= n_b
   untouched); out_bonus [B, H, dv] or NULL. */
ORC_API void orc_replay_bonus(double *state, int n_slots, const int32_t *slot, int B,
                              int H, int dk, int dv, int K, const double *q,
                              const double *k, const double *v, const double *alpha,
                              int per_channel, const double *beta,
                              const int32_t *n_accept, double *out, const double *qb,
                              const double *kb, const double *vb, const double *alpha_b,
                              const double *beta_b, double *out_b)
{
    double *a = (double *)malloc(sizeof(double) * dk);
    orc_replay(state, n_slots, slot, B, H, dk, dv, K, q, k, v, alpha, per_channel, beta,
               n_accept, out);
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        for (int h = 0; h < H; ++h) {
            long bh = (long)b * H + h;
            for (int i = 0; i < dk; ++i)
                a[i] = per_channel ? alpha_b[bh * dk + i] : alpha_b[bh];
            orc_step_head(state + (s * H + h) * (long)dk * dv, dk, dv, qb + bh * dk,
                          kb + bh * dk, vb + bh * dv, a, beta_b[bh],
                          out_b ? out_b + bh * dv : NULL);
        }
    }
    free(a);
}

/* ------------------------------------------------------------------------ */
/* IEEE-754 binary16, written from the format's definition (1 sign bit,      */
/* 5 exponent bits with bias 15, 10 fraction bits, subnormals, round to      */
/* nearest with ties to even).  Used for the FP16 rows of the mixed-precision */
/* state ([DAMP] §5.2).                                                       */
/* ------------------------------------------------------------------------ */
ORC_API double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) 2^(e-15) */
    return sign ? -mag : mag;
}

ORC_API uint16_t orc_double_to_half(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00);
    double a = fabs(x);
    /* 65504 is the largest finite half; the midpoint to the next binade
       (65536) is 65520, which ties to the even neighbour, i.e. infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-24, m in [0, 1024] after rounding */
        double m = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)m); /* m == 1024 encodes 2^-14 */
    }
    int e;
    double f = frexp(a, &e);           /* a = f 2^e, f in [0.5, 1)        */
    double m = nearbyint(ldexp(f, 11)); /* significand with 10 fraction bits */
    int E = e - 1;                     /* a = (m / 1024) 2^E              */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | ((E + 15) << 10) | ((int)m - 1024));
}

/* ------------------------------------------------------------------------ */
/* Symmetric INT8 row quantiser: [DAMP] §3.2 Eq. (5)-(6) with b = 8, made     */
/* concrete by [dasc] App. E.1 Eq. (8): codes in [-127, 127], no zero point,  */
/* scale floored at 1e-8, and the maximum, the division and the rounding      */
/* computed in FP32 with the scale stored in FP32.  round() is taken as       */
/* round-half-to-even (the IEEE default; the pages do not name the mode).     */
/* ------------------------------------------------------------------------ */
ORC_API void orc_quantize_row_int8(const double *x, int n, int8_t *code, float *scale)
{
    float amax = 0.0f;
    for (int j = 0; j < n; ++j) {
        float xf = (float)x[j];
        float ax = fabsf(xf);
        if (ax > amax) amax = ax;
    }
    float s = fmaxf(amax, 1e-8f) / 127.0f;
    for (int j = 0; j < n; ++j) {
        float y = (float)x[j] / s;
        float r = nearbyintf(y);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        code[j] = (int8_t)r;
    }
    *scale = s;
}

/* ------------------------------------------------------------------------ */
/* Value scaling and reordering ("SR", [DAMP] App. A.1 and App. A.3         */
/* Eq. (17)-(18)).  Per head, a value permutation pi and positive scales c   */
/* define the transformed state T = S D_c^{-1} P_V^T, i.e.                   */
/*     T[i][j] = S[i][pi(j)] / c'_j ,   c'_j = c_{pi(j)} ,                   */
/* where c' (`val_scale`, [H, dv] fp32) is given in the transformed (stored) */
/* value order.  The update runs on T with v' = P_V D_c^{-1} v, i.e.        */
/* v'_j = v_{pi(j)} / c'_j, and the readout is o'_j = c'_j (T^T q)_j, which  */
/* equals o_{pi(j)}.  `val_perm` ([H, dv] int32, pi) may be NULL: then v is  */
/* already in stored value order and o is written in stored order (the page  */
/* absorbs P_V into the projection weights); otherwise v is read and o is    */
/* written in original value order.  `val_scale` NULL means c' = 1.          */
/* The key-channel side of Eq. (17) (P_K) is the packed row order below; the */
/* oracle keeps rows in original key order while it computes, which is the   */
/* same arithmetic with the rows relabelled.                                 */
/* ------------------------------------------------------------------------ */
static int orc_vperm(const int32_t *val_perm, int h, int dv, int j)
{
    return val_perm ? val_perm[(long)h * dv + j] : j;
}

static double orc_vscale(const float *val_scale, int h, int dv, int j)
{
    return val_scale ? (double)val_scale[(long)h * dv + j] : 1.0;
}

/* Eq. (18) for one head and one token on T (float64, no quantisation). */
static void orc_sr_step_head(double *T, int dk, int dv, int h, const double *q,
                             const double *k, const double *v, const double *a,
                             double beta, const int32_t *val_perm,
                             const float *val_scale, double *o /* may be NULL */)
{
    double *vt = (double *)calloc((size_t)dv, sizeof(double));
    double *ot = (double *)calloc((size_t)dv, sizeof(double));
    for (int j = 0; j < dv; ++j)
        vt[j] = v[orc_vperm(val_perm, h, dv, j)] / orc_vscale(val_scale, h, dv, j);
    orc_step_head(T, dk, dv, q, k, vt, a, beta, o ? ot : NULL);
    if (o)
        for (int j = 0; j < dv; ++j)
            o[orc_vperm(val_perm, h, dv, j)] = orc_vscale(val_scale, h, dv, j) * ot[j];
    free(ot);
    free(vt);
}

/* Batched Eq. (18) on a float64 transformed state [n_slots, H, dk, dv] (no
   quantisation): the transformed block is functionally the original one
   ([DAMP] App. A.3), which the tests check against orc_kda_step. */
ORC_API void orc_sr_step(double *state, int n_slots, const int32_t *slot, int B, int H,
                         int dk, int dv, const double *q, const double *k,
                         const double *v, const double *alpha, int decay_per_channel,
                         const double *beta, const int32_t *val_perm,
                         const float *val_scale, double *out)
{
    double *a = (double *)malloc(sizeof(double) * dk);
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        for (int h = 0; h < H; ++h) {
            long bh = (long)b * H + h;
            for (int i = 0; i < dk; ++i)
                a[i] = decay_per_channel ? alpha[bh * dk + i] : alpha[bh];
            orc_sr_step_head(state + (s * H + h) * (long)dk * dv, dk, dv, h, q + bh * dk,
                             k + bh * dk, v + bh * dv, a, beta[bh], val_perm, val_scale,
                             out ? out + bh * dv : NULL);
        }
    }
    free(a);
}

/* ------------------------------------------------------------------------ */
/* Mixed-precision packed state ([DAMP] §5.2, App. A.1 and A.4): for each    */
/* head the rows are reordered by key_perm so that packed row r holds key    */
/* channel key_perm[h*dk + r]; rows r < K_hi are stored as FP16 in `hi`      */
/* [S, H, K_hi, dv], rows r >= K_hi as INT8 codes in `lo`                    */
/* [S, H, dk-K_hi, dv] with one FP32 scale per `group` consecutive values of */
/* the row in `scale` [S, H, dk-K_hi, dv/group] (group = dv: one scale per   */
/* row, as [DAMP] §3.2 and [dasc] App. E.1; group = 32: App. A.1 / A.4).     */
/* Every group is quantised on its own by the quantiser above.  The stored  */
/* values are those of T (value side of Eq. (17)); key_perm == NULL means    */
/* identity key order.                                                       */
/* ------------------------------------------------------------------------ */
static int orc_perm(const int32_t *key_perm, int h, int dk, int r)
{
    return key_perm ? key_perm[(long)h * dk + r] : r;
}

/* Reconstruct one head (hi/lo/scale point at that head's rows) into a
   float64 dk x dv matrix T, rows in original key order, values in stored
   order: an FP16 value becomes its exact value, an INT8 code c of group g
   becomes c * s_g. */
static void orc_damp_unpack_head(const uint16_t *hi, const int8_t *lo,
                                 const float *scale, const int32_t *key_perm, int h,
                                 int K_hi, int group, int dk, int dv, double *T)
{
    int ng = dv / group;
    for (int r = 0; r < dk; ++r) {
        int u = orc_perm(key_perm, h, dk, r);
        for (int j = 0; j < dv; ++j) {
            double x;
            if (r < K_hi)
                x = orc_half_to_double(hi[(long)r * dv + j]);
            else
                x = (double)lo[(long)(r - K_hi) * dv + j] *
                    (double)scale[(long)(r - K_hi) * ng + j / group];
            T[(long)u * dv + j] = x;
        }
    }
}

/* Store one head of T: FP16 rows round the float64 value to the nearest
   half (ties to even); INT8 rows are quantised group by group. */
static void orc_damp_pack_head(const double *T, const int32_t *key_perm, int h,
                               int K_hi, int group, int dk, int dv, uint16_t *hi,
                               int8_t *lo, float *scale)
{
    int ng = dv / group;
    for (int r = 0; r < dk; ++r) {
        int u = orc_perm(key_perm, h, dk, r);
        const double *row = T + (long)u * dv;
        if (r < K_hi) {
            for (int j = 0; j < dv; ++j)
                hi[(long)r * dv + j] = orc_double_to_half(row[j]);
        } else {
            for (int g = 0; g < ng; ++g)
                orc_quantize_row_int8(row + (long)g * group, group,
                                      lo + (long)(r - K_hi) * dv + (long)g * group,
                                      scale + (long)(r - K_hi) * ng + g);
        }
    }
}

/* state S [S, H, dk, dv] in original coordinates -> packed T (Eq. (17)). */
ORC_API void orc_damp_quantize(const double *state, int S, int H, int dk, int dv,
                               const int32_t *key_perm, int K_hi, int group,
                               const int32_t *val_perm, const float *val_scale,
                               uint16_t *hi, int8_t *lo, float *scale)
{
    int nlo = dk - K_hi, ng = dv / group;
    double *T = (double *)malloc(sizeof(double) * dk * dv);
    for (long sh = 0; sh < (long)S * H; ++sh) {
        int h = (int)(sh % H);
        const double *Sh = state + sh * dk * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                T[(long)i * dv + j] = Sh[(long)i * dv + orc_vperm(val_perm, h, dv, j)] /
                                      orc_vscale(val_scale, h, dv, j);
        orc_damp_pack_head(T, key_perm, h, K_hi, group, dk, dv, hi + sh * K_hi * dv,
                           lo + sh * nlo * dv, scale + sh * nlo * ng);
    }
    free(T);
}

/* packed T -> state S in original coordinates: S[i][pi(j)] = T[i][j] c'_j. */
ORC_API void orc_damp_dequantize(const uint16_t *hi, const int8_t *lo,
                                 const float *scale, int S, int H, int dk, int dv,
                                 const int32_t *key_perm, int K_hi, int group,
                                 const int32_t *val_perm, const float *val_scale,
                                 double *state)
{
    int nlo = dk - K_hi, ng = dv / group;
    double *T = (double *)malloc(sizeof(double) * dk * dv);
    for (long sh = 0; sh < (long)S * H; ++sh) {
        int h = (int)(sh % H);
        orc_damp_unpack_head(hi + sh * K_hi * dv, lo + sh * nlo * dv, scale + sh * nlo * ng,
                             key_perm, h, K_hi, group, dk, dv, T);
        double *Sh = state + sh * dk * dv;
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                Sh[(long)i * dv + orc_vperm(val_perm, h, dv, j)] =
                    T[(long)i * dv + j] * orc_vscale(val_scale, h, dv, j);
    }
    free(T);
}

/* Quantised recurrence, [DAMP] §3.3 Eq. (7): S^q_t = Q(A_t S^q_{t-1} +
   beta k v^T), run in the transformed coordinates of App. A.3 Eq. (18).
   Reconstruct the stored T, run the float64 transformed step, take the
   readout from the updated T before it is stored again (App. A.4: update and
   readout in full precision, then requantise with recomputed group scales),
   then store it back in the packed format.
   alpha is [B, H] (decay_per_channel == 0, GDN) or [B, H, dk] (KDA), always in
   original key-channel order, like q and k. */
ORC_API void orc_damp_step(uint16_t *hi, int8_t *lo, float *scale, int n_slots,
                           const int32_t *key_perm, int K_hi, int group,
                           const int32_t *val_perm, const float *val_scale,
                           const int32_t *slot, int B, int H, int dk, int dv,
                           const double *q, const double *k, const double *v,
                           const double *alpha, int decay_per_channel,
                           const double *beta, double *out)
{
    int nlo = dk - K_hi, ng = dv / group;
    double *T = (double *)malloc(sizeof(double) * dk * dv);
    double *a = (double *)malloc(sizeof(double) * dk);
    for (int b = 0; b < B; ++b) {
        long s = orc_slot(slot, b, n_slots);
        if (s < 0) continue;
        for (int h = 0; h < H; ++h) {
            long bh = (long)b * H + h;
            long sh = s * H + h;
            for (int i = 0; i < dk; ++i)
                a[i] = decay_per_channel ? alpha[bh * dk + i] : alpha[bh];
            orc_damp_unpack_head(hi + sh * K_hi * dv, lo + sh * nlo * dv,
                                 scale + sh * nlo * ng, key_perm, h, K_hi, group, dk, dv,
                                 T);
            orc_sr_step_head(T, dk, dv, h, q + bh * dk, k + bh * dk, v + bh * dv, a,
                             beta[bh], val_perm, val_scale, out ? out + bh * dv : NULL);
            orc_damp_pack_head(T, key_perm, h, K_hi, group, dk, dv, hi + sh * K_hi * dv,
                               lo + sh * nlo * dv, scale + sh * nlo * ng);
        }
    }
    free(a);
    free(T);
}

/* ------------------------------------------------------------------------ */
/* Ragged state checkpoints ([dasc] §4.1 and App. B, "Ragged (Scheme 2)").   */
/* A unit is unit_bytes contiguous bytes: a whole head state for GDN, one    */
/* key channel's dv values for KDA.  Layer l keeps r_l = sum of its mask;     */
/* offsets o_0 = 0, o_{l+1} = o_l + r_l (0-based layers), and layer l owns    */
/* flat positions [o_l, o_{l+1}).  Inside a layer, retained units are listed  */
/* in ascending unit id (the pages do not fix the order).                     */
/* ------------------------------------------------------------------------ */
ORC_API int orc_dasc_plan(const uint8_t *mask, int L, int n_units, int32_t *offsets,
                          int32_t *unit_index)
{
    int pos = 0;
    offsets[0] = 0;
    for (int l = 0; l < L; ++l) {
        for (int u = 0; u < n_units; ++u)
            if (mask[(long)l * n_units + u]) unit_index[pos++] = u;
        offsets[l + 1] = pos;
    }
    return pos;
}

/* Store path ([dasc] App. B.1 "Runtime store", single-rank part): for each
   pair n, copy every retained unit of active slot src_slot[n] into checkpoint
   slot dst_slot[n] at its ragged position.  Layer l's active state is
   [S_act, n_units, unit_bytes] starting layer_stride_bytes * l into `active`;
   the checkpoint buffer is [S_ckpt, R_total, unit_bytes]. */
ORC_API void orc_dasc_pack(const uint8_t *active, long layer_stride_bytes, int S_act,
                           int L, int n_units, long unit_bytes, const int32_t *offsets,
                           const int32_t *unit_index, int R_total,
                           const int32_t *src_slot, const int32_t *dst_slot, int N,
                           uint8_t *packed, int S_ckpt)
{
    (void)S_act;
    (void)S_ckpt;
    for (int n = 0; n < N; ++n) {
        for (int l = 0; l < L; ++l) {
            for (int p = offsets[l]; p < offsets[l + 1]; ++p) {
                const uint8_t *src = active + (long)l * layer_stride_bytes +
                                     ((long)src_slot[n] * n_units + unit_index[p]) * unit_bytes;
                uint8_t *dst = packed + ((long)dst_slot[n] * R_total + p) * unit_bytes;
                memcpy(dst, src, (size_t)unit_bytes);
            }
        }
    }
}

/* Load path, no refresh ([dasc] §4.2 dasc-nr; App. B.2 "Insertion and
   reuse"): the retained units are restored exactly and every omitted unit of
   the destination slot reads as zero; the checkpoint itself is only read
   ([K3], the part on prefix caching: a hit gives the request its own copy). */
ORC_API void orc_dasc_restore(const uint8_t *packed, int S_ckpt, int R_total,
                              const int32_t *offsets, const int32_t *unit_index, int L,
                              int n_units, long unit_bytes, const int32_t *src_slot,
                              const int32_t *dst_slot, int N, uint8_t *active_out,
                              long layer_stride_bytes, int S_dst)
{
    (void)S_ckpt;
    (void)S_dst;
    for (int n = 0; n < N; ++n) {
        for (int l = 0; l < L; ++l) {
            uint8_t *layer = active_out + (long)l * layer_stride_bytes +
                             (long)dst_slot[n] * n_units * unit_bytes;
            memset(layer, 0, (size_t)(n_units * unit_bytes));
            for (int p = offsets[l]; p < offsets[l + 1]; ++p) {
                const uint8_t *src = packed + ((long)src_slot[n] * R_total + p) * unit_bytes;
                memcpy(layer + (long)unit_index[p] * unit_bytes, src, (size_t)unit_bytes);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Static retention horizons ([dasc] §3.3 Eq. (2)-(3)) and the selection    */
/* mask of §4.1.  For unit u (a GDN head or a KDA (head, key) channel) with   */
/* learned log-scale A_log[u] and decay bias d[u], and the model-level        */
/* representative gate input a_s:                                            */
/*   gate 0 (softplus gate):  g = -exp(A_log) * softplus(a_s + d),           */
/*                            softplus(z) = ln(1 + e^z);                      */
/*   gate 1 (bounded gate):   g = l * sigmoid(exp(A_log) * (a_s + d)),       */
/*                            l = -5, sigmoid(z) = 1 / (1 + e^-z);           */
/*   H = ln(eps) / g  (eps = 1e-3 on the page).                               */
/* A unit is global (retained in the checkpoint) when H > W_max.             */
/* ------------------------------------------------------------------------ */
static double orc_softplus(double z)
{
    /* ln(1 + e^z), written so that e^z cannot overflow */
    return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
}

ORC_API void orc_static_horizon(const double *A_log, const double *d, int n, int gate,
                                double a_s, double eps, double *H)
{
    for (int u = 0; u < n; ++u) {
        double z = a_s + d[u];
        double g;
        if (gate == 0)
            g = -exp(A_log[u]) * orc_softplus(z);
        else
            g = -5.0 / (1.0 + exp(-exp(A_log[u]) * z));
        H[u] = log(eps) / g;
    }
}

ORC_API void orc_static_mask(const double *H, int n, double W_max, uint8_t *mask)
{
    for (int u = 0; u < n; ++u) mask[u] = H[u] > W_max ? 1 : 0;
}

/* Refresh window of dasc-wr ([dasc] §4.2 Eq. (7)), for W_max >= 4:
     next_pow2(x) = 2^ceil(log2 x) for x > 0, next_pow2(0) = 4;
     W_u = clamp(next_pow2(H_u), 4, W_max);
     W_replay = min(n_prefix, max of W_u over the omitted (local) units),
   and W_replay = 0 when no unit is omitted.  W_u is written for every unit. */
ORC_API int orc_replay_window(const double *H, const uint8_t *mask, int n, int n_prefix,
                              int W_max, int32_t *W_u)
{
    int any_local = 0;
    double w_max_local = 0.0;
    for (int u = 0; u < n; ++u) {
        double w = H[u] > 0.0 ? pow(2.0, ceil(log2(H[u]))) : 4.0;
        if (w < 4.0) w = 4.0;
        if (w > (double)W_max) w = (double)W_max;
        W_u[u] = (int32_t)w;
        if (!mask[u]) {
            any_local = 1;
            if (w > w_max_local) w_max_local = w;
        }
    }
    if (!any_local) return 0;
    return (double)n_prefix < w_max_local ? n_prefix : (int)w_max_local;
}

/* ------------------------------------------------------------------------ */
/* INT8-composed checkpoints ([dasc] App. E.1 and E.2): the retained units   */
/* of the FP32 temporal state are quantised once when the checkpoint is      */
/* stored, one scale per key-channel row over its dv values (Eq. (8), the    */
/* row quantiser above), and dequantised once, q * s in FP32, into a fresh   */
/* active slot on a hit; omitted units read as zero (dasc-nr).               */
/* A unit is unit_rows rows of dv FP32 values: dk rows for a GDN head, one   */
/* row for a KDA key channel.  Layer l's active state is                     */
/* [S, n_units, unit_rows, dv] starting layer_stride_bytes * l into `active`;*/
/* codes are [S_ckpt, R_total, unit_rows, dv] int8 and scales               */
/* [S_ckpt, R_total, unit_rows] float32.                                     */
/* ------------------------------------------------------------------------ */
ORC_API void orc_dasc_pack_int8(const uint8_t *active, long layer_stride_bytes, int L,
                                int n_units, int unit_rows, int dv, const int32_t *offsets,
                                const int32_t *unit_index, int R_total,
                                const int32_t *src_slot, const int32_t *dst_slot, int N,
                                int8_t *codes, float *scales)
{
    double *row = (double *)malloc(sizeof(double) * dv);
    for (int n = 0; n < N; ++n) {
        for (int l = 0; l < L; ++l) {
            for (int p = offsets[l]; p < offsets[l + 1]; ++p) {
                const float *unit = (const float *)(active + (long)l * layer_stride_bytes) +
                                    ((long)src_slot[n] * n_units + unit_index[p]) *
                                        unit_rows * dv;
                for (int r = 0; r < unit_rows; ++r) {
                    for (int j = 0; j < dv; ++j) row[j] = (double)unit[(long)r * dv + j];
                    long dst_row = ((long)dst_slot[n] * R_total + p) * unit_rows + r;
                    orc_quantize_row_int8(row, dv, codes + dst_row * dv, scales + dst_row);
                }
            }
        }
    }
    free(row);
}

ORC_API void orc_dasc_restore_int8(const int8_t *codes, const float *scales, int R_total,
                                   const int32_t *offsets, const int32_t *unit_index, int L,
                                   int n_units, int unit_rows, int dv,
                                   const int32_t *src_slot, const int32_t *dst_slot, int N,
                                   uint8_t *active_out, long layer_stride_bytes)
{
    long unit_vals = (long)unit_rows * dv;
    for (int n = 0; n < N; ++n) {
        for (int l = 0; l < L; ++l) {
            float *layer = (float *)(active_out + (long)l * layer_stride_bytes) +
                           (long)dst_slot[n] * n_units * unit_vals;
            memset(layer, 0, sizeof(float) * (size_t)(n_units * unit_vals));
            for (int p = offsets[l]; p < offsets[l + 1]; ++p) {
                float *unit = layer + (long)unit_index[p] * unit_vals;
                for (int r = 0; r < unit_rows; ++r) {
                    long src_row = ((long)src_slot[n] * R_total + p) * unit_rows + r;
                    double s = (double)scales[src_row];
                    for (int j = 0; j < dv; ++j)  /* exact product, rounded once to FP32 */
                        unit[(long)r * dv + j] = (float)((double)codes[src_row * dv + j] * s);
                }
            }
        }
    }
}

/* dasc-wr copy-back ([dasc] §4.2): after the refresh window has been
   replayed from a zero-initialised scratch state, only the refreshed local
   units are copied into the active state; the retained global units keep
   their exact checkpoint values.  `local` is uint8 [L, n_units], 1 for a
   local (omitted) unit.  Both states are [S, n_units, unit_bytes] per layer
   with their own layer strides. */
ORC_API void orc_dasc_refresh_local(const uint8_t *scratch, long scratch_layer_stride,
                                    uint8_t *active, long layer_stride, int L, int n_units,
                                    long unit_bytes, const uint8_t *local,
                                    const int32_t *src_slot, const int32_t *dst_slot, int N)
{
    for (int n = 0; n < N; ++n)
        for (int l = 0; l < L; ++l)
            for (int u = 0; u < n_units; ++u) {
                if (!local[(long)l * n_units + u]) continue;
                memcpy(active + l * layer_stride + ((long)dst_slot[n] * n_units + u) * unit_bytes,
                       scratch + l * scratch_layer_stride +
                           ((long)src_slot[n] * n_units + u) * unit_bytes,
                       (size_t)unit_bytes);
            }
}

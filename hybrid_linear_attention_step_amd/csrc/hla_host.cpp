// Host-only parts of the C ABI: status strings, argument validation and the
// ragged checkpoint plan.  Nothing here calls the HIP runtime.
#include <limits.h>
#include <math.h>
#include <string.h>

#include "hla.h"
#include "hla_internal.h"

namespace hla {

static const size_t kMaxIndex = (size_t)INT_MAX;

// Products and sums of sizes in int64, refused (false) where they would overflow.
static bool mul_ok(int64_t a, int64_t b, int64_t &out) { return !__builtin_mul_overflow(a, b, &out); }
static bool mul3_ok(int64_t a, int64_t b, int64_t c, int64_t &out)
{
    int64_t t;
    return mul_ok(a, b, t) && mul_ok(t, c, out);
}

int check_step(const StepArgs &a)
{
    const bool multi = a.mode != MODE_STEP;
    const bool replay = a.mode == MODE_REPLAY || a.mode == MODE_BONUS;
    const bool bonus = a.mode == MODE_BONUS;
    if (a.B < 0 || a.H <= 0 || a.n_slots < 0) return HLA_ERR_SHAPE;
    if (multi && (a.K < 1 || a.K > 16)) return HLA_ERR_SHAPE;
    if (!dtype_ok(a.in_dtype) || !dtype_ok(a.out_dtype)) return HLA_ERR_DTYPE;
    if (a.decay != HLA_DECAY_SCALAR && a.decay != HLA_DECAY_VECTOR) return HLA_ERR_DTYPE;
    if (a.B == 0) return HLA_OK;
    if (!a.state || !a.q || !a.k || !a.v || !a.alpha || !a.beta) return HLA_ERR_NULL;
    if (replay && !a.n_accept) return HLA_ERR_NULL;
    if (a.mode == MODE_VERIFY && !a.out) return HLA_ERR_NULL;  // readouts are the result
    if (bonus && (!a.qb || !a.kb || !a.vb || !a.alpha_b || !a.beta_b)) return HLA_ERR_NULL;
    if (!a.slot && a.n_slots < a.B) return HLA_ERR_SHAPE;
    if (!head_dim_ok(a.dk) || !head_dim_ok(a.dv)) return HLA_ERR_UNSUPPORTED;
    if ((size_t)a.B * a.H > kMaxIndex || (size_t)a.n_slots * a.H > kMaxIndex)
        return HLA_ERR_SHAPE;
    const bool vec = a.decay == HLA_DECAY_VECTOR;
    if (!aligned16(a.state) || !aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) ||
        (a.out && !aligned16(a.out)) || (vec && !aligned16(a.alpha)))
        return HLA_ERR_ALIGN;
    if (bonus && (!aligned16(a.qb) || !aligned16(a.kb) || !aligned16(a.vb) ||
                  (a.out_b && !aligned16(a.out_b)) || (vec && !aligned16(a.alpha_b))))
        return HLA_ERR_ALIGN;

    const size_t bh = (size_t)a.B * a.H;
    const size_t tok = bh * a.K;  // (request, token, head) triples
    const size_t es = dtype_bytes(a.in_dtype), os = dtype_bytes(a.out_dtype);
    const size_t adk = vec ? a.dk : 1;
    Range state{a.state, (size_t)a.n_slots * a.H * a.dk * a.dv * sizeof(float)};
    Range out{a.out, tok * a.dv * os};
    Range out_b{bonus ? a.out_b : nullptr, bh * a.dv * os};
    Range ins[] = {
        {a.q, tok * a.dk * es},
        {a.k, tok * a.dk * es},
        {a.v, tok * a.dv * es},
        {a.alpha, tok * adk * sizeof(float)},
        {a.beta, tok * sizeof(float)},
        {a.slot, (size_t)a.B * sizeof(int32_t)},
        {a.n_accept, (size_t)a.B * sizeof(int32_t)},
        {bonus ? a.qb : nullptr, bh * a.dk * es},
        {bonus ? a.kb : nullptr, bh * a.dk * es},
        {bonus ? a.vb : nullptr, bh * a.dv * es},
        {bonus ? a.alpha_b : nullptr, bh * adk * sizeof(float)},
        {bonus ? a.beta_b : nullptr, bh * sizeof(float)},
    };
    for (const Range &r : ins)
        if (overlaps(state, r) || overlaps(out, r) || overlaps(out_b, r)) return HLA_ERR_ALIAS;
    if (overlaps(state, out) || overlaps(state, out_b) || overlaps(out, out_b))
        return HLA_ERR_ALIAS;
    return HLA_OK;
}

int check_damp(const DampArgs &a)
{
    if (a.B < 0 || a.H <= 0 || a.n_slots < 0) return HLA_ERR_SHAPE;
    if (!dtype_ok(a.in_dtype) || !dtype_ok(a.out_dtype)) return HLA_ERR_DTYPE;
    if (a.decay != HLA_DECAY_SCALAR && a.decay != HLA_DECAY_VECTOR) return HLA_ERR_DTYPE;
    if (a.B == 0) return HLA_OK;
    if (!head_dim_ok(a.dk) || !head_dim_ok(a.dv)) return HLA_ERR_UNSUPPORTED;
    if (!damp_group_ok(a.group, a.dv)) return HLA_ERR_UNSUPPORTED;
    if (a.K_hi < 0 || a.K_hi > a.dk) return HLA_ERR_SHAPE;
    const int nlo = a.dk - a.K_hi;
    if ((a.K_hi > 0 && !a.hi) || (nlo > 0 && (!a.lo || !a.lo_scale)) || !a.q || !a.k || !a.v ||
        !a.alpha || !a.beta)
        return HLA_ERR_NULL;
    if (!a.slot && a.n_slots < a.B) return HLA_ERR_SHAPE;
    if ((size_t)a.B * a.H > kMaxIndex || (size_t)a.n_slots * a.H > kMaxIndex)
        return HLA_ERR_SHAPE;
    if ((a.hi && !aligned16(a.hi)) || (a.lo && !aligned16(a.lo)) || !aligned16(a.q) ||
        !aligned16(a.k) || !aligned16(a.v) || (a.out && !aligned16(a.out)))
        return HLA_ERR_ALIGN;
    const size_t sh = (size_t)a.n_slots * a.H;
    const size_t bh = (size_t)a.B * a.H;
    const size_t es = dtype_bytes(a.in_dtype);
    const size_t ng = (size_t)(a.dv / a.group);
    Range outs[] = {
        {a.hi, sh * a.K_hi * a.dv * 2},
        {a.lo, sh * nlo * a.dv},
        {a.lo_scale, sh * nlo * ng * sizeof(float)},
        {a.out, bh * a.dv * dtype_bytes(a.out_dtype)},
    };
    Range ins[] = {
        {a.q, bh * a.dk * es},
        {a.k, bh * a.dk * es},
        {a.v, bh * a.dv * es},
        {a.alpha, bh * (a.decay == HLA_DECAY_VECTOR ? a.dk : 1) * sizeof(float)},
        {a.beta, bh * sizeof(float)},
        {a.slot, (size_t)a.B * sizeof(int32_t)},
        {a.key_perm, (size_t)a.H * a.dk * sizeof(int32_t)},
        {a.val_perm, (size_t)a.H * a.dv * sizeof(int32_t)},
        {a.val_scale, (size_t)a.H * a.dv * sizeof(float)},
    };
    for (int i = 0; i < 4; ++i) {
        for (const Range &r : ins)
            if (overlaps(outs[i], r)) return HLA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(outs[i], outs[j])) return HLA_ERR_ALIAS;
    }
    return HLA_OK;
}

int check_damp_codec(const CodecArgs &c)
{
    if (c.n_slots < 0 || c.H <= 0) return HLA_ERR_SHAPE;
    if (c.n_slots == 0) return HLA_OK;
    if (!head_dim_ok(c.dk) || !head_dim_ok(c.dv)) return HLA_ERR_UNSUPPORTED;
    if (!damp_group_ok(c.group, c.dv)) return HLA_ERR_UNSUPPORTED;
    if (c.K_hi < 0 || c.K_hi > c.dk) return HLA_ERR_SHAPE;
    const int nlo = c.dk - c.K_hi;
    const void *state = c.state_in ? (const void *)c.state_in : (const void *)c.state_out;
    if (!state || (c.K_hi > 0 && !c.hi) || (nlo > 0 && (!c.lo || !c.lo_scale)))
        return HLA_ERR_NULL;
    if ((size_t)c.n_slots * c.H > kMaxIndex) return HLA_ERR_SHAPE;
    if (!aligned16(state) || (c.hi && !aligned16(c.hi)) || (c.lo && !aligned16(c.lo)))
        return HLA_ERR_ALIGN;
    const size_t sh = (size_t)c.n_slots * c.H;
    const size_t ng = (size_t)(c.dv / c.group);
    Range st{state, sh * c.dk * c.dv * sizeof(float)};
    Range packed[] = {{c.hi, sh * c.K_hi * c.dv * 2},
                      {c.lo, sh * nlo * c.dv},
                      {c.lo_scale, sh * nlo * ng * 4}};
    Range tables[] = {{c.key_perm, (size_t)c.H * c.dk * 4},
                      {c.val_perm, (size_t)c.H * c.dv * 4},
                      {c.val_scale, (size_t)c.H * c.dv * 4}};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(st, packed[i])) return HLA_ERR_ALIAS;
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(packed[i], packed[j])) return HLA_ERR_ALIAS;
    }
    // the codec's output must not overwrite its plan tables
    for (const Range &t : tables) {
        if (c.state_out && overlaps(st, t)) return HLA_ERR_ALIAS;
        if (c.state_in)
            for (const Range &p : packed)
                if (overlaps(p, t)) return HLA_ERR_ALIAS;
    }
    return HLA_OK;
}

int check_dasc(const void *active, int64_t layer_stride_bytes, int S_act, int L, int n_units,
               int64_t unit_bytes, const void *table_a, const void *table_b, int R_total,
               const int32_t *src_slot, const int32_t *dst_slot, int N, const void *packed,
               int S_ckpt)
{
    if (N < 0 || L <= 0 || n_units <= 0 || S_act < 0 || S_ckpt < 0 || R_total < 0 ||
        unit_bytes <= 0 || layer_stride_bytes < 0)
        return HLA_ERR_SHAPE;
    if (R_total > (int64_t)L * n_units) return HLA_ERR_PLAN;
    if (N == 0) return HLA_OK;
    if (!active || !packed || !table_a || (R_total > 0 && !table_b) || !src_slot || !dst_slot)
        return HLA_ERR_NULL;
    if (unit_bytes % 16 != 0 || layer_stride_bytes % 16 != 0) return HLA_ERR_ALIGN;
    if (!aligned16(active) || !aligned16(packed)) return HLA_ERR_ALIGN;
    // per-pair vector counts must fit the kernels' 32-bit indexing
    const int64_t unit_vecs = unit_bytes / 16;
    int64_t per_pair, layer_bytes, span, pk_bytes;
    if (!mul3_ok(unit_vecs, L, n_units, per_pair) || per_pair > (int64_t)INT_MAX)
        return HLA_ERR_SHAPE;
    if (!mul3_ok(S_act, n_units, unit_bytes, layer_bytes)) return HLA_ERR_SHAPE;
    if (L > 1 && layer_stride_bytes < layer_bytes) return HLA_ERR_SHAPE;
    if (!mul_ok(L - 1, layer_stride_bytes, span) ||
        __builtin_add_overflow(span, layer_bytes, &span) ||
        !mul3_ok(S_ckpt, R_total, unit_bytes, pk_bytes))
        return HLA_ERR_SHAPE;
    Range act{active, (size_t)span};
    Range pk{packed, (size_t)pk_bytes};
    if (overlaps(act, pk)) return HLA_ERR_ALIAS;
    return HLA_OK;
}

int check_dasc_tables(Range w0, Range w1, const int32_t *offsets, int L,
                      const int32_t *unit_index, int R, const int32_t *unit_pos, int n_units,
                      const int32_t *src_slot, const int32_t *dst_slot, int N)
{
    const Range tables[] = {{offsets, (size_t)(L + 1) * sizeof(int32_t)},
                            {unit_index, (size_t)R * sizeof(int32_t)},
                            {unit_pos, (size_t)L * n_units * sizeof(int32_t)},
                            {src_slot, (size_t)N * sizeof(int32_t)},
                            {dst_slot, (size_t)N * sizeof(int32_t)}};
    for (const Range &t : tables)
        if (overlaps(w0, t) || overlaps(w1, t)) return HLA_ERR_ALIAS;
    return HLA_OK;
}

int check_restore_replay(const RestoreReplayArgs &a)
{
    if (a.N < 0 || a.L <= 0 || a.H <= 0 || a.S_ckpt < 0 || a.S_dst < 0 || a.R_total < 0 ||
        a.layer_stride_bytes < 0)
        return HLA_ERR_SHAPE;
    if (a.K < 1 || a.K > 16) return HLA_ERR_SHAPE;
    if (!dtype_ok(a.in_dtype) || !dtype_ok(a.out_dtype)) return HLA_ERR_DTYPE;
    if (a.decay != HLA_DECAY_SCALAR && a.decay != HLA_DECAY_VECTOR) return HLA_ERR_DTYPE;
    if (!head_dim_ok(a.dk) || !head_dim_ok(a.dv)) return HLA_ERR_UNSUPPORTED;
    if (a.unit_rows < 1 || a.unit_rows > a.dk || (a.unit_rows & (a.unit_rows - 1)) != 0)
        return HLA_ERR_SHAPE;
    int64_t units;  // in the plan; the kernel indexes unit_pos in 32 bits
    if (!mul3_ok(a.L, a.H, a.dk / a.unit_rows, units) || units > (int64_t)INT_MAX)
        return HLA_ERR_SHAPE;
    if ((int64_t)a.R_total > units) return HLA_ERR_PLAN;
    if (a.N == 0) return HLA_OK;
    const bool q8 = a.q8;
    if ((a.R_total > 0 && (!a.packed || (q8 && !a.scales))) || !a.unit_pos || !a.src_slot ||
        !a.dst_slot || !a.active_out || !a.q || !a.k || !a.v || !a.alpha || !a.beta ||
        !a.n_accept)
        return HLA_ERR_NULL;
    const bool vec = a.decay == HLA_DECAY_VECTOR;
    if ((a.packed && !aligned16(a.packed)) || !aligned16(a.active_out) || !aligned16(a.q) ||
        !aligned16(a.k) || !aligned16(a.v) || (a.out && !aligned16(a.out)) ||
        (vec && !aligned16(a.alpha)) || !aligned16(a.unit_pos) ||
        (q8 && a.scales && !aligned16(a.scales)) || a.layer_stride_bytes % 16 != 0)
        return HLA_ERR_ALIGN;
    // sizes: workgroups (l, n, h) and (l, n, t, h) tokens must fit 32-bit indices; the
    // byte spans must fit 64 bits
    const int64_t head = (int64_t)a.dk * a.dv * 4;
    int64_t groups, toks, layer_bytes, span, pk_bytes;
    if (!mul3_ok(a.L, a.N, a.H, groups) || groups > (int64_t)INT_MAX ||
        !mul_ok(groups, a.K, toks) || toks > (int64_t)INT_MAX)
        return HLA_ERR_SHAPE;
    if (!mul3_ok(a.S_dst, a.H, head, layer_bytes)) return HLA_ERR_SHAPE;
    if (a.L > 1 && a.layer_stride_bytes < layer_bytes) return HLA_ERR_SHAPE;
    if (!mul_ok(a.L - 1, a.layer_stride_bytes, span) ||
        __builtin_add_overflow(span, layer_bytes, &span) ||
        !mul3_ok(a.S_ckpt, a.R_total, (int64_t)a.unit_rows * a.dv * (q8 ? 1 : 4), pk_bytes))
        return HLA_ERR_SHAPE;
    int64_t sc_bytes = 0;  // INT8: one FP32 scale per checkpoint row
    if (q8 && !mul3_ok(a.S_ckpt, a.R_total, (int64_t)a.unit_rows * 4, sc_bytes))
        return HLA_ERR_SHAPE;
    const size_t es = dtype_bytes(a.in_dtype), os = dtype_bytes(a.out_dtype);
    const size_t nt = (size_t)toks;
    const Range act{a.active_out, (size_t)span};
    const Range outr{a.out, nt * a.dv * os};
    const Range ins[] = {
        {a.packed, (size_t)pk_bytes},
        {a.scales, (size_t)sc_bytes},
        {a.q, nt * a.dk * es},
        {a.k, nt * a.dk * es},
        {a.v, nt * a.dv * es},
        {a.alpha, nt * (vec ? a.dk : 1) * sizeof(float)},
        {a.beta, nt * sizeof(float)},
        {a.unit_pos, (size_t)units * sizeof(int32_t)},
        {a.src_slot, (size_t)a.N * sizeof(int32_t)},
        {a.dst_slot, (size_t)a.N * sizeof(int32_t)},
        {a.n_accept, (size_t)a.N * sizeof(int32_t)},
    };
    for (const Range &r : ins)
        if (overlaps(act, r) || overlaps(outr, r)) return HLA_ERR_ALIAS;
    if (overlaps(act, outr)) return HLA_ERR_ALIAS;
    return HLA_OK;
}

int check_dasc_int8(const void *active, int64_t layer_stride_bytes, int S_act, int L,
                    int n_units, int unit_rows, int dv, const void *table_a,
                    const void *table_b, int R_total, const int32_t *src_slot,
                    const int32_t *dst_slot, int N, const void *codes, const void *scales,
                    int S_ckpt)
{
    if (unit_rows <= 0 || unit_rows > 256 || (unit_rows & (unit_rows - 1)) != 0)
        return HLA_ERR_SHAPE;
    if (dv != 64 && dv != 128) return HLA_ERR_UNSUPPORTED;
    const int64_t unit_bytes = (int64_t)unit_rows * dv * 4;
    // the FP32 side, with the codes standing in for the packed operand (sized below)
    int rc = check_dasc(active, layer_stride_bytes, S_act, L, n_units, unit_bytes, table_a,
                        table_b, R_total, src_slot, dst_slot, N, codes, 0);
    if (rc != HLA_OK || N == 0) return rc;
    if (!scales) return HLA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(scales) & 3u) != 0) return HLA_ERR_ALIGN;
    // checkpoint rows must fit the kernels' 32-bit row indexing (so the code and scale
    // byte counts below fit as well)
    int64_t ck_rows, layer_bytes, span;
    if (!mul3_ok(S_ckpt, R_total, unit_rows, ck_rows) || ck_rows > (int64_t)INT_MAX)
        return HLA_ERR_SHAPE;
    if (!mul3_ok(S_act, n_units, unit_bytes, layer_bytes) ||
        !mul_ok(L - 1, layer_stride_bytes, span) ||
        __builtin_add_overflow(span, layer_bytes, &span))
        return HLA_ERR_SHAPE;
    Range act{active, (size_t)span};
    Range cd{codes, (size_t)ck_rows * dv};
    Range sc{scales, (size_t)ck_rows * sizeof(float)};
    if (overlaps(act, cd) || overlaps(act, sc) || overlaps(cd, sc)) return HLA_ERR_ALIAS;
    return HLA_OK;
}

} // namespace hla

extern "C" {

const char *hla_status_str(int status)
{
    switch (status) {
    case HLA_OK: return "ok";
    case HLA_ERR_NULL: return "a required pointer is NULL";
    case HLA_ERR_SHAPE: return "invalid size or shape";
    case HLA_ERR_ALIGN: return "pointer or size not 16-byte aligned";
    case HLA_ERR_DTYPE: return "unknown dtype or decay kind";
    case HLA_ERR_PLAN: return "inconsistent checkpoint plan";
    case HLA_ERR_ALIAS: return "an output buffer overlaps an input";
    case HLA_ERR_UNSUPPORTED: return "head size not supported (dk, dv must be 64 or 128)";
    case HLA_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int hla_version(void) { return 102; }

// Ragged plan ([dasc] App. B, Scheme 2): r_l retained units per layer,
// o_0 = 0, o_{l+1} = o_l + r_l, retained units of layer l at flat positions
// [o_l, o_{l+1}) in ascending unit id; unit_pos inverts the map (-1 = omitted).
int dasc_plan(const uint8_t *mask, int L, int n_units, int32_t *offsets, int32_t *unit_index,
              int cap, int32_t *unit_pos, int32_t *R_total)
{
    if (!mask || !offsets || !R_total || (cap > 0 && !unit_index)) return HLA_ERR_NULL;
    if (L <= 0 || n_units <= 0 || cap < 0) return HLA_ERR_SHAPE;
    if ((int64_t)L * n_units > (int64_t)INT_MAX) return HLA_ERR_SHAPE;
    int64_t total = 0;
    for (int64_t i = 0; i < (int64_t)L * n_units; ++i) total += mask[i] ? 1 : 0;
    if (total > cap) return HLA_ERR_PLAN;
    int32_t pos = 0;
    offsets[0] = 0;
    for (int l = 0; l < L; ++l) {
        for (int u = 0; u < n_units; ++u) {
            const int64_t g = (int64_t)l * n_units + u;
            if (mask[g]) {
                unit_index[pos] = u;
                if (unit_pos) unit_pos[g] = pos;
                ++pos;
            } else if (unit_pos) {
                unit_pos[g] = -1;
            }
        }
        offsets[l + 1] = pos;
    }
    *R_total = pos;
    return HLA_OK;
}

int dasc_static_horizon(const float *A_log, const float *d, int n, int gate, double a_s,
                        double eps, double W_max, double *H_out, uint8_t *mask_out)
{
    if (n < 0) return HLA_ERR_SHAPE;
    if (gate != HLA_GATE_SOFTPLUS && gate != HLA_GATE_BOUNDED) return HLA_ERR_UNSUPPORTED;
    if (!(eps > 0.0 && eps < 1.0)) return HLA_ERR_SHAPE;
    if (n == 0) return HLA_OK;
    if (!A_log || !d || (!H_out && !mask_out)) return HLA_ERR_NULL;
    const double log_eps = log(eps);
    for (int u = 0; u < n; ++u) {
        const double x = (double)a_s + (double)d[u];
        const double scale = exp((double)A_log[u]);
        double g;  // static one-step log-decay, < 0
        if (gate == HLA_GATE_SOFTPLUS) {
            const double sp = x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
            g = -scale * sp;
        } else {
            g = -5.0 / (1.0 + exp(-scale * x));
        }
        const double H = log_eps / g;
        if (H_out) H_out[u] = H;
        if (mask_out) mask_out[u] = H > W_max ? 1 : 0;
    }
    return HLA_OK;
}

int dasc_replay_window(const double *H, const uint8_t *mask, int n, int n_prefix, int W_max,
                       int32_t *W_u_out, int32_t *W_replay_out)
{
    if (n < 0 || n_prefix < 0 || W_max < 4) return HLA_ERR_SHAPE;
    if (!W_replay_out || (n > 0 && (!H || !mask))) return HLA_ERR_NULL;
    int32_t longest_local = -1;
    for (int u = 0; u < n; ++u) {
        // next power of two at or above H (H <= 0 maps to 4), clamped to [4, W_max]
        int64_t w = 4;
        if (H[u] > 0.0) {
            const double e = ceil(log2(H[u]));
            w = e >= 62.0 ? ((int64_t)1 << 62) : e <= 0.0 ? 1 : ((int64_t)1 << (int)e);
        }
        if (w < 4) w = 4;
        if (w > W_max) w = W_max;
        if (W_u_out) W_u_out[u] = (int32_t)w;
        if (!mask[u] && w > longest_local) longest_local = (int32_t)w;
    }
    *W_replay_out = longest_local < 0 ? 0 : (n_prefix < longest_local ? n_prefix : longest_local);
    return HLA_OK;
}

} // extern "C"

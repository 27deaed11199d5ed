/*
 * hla.h -- C ABI of the MI355X (gfx950) library for the gated delta-rule
 * recurrent-state step used in GDN and KDA decode, its mixed-precision state
 * variant, ragged state checkpoints, and the replay of accepted draft tokens.
 *
 * Pages this interface follows (cited by title and section/equation):
 *   [DAMP]  "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization"
 *   [dasc]  "dasc: Decay-Aware State Compression for Hybrid Linear-Attention
 *            Serving"
 *   [K3]    "Serving recurrent attention" (long-form explainer on Kimi K3)
 *
 * Conventions shared by every entry point
 *   - One head's state is S in R^{dk x dv}, row-major, row u = key channel u
 *     ([DAMP] §3.1).  A state tensor is [n_slots, H, dk, dv].
 *   - Every buffer is owned by the caller.  Buffers marked "device" live in
 *     GPU memory; buffers marked "host" in CPU memory.  The library never
 *     allocates, frees or synchronises; all work is enqueued on `stream`
 *     (a hipStream_t; NULL = the legacy default stream) and runs
 *     asynchronously.
 *   - The return value is a status (HLA_OK = 0).  Arguments are validated on
 *     the host before anything is launched; on an error nothing is launched
 *     and nothing is written.  HLA_ERR_LAUNCH reports a failed launch; faults
 *     that happen later surface at the caller's next synchronisation.
 *   - Index tables that live in device memory (slot maps, accepted counts,
 *     plan tables) cannot be checked on the host without a sync.  Kernels
 *     never access memory out of bounds because of them: a bad entry is
 *     skipped (or clamped, where stated) and, when `err_flag` (device int32,
 *     may be NULL) is given, the matching HLA_DEVERR_* bit is OR-ed into it.
 *   - Supported head sizes: dk, dv in {64, 128}.  Pointers to vectorised
 *     buffers must be 16-byte aligned.
 *   - All entry points are reentrant; the library keeps no mutable global
 *     state.  Concurrent calls that write the same buffers race.
 *   - Within one call, the non-negative entries of a slot map that selects
 *     state the call writes (slot of the state-updating entry points, dst_slot
 *     of the checkpoint copies) must be distinct: two requests or pairs naming
 *     the same slot would update it from two workgroups at once, and the
 *     result is undefined.  Maps the call only reads through (src_slot, the
 *     slot of verify_drafts) may repeat entries.
 */
#ifndef HLA_H
#define HLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from the shared library even when it is
   built with hidden default visibility. */
#if defined(__GNUC__) || defined(__clang__)
#define HLA_API __attribute__((visibility("default")))
#else
#define HLA_API
#endif

enum hla_status {
    HLA_OK = 0,
    HLA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    HLA_ERR_SHAPE = 2,       /* a size is negative, zero where not allowed,
                                or the problem exceeds 32-bit index limits     */
    HLA_ERR_ALIGN = 3,       /* a vectorised pointer is not 16-byte aligned    */
    HLA_ERR_DTYPE = 4,       /* unknown dtype or decay-kind code               */
    HLA_ERR_PLAN = 5,        /* inconsistent host plan (mask/offsets/capacity) */
    HLA_ERR_ALIAS = 6,       /* an output overlaps an input it must not        */
    HLA_ERR_UNSUPPORTED = 7, /* valid but not instantiated (e.g. dk = 96)      */
    HLA_ERR_LAUNCH = 8       /* the kernel launch failed                       */
};

/* Element types of q, k, v (in_dtype) and of the readout o (out_dtype): FP32,
 * bf16, or IEEE binary16; 2-byte outputs are rounded to nearest even. */
enum hla_dtype { HLA_F32 = 0, HLA_BF16 = 1, HLA_F16 = 2 };

/* Decay granularity: one scalar per head (GDN) or one per key channel (KDA). */
enum hla_decay { HLA_DECAY_SCALAR = 0, HLA_DECAY_VECTOR = 1 };

/* Bits OR-ed into *err_flag by kernels that meet a bad device-side index. */
enum hla_device_error {
    HLA_DEVERR_SLOT = 1,    /* slot / src / dst index >= its bound: pair skipped */
    HLA_DEVERR_ACCEPT = 2,  /* n_accept outside [0, K]: clamped                  */
    HLA_DEVERR_PLAN = 4     /* plan table entry out of range: unit skipped (a
                               restore writes that unit as zeros)               */
};

/* Static, NUL-terminated description of a status code.  Thread-safe. */
HLA_API const char *hla_status_str(int status);

/* Library ABI version (major * 100 + minor): 102 (1.01 added HLA_F16, 1.02
 * dasc_restore_replay and dasc_restore_int8_replay). */
HLA_API int hla_version(void);

/* -------------------------------------------------------------------------
 * gdn_step -- one GDN decode step for a batch of requests, in place.
 *
 * Computes, for every request b with a state slot and every head h
 * ([DAMP] §3.1 Eq. (1)-(2); [dasc] §3.1 Eq. (1), transposed):
 *     S' = alpha S                    (scalar decay per head)
 *     u  = beta (v - S'^T k)          (delta correction, in R^dv)
 *     S  = S' + k u^T                 (written back into the slot)
 *     o  = S^T q                      (readout of the updated state)
 *
 * state   device float32 [n_slots, H, dk, dv], read and written.
 * slot    device int32 [B] mapping request b to its state slot, or NULL for
 *         the identity (then n_slots >= B).  A negative entry marks a padding
 *         request: nothing is read or written for it (its rows of `out` are
 *         left untouched).  An entry >= n_slots is skipped likewise and sets
 *         HLA_DEVERR_SLOT.
 * q, k    device [B, H, dk] of in_dtype; v device [B, H, dv] of in_dtype.
 *         q and k are expected to be l2-normalised per head ([DAMP] §3.1);
 *         the kernel does not normalise them.
 * alpha   device float32 [B, H], the decay factors in (0, 1].
 * beta    device float32 [B, H], the delta-rule strengths in (0, 1).
 * out     device [B, H, dv] of out_dtype, or NULL for no readout.
 * Errors: NULL, SHAPE, ALIGN (state, q, k, v, out), DTYPE, UNSUPPORTED,
 *         ALIAS (out or state overlapping an input), LAUNCH.
 * ---------------------------------------------------------------------- */
HLA_API int gdn_step(float *state, int n_slots, const int32_t *slot, int B, int H, int dk,
             int dv, const void *q, const void *k, const void *v, int in_dtype,
             const float *alpha, const float *beta, void *out, int out_dtype,
             int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * kda_step -- one KDA decode step: as gdn_step, but the decay is a vector
 * over key channels, Lambda = diag(alpha_0 .. alpha_{dk-1}) = diag(exp g),
 * so row u of the state is multiplied by alpha_u ([DAMP] §3.1 Eq. (2);
 * [dasc] §3.1 Eq. (1)).
 *
 * alpha   device float32 [B, H, dk] (16-byte aligned).  All other arguments
 *         as gdn_step.
 * ---------------------------------------------------------------------- */
HLA_API int kda_step(float *state, int n_slots, const int32_t *slot, int B, int H, int dk,
             int dv, const void *q, const void *k, const void *v, int in_dtype,
             const float *alpha, const float *beta, void *out, int out_dtype,
             int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * Mixed-precision packed state ([DAMP] §5.2 and App. A.1-A.4).  For each slot
 * and head the dk key-channel rows are reordered by a static plan so that
 * packed row r holds key channel key_perm[h*dk + r]; rows r < K_hi are stored
 * in FP16, rows r >= K_hi as symmetric INT8 codes with one FP32 scale per
 * `group` consecutive values of the row:
 *     hi        device uint16 (IEEE binary16 bits) [n_slots, H, K_hi, dv]
 *     lo        device int8                        [n_slots, H, dk-K_hi, dv]
 *     lo_scale  device float32                     [n_slots, H, dk-K_hi, dv/group]
 * group is dv (one scale per row: [DAMP] §3.2, [dasc] App. E.1 Eq. (8)) or 32
 * (the deployed layout of [DAMP] App. A.1 / A.4, 9.875 bits per value at
 * 16 of 128 rows in FP16); other values return HLA_ERR_UNSUPPORTED.
 * The INT8 quantiser is [DAMP] §3.2 Eq. (5)-(6) with b = 8 as made concrete in
 * [dasc] App. E.1 Eq. (8), applied to each group on its own: a = max |x| over
 * the group, s = max(a, 1e-8) / 127, c = clip(round(x / s), -127, 127),
 * computed in FP32, s stored in FP32, round = nearest-even.  FP16 rows are
 * rounded to nearest-even.  key_perm is device int32 [H, dk], a permutation of
 * 0..dk-1 per head, or NULL for the identity (the pages fold the order into
 * the projection weights, [DAMP] §5.2).  0 <= K_hi <= dk.
 *
 * Value scaling and reordering ([DAMP] App. A.3 Eq. (17)-(18)).  The stored
 * values are those of T = S D^-1 P_V^T: stored column j of every row holds
 * original value index pi(j) = val_perm[h*dv + j] divided by c'_j =
 * val_scale[h*dv + j] (c'_j > 0, given in stored order).  val_perm is device
 * int32 [H, dv], a permutation per head, or NULL when the value order is
 * already folded into the projection weights (then v is read and o written in
 * stored order); val_scale is device float32 [H, dv], or NULL for c' = 1.
 * Both NULL is the untransformed state.
 * ---------------------------------------------------------------------- */

/* damp_step -- one decode step on the packed state, in place ([DAMP] §3.3
 * Eq. (7), S^q_t = Q(A_t S^q_{t-1} + beta k v^T), fused as in App. A.4):
 * reconstruct each row (FP16 value, or code * group scale), run the
 * gdn_step / kda_step update and readout in FP32 on T (App. A.3 Eq. (18):
 * v'_j = v_{pi(j)} / c'_j, o_{pi(j)} = c'_j (T^T q)_j), then requantise every
 * INT8 group with a freshly computed scale and round every FP16 row, and
 * write all three regions back.  The readout o is taken from the FP32
 * updated state before it is requantised.
 *
 * q, k, alpha (when decay_kind == HLA_DECAY_VECTOR) are indexed by ORIGINAL
 * key channel, [B, H, dk]; the kernel gathers them through key_perm.
 * alpha is [B, H] for HLA_DECAY_SCALAR.  v and out are indexed by original
 * value index when val_perm is given, else by stored column.  slot, beta,
 * err_flag as gdn_step; a val_perm entry outside [0, dv) sets
 * HLA_DEVERR_PLAN and is read as the identity.
 * Errors: as gdn_step, plus SHAPE for K_hi outside [0, dk] and UNSUPPORTED
 * for another group.
 */
HLA_API int damp_step(uint16_t *hi, int8_t *lo, float *lo_scale, int n_slots,
              const int32_t *key_perm, int K_hi, int group, const int32_t *val_perm,
              const float *val_scale, const int32_t *slot, int B, int H, int dk, int dv,
              const void *q, const void *k, const void *v, int in_dtype,
              const float *alpha, int decay_kind, const float *beta, void *out,
              int out_dtype, int32_t *err_flag, void *stream);

/* damp_quantize -- pack an FP32 state S [n_slots, H, dk, dv] (device, original
 * coordinates) into the three regions above: T = S D^-1 P_V^T (FP32 division,
 * [DAMP] App. A.3 Eq. (17)), then the quantiser of [DAMP] §3.2 Eq. (5)-(6)
 * for the INT8 groups and nearest-even FP16 for the K_hi selected rows
 * ([DAMP] §5.2, App. A.4).  The FP32 input is only read; hi, lo and lo_scale
 * are caller-owned device buffers, entirely written.  Nothing is allocated.
 * Errors: NULL for a missing buffer the layout needs; SHAPE for n_slots < 0,
 * H <= 0 or K_hi outside [0, dk]; UNSUPPORTED for dk, dv outside {64, 128}
 * or a group other than dv or 32; ALIGN for a state, hi or lo pointer that
 * is not 16-byte aligned; ALIAS when the packed regions overlap the state,
 * each other or the plan tables.  n_slots == 0 launches nothing. */
HLA_API int damp_quantize(const float *state, int n_slots, int H, int dk, int dv,
                  const int32_t *key_perm, int K_hi, int group, const int32_t *val_perm,
                  const float *val_scale, uint16_t *hi, int8_t *lo, float *lo_scale,
                  void *stream);

/* damp_dequantize -- reconstruct the FP32 state in original coordinates from
 * the packed regions ([DAMP] §3.2, App. A.3 Eq. (17) inverted): FP16 values
 * exactly, INT8 values as code * group scale (one FP32 rounding), then
 * S[i][pi(j)] = T[i][j] * c'_j.  The packed regions are only read; state is
 * a caller-owned device buffer, entirely written.  Errors: as damp_quantize
 * (ALIAS when the state overlaps a packed region or a plan table). */
HLA_API int damp_dequantize(const uint16_t *hi, const int8_t *lo, const float *lo_scale,
                    int n_slots, int H, int dk, int dv, const int32_t *key_perm,
                    int K_hi, int group, const int32_t *val_perm, const float *val_scale,
                    float *state, void *stream);

/* -------------------------------------------------------------------------
 * Ragged state checkpoints ([dasc] §4.1, §4.2 and App. B "Ragged (Scheme 2)").
 * A unit is unit_bytes contiguous bytes of one slot's state in one layer: a
 * whole head for GDN (dk*dv*4 bytes), one key channel's row for KDA (dv*4
 * bytes).  Layer l of the active state is [S, n_units, unit_bytes] starting
 * l * layer_stride_bytes into the buffer.  A static mask selects the retained
 * units; layer l keeps r_l of them, offsets o_0 = 0, o_{l+1} = o_l + r_l, and
 * its units occupy flat positions [o_l, o_{l+1}) of a checkpoint slot
 * [R_total, unit_bytes], R_total = sum_l r_l, listed in ascending unit id.
 * ---------------------------------------------------------------------- */

/* dasc_plan -- HOST-only.  Build the ragged plan once from the mask
 * ([dasc] App. B.2: masks, offsets and maps are precomputed once).
 * mask        host uint8 [L, n_units]; nonzero = retained.
 * offsets     host int32 [L + 1] (written).
 * unit_index  host int32 [cap] (written: first R_total entries).
 * unit_pos    host int32 [L * n_units] or NULL (written: flat position of
 *             each unit, -1 for an omitted unit); dasc_restore uses it.
 * R_total     host int32 (written).
 * Errors: NULL, SHAPE, PLAN (cap < R_total). */
HLA_API int dasc_plan(const uint8_t *mask, int L, int n_units, int32_t *offsets,
              int32_t *unit_index, int cap, int32_t *unit_pos, int32_t *R_total);

/* dasc_pack -- store path ([dasc] App. B.1 "Runtime store", the single-rank
 * fused pack): for each pair n < N, copy every retained unit of active slot
 * src_slot[n] of every layer into checkpoint slot dst_slot[n] at its flat
 * position.  Bit copy.  The active state is only read.
 * active      device, layer l at active + l * layer_stride_bytes, each layer
 *             [S_act, n_units, unit_bytes].
 * offsets     device int32 [L + 1]; unit_index device int32 [R_total].
 * src_slot    device int32 [N] (< S_act); dst_slot device int32 [N] (< S_ckpt).
 * packed      device [S_ckpt, R_total, unit_bytes].
 * unit_bytes must be a positive multiple of 16; layer_stride_bytes a multiple
 * of 16 and >= S_act * n_units * unit_bytes.
 * Errors: NULL, SHAPE, ALIGN, ALIAS (packed overlapping active), LAUNCH. */
HLA_API int dasc_pack(const void *active, int64_t layer_stride_bytes, int S_act, int L,
              int n_units, int64_t unit_bytes, const int32_t *offsets,
              const int32_t *unit_index, int R_total, const int32_t *src_slot,
              const int32_t *dst_slot, int N, void *packed, int S_ckpt,
              int32_t *err_flag, void *stream);

/* dasc_restore -- load path without refresh ([dasc] §4.2 dasc-nr; App. B.2
 * "Insertion and reuse"): for each pair n < N, write EVERY unit of every layer
 * of private slot dst_slot[n]: a retained unit receives its packed bytes from
 * checkpoint slot src_slot[n], an omitted unit is zero-filled.  The checkpoint
 * is only read: a hit leaves the checkpoint as it is and gives the request a
 * state of its own ([K3], the part on prefix caching).
 * unit_pos    device int32 [L * n_units] from dasc_plan.
 * active_out  device, layer l at active_out + l * layer_stride_bytes, each
 *             layer [S_dst, n_units, unit_bytes].
 * Errors: as dasc_pack; a unit_pos entry >= R_total sets HLA_DEVERR_PLAN and
 * that unit is written as zeros. */
HLA_API int dasc_restore(const void *packed, int S_ckpt, int R_total, const int32_t *unit_pos,
                 int L, int n_units, int64_t unit_bytes, const int32_t *src_slot,
                 const int32_t *dst_slot, int N, void *active_out,
                 int64_t layer_stride_bytes, int S_dst, int32_t *err_flag,
                 void *stream);

/* -------------------------------------------------------------------------
 * replay_accepted -- advance each request's state by its accepted draft
 * tokens only ([K3] "Speculative decoding without state snapshots": the
 * verify pass caches the projected inputs of the K draft tokens; after
 * verification the accepted ones are replayed on-chip into the state).
 * For request b, for t = 0 .. n_b - 1 in order, the gdn_step / kda_step
 * update is applied with draft projection t; the state is read once and
 * written once, and not touched at all when n_b = 0.  The bonus token is not
 * part of this call (it is the next ordinary step).
 *
 * q, k     device [B, K, H, dk]; v device [B, K, H, dv] (in_dtype).
 * alpha    device float32 [B, K, H] (HLA_DECAY_SCALAR) or [B, K, H, dk].
 * beta     device float32 [B, K, H].
 * n_accept device int32 [B]; values outside [0, K] are clamped and set
 *          HLA_DEVERR_ACCEPT.
 * out      device [B, K, H, dv] of out_dtype or NULL: the readout after each
 *          replayed token; rows t >= n_b are left untouched.  With NULL the
 *          readout is not formed and q is not read (it must still be given).
 * 1 <= K <= 16.  state, slot, err_flag as gdn_step.
 * Errors: as gdn_step, plus SHAPE for K outside [1, 16] and NULL for a
 * missing n_accept.
 * ---------------------------------------------------------------------- */
HLA_API int replay_accepted(float *state, int n_slots, const int32_t *slot, int B, int H,
                    int dk, int dv, int K, const void *q, const void *k, const void *v,
                    int in_dtype, const float *alpha, int decay_kind, const float *beta,
                    const int32_t *n_accept, void *out, int out_dtype, int32_t *err_flag,
                    void *stream);

/* -------------------------------------------------------------------------
 * replay_accepted_bonus -- replay_accepted fused with the next ordinary step
 * ([K3] "Speculative decoding without state snapshots": the replay of the
 * accepted drafts and the step of the token the target model itself emitted
 * after them run in one kernel).  For request b: the first n_b draft
 * tokens as replay_accepted, then one gdn_step / kda_step update with the
 * bonus token's own projections, all on one read and one write of the state.
 * The bonus token is applied for every live request, also when n_b = 0.
 *
 * q .. n_accept, out  as replay_accepted (out may be NULL: no draft
 *                     readouts; the drafts' q is read either way).
 * q_bonus, k_bonus    device [B, H, dk]; v_bonus [B, H, dv] (in_dtype).
 * alpha_bonus         device float32 [B, H] or [B, H, dk] (decay_kind).
 * beta_bonus          device float32 [B, H].
 * out_bonus           device [B, H, dv] of out_dtype, or NULL: the bonus
 *                     token's readout from the updated state.
 * Errors: as replay_accepted, plus NULL for a missing bonus input.
 * ---------------------------------------------------------------------- */
HLA_API int replay_accepted_bonus(float *state, int n_slots, const int32_t *slot, int B, int H,
                          int dk, int dv, int K, const void *q, const void *k, const void *v,
                          int in_dtype, const float *alpha, int decay_kind, const float *beta,
                          const int32_t *n_accept, void *out, const void *q_bonus,
                          const void *k_bonus, const void *v_bonus, const float *alpha_bonus,
                          const float *beta_bonus, void *out_bonus, int out_dtype,
                          int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * dasc_restore_replay -- dasc_restore of a checkpoint followed by
 * replay_accepted, in one pass over each private head ([dasc] §4.2 dasc-nr
 * restore, then [K3] "Speculative decoding without state snapshots": the
 * accepted drafts are applied on-chip).  A unit is unit_rows consecutive key
 * channels (rows) of one head: unit_rows = dk for whole-head units (GDN, [dasc]
 * §4.1), 1 for single key channels (KDA, [dasc] §3.3 / §4.1); head h, rows
 * [j * unit_rows, (j + 1) * unit_rows) is unit h * (dk / unit_rows) + j of its
 * layer.  For each pair n < N, layer l < L and head h: each unit of the head
 * of private slot dst_slot[n] in layer l starts as its packed copy from
 * checkpoint slot src_slot[n] when retained, and as zero otherwise; the first
 * n_b = n_accept[n] draft tokens of layer l are applied to the head in order
 * (clamped to [0, K]); it is written once.  The result equals dasc_restore
 * (unit_bytes = unit_rows * dv * 4) followed by replay_accepted on each layer,
 * bit for bit, with one read of the retained units and one write of each head
 * instead of a read, two writes and a read.
 *
 * packed      device float32 [S_ckpt, R_total, unit_rows, dv]: dasc_pack of
 *             the units.  Only read.
 * unit_pos    device int32 [L, H * dk / unit_rows] (16-byte aligned) from
 *             dasc_plan of the unit mask; an entry >= R_total sets
 *             HLA_DEVERR_PLAN and that unit starts from zero.
 * unit_rows   a power of two, 1 <= unit_rows <= dk.
 * src_slot    device int32 [N] (< S_ckpt); dst_slot device int32 [N] (< S_dst,
 *             distinct); a pair out of range is skipped (HLA_DEVERR_SLOT).
 * active_out  device float32, layer l at active_out + l * layer_stride_bytes,
 *             each layer [S_dst, H, dk, dv]; heads of slots no pair names are
 *             left as they are.
 * q, k        device [L, N, K, H, dk]; v device [L, N, K, H, dv] (in_dtype):
 *             the draft projections of every layer.
 * alpha       device float32 [L, N, K, H] (HLA_DECAY_SCALAR) or
 *             [L, N, K, H, dk]; beta device float32 [L, N, K, H].
 * n_accept    device int32 [N]: accepted drafts per request (every layer
 *             replays the same count); values outside [0, K] are clamped and set
 *             HLA_DEVERR_ACCEPT.
 * out         device [L, N, K, H, dv] of out_dtype, or NULL: the readout after
 *             each replayed token; rows t >= n_b are left untouched.  With NULL
 *             the readouts are not formed and q is not read.
 * 1 <= K <= 16; dk, dv in {64, 128}; layer_stride_bytes a multiple of 16 and
 * >= S_dst * H * dk * dv * 4.
 * Errors: NULL, SHAPE (including unit_rows), ALIGN, DTYPE, UNSUPPORTED, PLAN
 * (R_total above the unit count L * H * dk / unit_rows), ALIAS (the private
 * state overlapping the checkpoint, an input, a plan table or a slot map; the
 * readout overlapping an input), LAUNCH.
 * ---------------------------------------------------------------------- */
HLA_API int dasc_restore_replay(const float *packed, int S_ckpt, int R_total,
                                const int32_t *unit_pos, int L, int unit_rows,
                                const int32_t *src_slot, const int32_t *dst_slot, int N,
                                float *active_out, int64_t layer_stride_bytes, int S_dst, int H,
                                int dk, int dv, int K, const void *q, const void *k,
                                const void *v, int in_dtype, const float *alpha, int decay_kind,
                                const float *beta, const int32_t *n_accept, void *out,
                                int out_dtype, int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * verify_drafts -- the recurrent layer's part of the target model's verify
 * pass over K draft tokens ([K3] "Speculative decoding without state
 * snapshots": the committed state must not absorb drafts that may be
 * rejected).  For every request, out[b, t] is the readout after the committed
 * state has been advanced through draft tokens 0..t in order; the state in
 * memory is only read.  The kernel evaluates the drafts in unrolled form (the
 * state enters only through S^T [c_t k_t | c_t q_t], c_t the cumulative decay,
 * computed on the matrix cores in FP32), so the readouts equal a token-by-token
 * replay's up to FP32 summation order, not bit for bit.  The same
 * projections, kept by the caller, are what replay_accepted later replays.
 *
 * state    device float32 [n_slots, H, dk, dv], read only.
 * q .. beta, slot, K  as replay_accepted.
 * out      device [B, K, H, dv] of out_dtype; required.
 * Errors: as replay_accepted; NULL if out is NULL.
 * ---------------------------------------------------------------------- */
HLA_API int verify_drafts(const float *state, int n_slots, const int32_t *slot, int B, int H,
                  int dk, int dv, int K, const void *q, const void *k, const void *v,
                  int in_dtype, const float *alpha, int decay_kind, const float *beta,
                  void *out, int out_dtype, int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * INT8-composed checkpoints ([dasc] App. E.1 Eq. (8) and App. E.2): the
 * retained units of an FP32 temporal state are quantised once when the
 * checkpoint is stored, one FP32 scale per key-channel row over its dv values
 * (the row quantiser of the mixed-precision state: a = max |x|, s = max(a,
 * 1e-8) / 127, codes clip(round(x / s), -127, 127), FP32), and dequantised
 * once on a hit, q * s rounded once to FP32, into a fresh active slot; the
 * omitted units of that slot read as zero (dasc-nr).
 *
 * A unit is unit_rows consecutive rows of dv FP32 values: unit_rows = dk for
 * a GDN head, 1 for a KDA (head, key) channel.  unit_rows is a power of two
 * <= 256; dv is 64 or 128.  Layer l's active state is
 * [S, n_units, unit_rows, dv] starting layer_stride_bytes * l into active
 * (16-byte aligned, stride a multiple of 16).
 *   codes   device int8    [S_ckpt, R_total, unit_rows, dv] (16-byte aligned)
 *   scales  device float32 [S_ckpt, R_total, unit_rows]
 * Plans, slots, N, err_flag and errors as dasc_pack / dasc_restore.
 * ---------------------------------------------------------------------- */
HLA_API int dasc_pack_int8(const float *active, int64_t layer_stride_bytes, int S_act, int L,
                   int n_units, int unit_rows, int dv, const int32_t *offsets,
                   const int32_t *unit_index, int R_total, const int32_t *src_slot,
                   const int32_t *dst_slot, int N, int8_t *codes, float *scales, int S_ckpt,
                   int32_t *err_flag, void *stream);

HLA_API int dasc_restore_int8(const int8_t *codes, const float *scales, int S_ckpt,
                      int R_total, const int32_t *unit_pos, int L, int n_units, int unit_rows,
                      int dv, const int32_t *src_slot, const int32_t *dst_slot, int N,
                      float *active_out, int64_t layer_stride_bytes, int S_dst,
                      int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * dasc_restore_int8_replay -- dasc_restore_int8 followed by replay_accepted in
 * one pass over each private head, as dasc_restore_replay does for an FP32
 * checkpoint ([dasc] App. E.1 Eq. (8): a hit dequantises each retained row
 * once, value = code * scale in FP32; [dasc] §4.2 dasc-nr; [K3] "Speculative
 * decoding without state snapshots").  The result equals dasc_restore_int8
 * (n_units = H * dk / unit_rows) followed by replay_accepted on each layer, bit
 * for bit.
 *
 * codes       device int8 [S_ckpt, R_total, unit_rows, dv] (16-byte aligned)
 * scales      device float32 [S_ckpt, R_total, unit_rows] (16-byte aligned):
 *             dasc_pack_int8 of the units.  Only read.
 * Every other argument, the unit geometry, the device errors and the status
 * codes are those of dasc_restore_replay (ALIAS also when the private state or
 * the readout overlaps the codes or the scales).
 * ---------------------------------------------------------------------- */
HLA_API int dasc_restore_int8_replay(const int8_t *codes, const float *scales, int S_ckpt,
                                     int R_total, const int32_t *unit_pos, int L, int unit_rows,
                                     const int32_t *src_slot, const int32_t *dst_slot, int N,
                                     float *active_out, int64_t layer_stride_bytes, int S_dst,
                                     int H, int dk, int dv, int K, const void *q, const void *k,
                                     const void *v, int in_dtype, const float *alpha,
                                     int decay_kind, const float *beta, const int32_t *n_accept,
                                     void *out, int out_dtype, int32_t *err_flag, void *stream);

/* -------------------------------------------------------------------------
 * Static selection ([dasc] §3.3 Eq. (2)-(3), §4.1).  Host-only, float64.
 * For each of n units (a GDN head or a KDA (head, key) channel) with learned
 * log-scale A_log[u] and decay bias d[u], and the model-level representative
 * gate input a_s:
 *   HLA_GATE_SOFTPLUS  g = -exp(A_log) * ln(1 + exp(a_s + d))
 *   HLA_GATE_BOUNDED   g = -5 / (1 + exp(-exp(A_log) * (a_s + d)))
 *   H = ln(eps) / g  (the pages use eps = 1e-3),
 * and the unit is global (retained, mask 1) when H > W_max.  H_out (double
 * [n]) and mask_out (uint8 [n]) may each be NULL, not both.  The mask feeds
 * dasc_plan.  Errors: SHAPE for n < 0 or eps outside (0, 1), UNSUPPORTED for
 * another gate, NULL.
 * ---------------------------------------------------------------------- */
enum hla_gate { HLA_GATE_SOFTPLUS = 0, HLA_GATE_BOUNDED = 1 };

HLA_API int dasc_static_horizon(const float *A_log, const float *d, int n, int gate,
                        double a_s, double eps, double W_max, double *H_out,
                        uint8_t *mask_out);

/* dasc_replay_window -- the dasc-wr refresh window ([dasc] §4.2 Eq. (7)).
 * Host-only.  W_u = clamp(next_pow2(H_u), 4, W_max) with next_pow2(x) =
 * 2^ceil(log2 x) for x > 0 and 4 for x <= 0; W_replay = min(n_prefix, max of
 * W_u over the local units (mask 0)), and 0 when no unit is local.  W_u_out
 * (int32 [n]) may be NULL.  Errors: SHAPE for W_max < 4 or negative sizes,
 * NULL. */
HLA_API int dasc_replay_window(const double *H, const uint8_t *mask, int n, int n_prefix,
                       int W_max, int32_t *W_u_out, int32_t *W_replay_out);

/* dasc_refresh_local -- the copy-back of dasc-wr ([dasc] §4.2): after the
 * refresh window has been replayed from a zero-initialised scratch state,
 * copy only the local (omitted) units of scratch slot src_slot[n] into
 * active slot dst_slot[n]; every other unit of the active slot, the global
 * ones included, is left as it is.  offsets / unit_index / R_local are the
 * ragged plan of the LOCAL units, i.e. dasc_plan of the inverted selection
 * mask.  The scratch state has the active state's unit geometry with its own
 * layer stride and slot count.  Units, alignment, err_flag and errors as
 * dasc_pack; ALIAS when the two states overlap. */
HLA_API int dasc_refresh_local(const void *scratch, int64_t scratch_layer_stride_bytes,
                       int S_scratch, void *active, int64_t layer_stride_bytes, int S_act,
                       int L, int n_units, int64_t unit_bytes, const int32_t *offsets,
                       const int32_t *unit_index, int R_local, const int32_t *src_slot,
                       const int32_t *dst_slot, int N, int32_t *err_flag, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HLA_H */

// Host-side argument checking shared by the launchers.  Pure C++: nothing in
// here touches the GPU, so every error path can be exercised without one.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "hla.h"

namespace hla {

struct Range {
    const void *p;
    size_t bytes;
};

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool overlaps(Range a, Range b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

inline bool head_dim_ok(int d) { return d == 64 || d == 128; }
inline bool dtype_ok(int t) { return t == HLA_F32 || t == HLA_BF16 || t == HLA_F16; }
inline size_t dtype_bytes(int t) { return t == HLA_F32 ? 4 : 2; }

// What a step-kernel launch does with its tokens.
enum StepMode {
    MODE_STEP = 0,    // one token, state updated (gdn_step / kda_step)
    MODE_REPLAY = 1,  // first n_b of K tokens, state updated (replay_accepted)
    MODE_BONUS = 2,   // first n_b of K tokens, then one bonus token (replay_accepted_bonus)
    MODE_VERIFY = 3,  // all K tokens with readouts, state not written (verify_drafts)
};

// Everything the step / replay / verify launchers need, in one place.
struct StepArgs {
    float *state;
    int n_slots;
    const int32_t *slot;
    int B, H, dk, dv;
    int K;  // tokens per request: 1 for a step, the draft count otherwise
    const void *q, *k, *v;
    int in_dtype;
    const float *alpha;
    int decay;
    const float *beta;
    const int32_t *n_accept;  // replay modes only
    void *out;
    int out_dtype;
    int mode;
    // bonus token [B, H, .] (MODE_BONUS only)
    const void *qb, *kb, *vb;
    const float *alpha_b, *beta_b;
    void *out_b;
};

// Returns HLA_OK or the first error found.
int check_step(const StepArgs &a);

// Launches the verify pass (MODE_VERIFY) for arguments that passed check_step
// with B > 0; `stream` is a hipStream_t.  Defined with its kernel in hla_verify.hip.
int run_verify(const StepArgs &a, int32_t *err, void *stream);

struct DampArgs {
    uint16_t *hi;
    int8_t *lo;
    float *lo_scale;
    int n_slots;
    const int32_t *key_perm;
    int K_hi;
    int group;                 // INT8 values per FP32 scale: dv (per row) or 32
    const int32_t *val_perm;   // [H, dv] stored column -> original value index, or NULL
    const float *val_scale;    // [H, dv] value scale of each stored column, or NULL
    const int32_t *slot;
    int B, H, dk, dv;
    const void *q, *k, *v;
    int in_dtype;
    const float *alpha;
    int decay;
    const float *beta;
    void *out;
    int out_dtype;
};

int check_damp(const DampArgs &a);

// damp_quantize (state_in set) / damp_dequantize (state_out set).
struct CodecArgs {
    const float *state_in;
    float *state_out;
    int n_slots, H, dk, dv;
    const int32_t *key_perm;
    int K_hi;
    int group;
    const int32_t *val_perm;
    const float *val_scale;
    uint16_t *hi;
    int8_t *lo;
    float *lo_scale;
};

int check_damp_codec(const CodecArgs &c);

// Scale groups the kernels are built for: one scale per row, or per 32 values.
inline bool damp_group_ok(int group, int dv) { return group == dv || group == 32; }

int check_dasc(const void *active, int64_t layer_stride_bytes, int S_act, int L, int n_units,
               int64_t unit_bytes, const void *table_a, const void *table_b, int R_total,
               const int32_t *src_slot, const int32_t *dst_slot, int N, const void *packed,
               int S_ckpt);

// The plan tables and slot maps a checkpoint kernel reads while it writes
// (offsets [L+1], unit_index [R], unit_pos [L*n_units], src/dst [N]; NULL
// entries are skipped) must not overlap what the call writes (w0, w1):
// HLA_ERR_ALIAS if one does.
int check_dasc_tables(Range w0, Range w1, const int32_t *offsets, int L,
                      const int32_t *unit_index, int R, const int32_t *unit_pos, int n_units,
                      const int32_t *src_slot, const int32_t *dst_slot, int N);

// Bytes from the first byte of layer 0 to the end of layer L-1 of a layered
// state (arguments already validated by check_dasc / check_dasc_int8).
inline int64_t dasc_span(int64_t layer_stride_bytes, int L, int S, int n_units,
                         int64_t unit_bytes)
{
    return (int64_t)(L - 1) * layer_stride_bytes + (int64_t)S * n_units * unit_bytes;
}

// INT8 checkpoints: a unit is unit_rows (a power of two, <= 256) rows of dv
// (64 or 128) FP32 values; codes [S_ckpt, R_total, unit_rows, dv] int8 and
// scales [S_ckpt, R_total, unit_rows] float32.
int check_dasc_int8(const void *active, int64_t layer_stride_bytes, int S_act, int L,
                    int n_units, int unit_rows, int dv, const void *table_a,
                    const void *table_b, int R_total, const int32_t *src_slot,
                    const int32_t *dst_slot, int N, const void *codes, const void *scales,
                    int S_ckpt);

// dasc_restore_replay: a checkpoint of whole-head units restored into private
// slots with each request's accepted drafts replayed on the way.
struct RestoreReplayArgs {
    bool q8;               // an INT8 checkpoint (codes + one FP32 scale per row)
    const void *packed;    // FP32 units, or the INT8 codes
    const float *scales;   // INT8: the scales; unused for FP32
    int S_ckpt, R_total;
    const int32_t *unit_pos;
    int L;
    int unit_rows;  // key channels per unit: dk (whole heads) down to 1
    const int32_t *src_slot, *dst_slot;
    int N;
    float *active_out;
    int64_t layer_stride_bytes;
    int S_dst, H, dk, dv, K;
    const void *q, *k, *v;
    int in_dtype;
    const float *alpha;
    int decay;
    const float *beta;
    const int32_t *n_accept;
    void *out;
    int out_dtype;
};

int check_restore_replay(const RestoreReplayArgs &a);

// The INT8 checkpoint restore (arguments validated as dasc_restore_int8's) through the
// fused restore + replay kernel with no tokens, by blocks of 128 rows.  Returns false,
// with nothing launched, when the geometry or the alignment does not fit that kernel.
bool restore_int8_by_blocks(const int8_t *codes, const float *scales, int S_ckpt, int R_total,
                            const int32_t *unit_pos, int L, int n_units, int unit_rows, int dv,
                            const int32_t *src_slot, const int32_t *dst_slot, int N,
                            float *active_out, int64_t layer_stride_bytes, int S_dst,
                            int32_t *err, void *stream);

// log2 of a power of two (checked by the caller).
inline int log2_exact(int x)
{
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

} // namespace hla

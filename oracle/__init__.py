"""Float64 CPU oracle for the gated delta-rule state step (test infrastructure).

Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
import this package.  The HIP library never uses it; the two share no code.
Every routine here is a thin ctypes wrapper around ``oracle.c``, which cites the
passage each function follows.  Array arguments are converted (exactly) to the
C types the functions take: float64 for recurrence values, the stored integer
or FP16 bit patterns for the packed formats.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-fvisibility=hidden", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (plain gcc, no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long


def _declare(L):
    L.orc_gdn_step.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
    L.orc_kda_step.argtypes = L.orc_gdn_step.argtypes
    L.orc_replay.argtypes = [_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P]
    L.orc_verify.argtypes = [_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P]
    L.orc_replay_bonus.argtypes = [_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P,
                                   _P, _P, _P, _P, _P, _P, _P]
    _D = ctypes.c_double
    L.orc_static_horizon.argtypes = [_P, _P, _I, _I, _D, _D, _P]
    L.orc_static_mask.argtypes = [_P, _I, _D, _P]
    L.orc_replay_window.argtypes = [_P, _P, _I, _I, _I, _P]
    L.orc_replay_window.restype = _I
    L.orc_dasc_pack_int8.argtypes = [_P, _L, _I, _I, _I, _I, _P, _P, _I, _P, _P, _I, _P, _P]
    L.orc_dasc_restore_int8.argtypes = [_P, _P, _I, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P,
                                        _L]
    L.orc_dasc_refresh_local.argtypes = [_P, _L, _P, _L, _I, _I, _L, _P, _P, _P, _I]
    L.orc_half_to_double.argtypes = [ctypes.c_uint16]
    L.orc_half_to_double.restype = ctypes.c_double
    L.orc_double_to_half.argtypes = [ctypes.c_double]
    L.orc_double_to_half.restype = ctypes.c_uint16
    L.orc_quantize_row_int8.argtypes = [_P, _I, _P, _P]
    L.orc_damp_quantize.argtypes = [_P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P]
    L.orc_damp_dequantize.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P]
    L.orc_sr_step.argtypes = [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P]
    L.orc_damp_step.argtypes = [_P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _I, _I, _I, _I,
                                _P, _P, _P, _P, _I, _P, _P]
    L.orc_dasc_plan.argtypes = [_P, _I, _I, _P, _P]
    L.orc_dasc_plan.restype = _I
    L.orc_dasc_pack.argtypes = [_P, _L, _I, _I, _I, _L, _P, _P, _I, _P, _P, _I, _P, _I]
    L.orc_dasc_restore.argtypes = [_P, _I, _I, _P, _P, _I, _I, _L, _P, _P, _I, _P, _L, _I]


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _need_f64_inplace(a, name):
    if not (isinstance(a, np.ndarray) and a.dtype == np.float64 and a.flags.c_contiguous):
        raise TypeError(f"{name} must be a C-contiguous float64 array (updated in place)")


def delta_step(state, q, k, v, alpha, beta, *, per_channel, slot=None, want_out=True):
    """One GDN (per_channel=False) or KDA (per_channel=True) step.

    state: float64 [S, H, dk, dv], updated in place.  q, k [B, H, dk]; v [B, H, dv];
    alpha [B, H] or [B, H, dk]; beta [B, H].  Returns out [B, H, dv] (float64);
    rows of skipped requests are NaN.
    """
    _need_f64_inplace(state, "state")
    S, H, dk, dv = state.shape
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B = q.shape[0]
    slot = _i32(slot)
    out = np.full((B, H, dv), np.nan) if want_out else None
    fn = lib().orc_kda_step if per_channel else lib().orc_gdn_step
    fn(_ptr(state), S, _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
       _ptr(beta), _ptr(out))
    return out


def gdn_step(state, q, k, v, alpha, beta, slot=None, want_out=True):
    return delta_step(state, q, k, v, alpha, beta, per_channel=False, slot=slot,
                      want_out=want_out)


def kda_step(state, q, k, v, alpha, beta, slot=None, want_out=True):
    return delta_step(state, q, k, v, alpha, beta, per_channel=True, slot=slot,
                      want_out=want_out)


def replay(state, q, k, v, alpha, beta, n_accept, *, per_channel, slot=None, want_out=True):
    """Advance each request's state by its first n_accept[b] draft tokens.

    q, k [B, K, H, dk]; v [B, K, H, dv]; alpha [B, K, H] or [B, K, H, dk];
    beta [B, K, H].  Returns out [B, K, H, dv] with NaN where t >= n_b.
    """
    _need_f64_inplace(state, "state")
    S, H, dk, dv = state.shape
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, K = q.shape[:2]
    slot = _i32(slot)
    n_accept = _i32(n_accept)
    out = np.full((B, K, H, dv), np.nan) if want_out else None
    lib().orc_replay(_ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k), _ptr(v),
                     _ptr(alpha), int(bool(per_channel)), _ptr(beta), _ptr(n_accept), _ptr(out))
    return out


def verify(state, q, k, v, alpha, beta, *, per_channel, slot=None):
    """Readout at every one of the K draft positions from the committed state advanced
    through the drafts in order; `state` is not changed.  Returns out [B, K, H, dv]
    (NaN for skipped requests)."""
    state = np.ascontiguousarray(state, np.float64)
    S, H, dk, dv = state.shape
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, K = q.shape[:2]
    slot = _i32(slot)
    out = np.full((B, K, H, dv), np.nan)
    lib().orc_verify(_ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k), _ptr(v),
                     _ptr(alpha), int(bool(per_channel)), _ptr(beta), _ptr(out))
    return out


def replay_bonus(state, q, k, v, alpha, beta, n_accept, qb, kb, vb, alpha_b, beta_b, *,
                 per_channel, slot=None, want_out=False):
    """Replay the first n_accept[b] drafts, then apply the bonus token (inputs [B, H, .])
    in place.  Returns (out [B, K, H, dv] or None, out_bonus [B, H, dv])."""
    _need_f64_inplace(state, "state")
    S, H, dk, dv = state.shape
    q, k, v, alpha, beta, qb, kb, vb, alpha_b, beta_b = map(
        _f64, (q, k, v, alpha, beta, qb, kb, vb, alpha_b, beta_b))
    B, K = q.shape[:2]
    slot = _i32(slot)
    n_accept = _i32(n_accept)
    out = np.full((B, K, H, dv), np.nan) if want_out else None
    out_b = np.full((B, H, dv), np.nan)
    lib().orc_replay_bonus(_ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k),
                           _ptr(v), _ptr(alpha), int(bool(per_channel)), _ptr(beta),
                           _ptr(n_accept), _ptr(out), _ptr(qb), _ptr(kb), _ptr(vb),
                           _ptr(alpha_b), _ptr(beta_b), _ptr(out_b))
    return out, out_b


# --------------------------------------------------------------------- FP16

def half_to_double(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    f = lib().orc_half_to_double
    return np.array([f(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


def double_to_half(x):
    x = np.asarray(x, dtype=np.float64)
    f = lib().orc_double_to_half
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def quantize_row_int8(x):
    """Returns (codes int8 [n], scale float32) for one row."""
    x = _f64(x)
    codes = np.zeros(x.shape[0], dtype=np.int8)
    scale = np.zeros(1, dtype=np.float32)
    lib().orc_quantize_row_int8(_ptr(x), x.shape[0], _ptr(codes), _ptr(scale))
    return codes, scale[0]


# --------------------------------------------------------------------- DAMP

def _group(group, dv):
    g = dv if group is None else int(group)
    if g <= 0 or dv % g:
        raise ValueError(f"group {g} must divide dv {dv}")
    return g


def _scale_shape(S, H, dk, dv, K_hi, group):
    """One FP32 scale per INT8 row ([S,H,dk-K_hi]) or per group ([S,H,dk-K_hi,dv/group])."""
    return (S, H, dk - K_hi) if group == dv else (S, H, dk - K_hi, dv // group)


def _sr(val_perm, val_scale):
    vp = None if val_perm is None else _i32(val_perm)
    vs = None if val_scale is None else np.ascontiguousarray(val_scale, np.float32)
    return vp, vs


def damp_alloc(S, H, dk, dv, K_hi, group=None):
    g = _group(group, dv)
    return (np.zeros((S, H, K_hi, dv), np.uint16), np.zeros((S, H, dk - K_hi, dv), np.int8),
            np.zeros(_scale_shape(S, H, dk, dv, K_hi, g), np.float32))


def _group_of(sc, dv):
    return dv if sc.ndim == 3 else dv // sc.shape[3]


def damp_quantize(state, key_perm, K_hi, group=None, val_perm=None, val_scale=None):
    """state S [S,H,dk,dv] in original coordinates -> packed (hi, lo, scale) of the
    transformed state T (value permutation val_perm, stored-order scales val_scale)."""
    state = _f64(state)
    S, H, dk, dv = state.shape
    g = _group(group, dv)
    hi, lo, sc = damp_alloc(S, H, dk, dv, K_hi, g)
    kp = _i32(key_perm)
    vp, vs = _sr(val_perm, val_scale)
    lib().orc_damp_quantize(_ptr(state), S, H, dk, dv, _ptr(kp), K_hi, g, _ptr(vp), _ptr(vs),
                            _ptr(hi), _ptr(lo), _ptr(sc))
    return hi, lo, sc


def damp_dequantize(hi, lo, sc, key_perm, K_hi, dk, val_perm=None, val_scale=None):
    S, H = sc.shape[:2]
    dv = lo.shape[-1] if lo.size else hi.shape[-1]
    g = _group_of(sc, dv)
    hi = np.ascontiguousarray(hi, np.uint16)
    lo = np.ascontiguousarray(lo, np.int8)
    sc = np.ascontiguousarray(sc, np.float32)
    kp = _i32(key_perm)
    vp, vs = _sr(val_perm, val_scale)
    out = np.zeros((S, H, dk, dv), np.float64)
    lib().orc_damp_dequantize(_ptr(hi), _ptr(lo), _ptr(sc), S, H, dk, dv, _ptr(kp), K_hi, g,
                              _ptr(vp), _ptr(vs), _ptr(out))
    return out


def damp_step(hi, lo, sc, key_perm, K_hi, q, k, v, alpha, beta, *, per_channel, slot=None,
              want_out=True, val_perm=None, val_scale=None):
    """One step of the quantised recurrence on the packed state (in place).  The scale
    granularity (per row or per group) is read off the shape of `sc`."""
    for a, dt, nm in ((hi, np.uint16, "hi"), (lo, np.int8, "lo"), (sc, np.float32, "scale")):
        if not (isinstance(a, np.ndarray) and a.dtype == dt and a.flags.c_contiguous):
            raise TypeError(f"{nm} must be a C-contiguous {np.dtype(dt).name} array")
    S, H = sc.shape[:2]
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B, _, dk = q.shape
    dv = v.shape[-1]
    g = _group_of(sc, dv)
    kp = _i32(key_perm)
    vp, vs = _sr(val_perm, val_scale)
    slot = _i32(slot)
    out = np.full((B, H, dv), np.nan) if want_out else None
    lib().orc_damp_step(_ptr(hi), _ptr(lo), _ptr(sc), S, _ptr(kp), K_hi, g, _ptr(vp),
                        _ptr(vs), _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                        _ptr(alpha), int(bool(per_channel)), _ptr(beta), _ptr(out))
    return out


def sr_step(state, q, k, v, alpha, beta, *, per_channel, val_perm=None, val_scale=None,
            slot=None, want_out=True):
    """Float64 transformed step ([DAMP] App. A.3 Eq. (18)) on T, in place, no quantisation."""
    _need_f64_inplace(state, "state")
    S, H, dk, dv = state.shape
    q, k, v, alpha, beta = map(_f64, (q, k, v, alpha, beta))
    B = q.shape[0]
    vp, vs = _sr(val_perm, val_scale)
    slot = _i32(slot)
    out = np.full((B, H, dv), np.nan) if want_out else None
    lib().orc_sr_step(_ptr(state), S, _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                      _ptr(alpha), int(bool(per_channel)), _ptr(beta), _ptr(vp), _ptr(vs),
                      _ptr(out))
    return out


# --------------------------------------------------------------------- dasc

def dasc_plan(mask):
    """mask uint8 [L, n_units] -> (offsets int32 [L+1], unit_index int32 [R_total])."""
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    L, n = mask.shape
    offsets = np.zeros(L + 1, np.int32)
    idx = np.zeros(max(1, L * n), np.int32)
    R = lib().orc_dasc_plan(_ptr(mask), L, n, _ptr(offsets), _ptr(idx))
    return offsets, idx[:R].copy()


def dasc_pack(active, offsets, unit_index, src_slot, dst_slot, S_ckpt):
    """active uint8 [L, S_act, n_units, unit_bytes] -> packed [S_ckpt, R_total, unit_bytes]
    (slots not named in dst_slot stay zero)."""
    active = np.ascontiguousarray(active, np.uint8)
    L, S_act, n_units, ub = active.shape
    offsets, unit_index = _i32(offsets), _i32(unit_index)
    R = int(offsets[-1])
    src, dst = _i32(src_slot), _i32(dst_slot)
    packed = np.zeros((S_ckpt, R, ub), np.uint8)
    lib().orc_dasc_pack(_ptr(active), S_act * n_units * ub, S_act, L, n_units, ub,
                        _ptr(offsets), _ptr(unit_index), R, _ptr(src), _ptr(dst), len(src),
                        _ptr(packed), S_ckpt)
    return packed


def dasc_restore(packed, offsets, unit_index, L, n_units, src_slot, dst_slot, active_out):
    """Restore into active_out uint8 [L, S_dst, n_units, unit_bytes] (in place)."""
    if not (isinstance(active_out, np.ndarray) and active_out.dtype == np.uint8
            and active_out.flags.c_contiguous):
        raise TypeError("active_out must be a C-contiguous uint8 array")
    packed = np.ascontiguousarray(packed, np.uint8)
    S_ckpt, R, ub = packed.shape
    _, S_dst, n_u, ub2 = active_out.shape
    assert n_u == n_units and ub2 == ub
    offsets, unit_index = _i32(offsets), _i32(unit_index)
    src, dst = _i32(src_slot), _i32(dst_slot)
    lib().orc_dasc_restore(_ptr(packed), S_ckpt, R, _ptr(offsets), _ptr(unit_index), L,
                           n_units, ub, _ptr(src), _ptr(dst), len(src), _ptr(active_out),
                           S_dst * n_units * ub, S_dst)
    return active_out


# --------------------------------------------------------------------- horizons

GATE_SOFTPLUS, GATE_BOUNDED = 0, 1


def static_horizon(A_log, d, gate, a_s, eps=1e-3):
    """Static retention horizon H per unit (dasc Eq. (2)-(3)); arrays of any shape."""
    A_log, d = _f64(A_log), _f64(d)
    H = np.zeros(A_log.shape, np.float64)
    lib().orc_static_horizon(_ptr(A_log), _ptr(d), A_log.size, int(gate), float(a_s),
                             float(eps), _ptr(H))
    return H


def static_mask(H, W_max):
    """uint8 mask, 1 where the unit is global (H > W_max)."""
    H = _f64(H)
    m = np.zeros(H.shape, np.uint8)
    lib().orc_static_mask(_ptr(H), H.size, float(W_max), _ptr(m))
    return m


def replay_window(H, mask, n_prefix, W_max):
    """(W_replay, W_u int32 per unit) of dasc Eq. (7)."""
    H = _f64(H)
    mask = np.ascontiguousarray(mask, np.uint8)
    W_u = np.zeros(H.shape, np.int32)
    w = lib().orc_replay_window(_ptr(H), _ptr(mask), H.size, int(n_prefix), int(W_max),
                                _ptr(W_u))
    return int(w), W_u


# --------------------------------------------------------------------- INT8 checkpoints

def dasc_pack_int8(active, offsets, unit_index, src_slot, dst_slot, S_ckpt):
    """active float32 [L, S_act, n_units, unit_rows, dv] -> (codes int8
    [S_ckpt, R, unit_rows, dv], scales float32 [S_ckpt, R, unit_rows]); rows of
    checkpoint slots no pair names are zero."""
    active = np.ascontiguousarray(active, np.float32)
    L, S_act, n_units, unit_rows, dv = active.shape
    R = int(offsets[-1])
    codes = np.zeros((S_ckpt, R, unit_rows, dv), np.int8)
    scales = np.zeros((S_ckpt, R, unit_rows), np.float32)
    offsets, unit_index = _i32(offsets), _i32(unit_index)
    src_slot, dst_slot = _i32(src_slot), _i32(dst_slot)
    lib().orc_dasc_pack_int8(_ptr(active), S_act * n_units * unit_rows * dv * 4, L, n_units,
                             unit_rows, dv, _ptr(offsets), _ptr(unit_index), R, _ptr(src_slot),
                             _ptr(dst_slot), len(src_slot), _ptr(codes), _ptr(scales))
    return codes, scales


def dasc_restore_int8(codes, scales, offsets, unit_index, L, n_units, src_slot, dst_slot,
                      active_out):
    """Dequantise into active_out float32 [L, S_dst, n_units, unit_rows, dv] (in place)."""
    if not (active_out.dtype == np.float32 and active_out.flags.c_contiguous):
        raise TypeError("active_out must be C-contiguous float32")
    _, S_dst, _, unit_rows, dv = active_out.shape
    codes = np.ascontiguousarray(codes, np.int8)
    scales = np.ascontiguousarray(scales, np.float32)
    R = codes.shape[1]
    offsets, unit_index = _i32(offsets), _i32(unit_index)
    src_slot, dst_slot = _i32(src_slot), _i32(dst_slot)
    lib().orc_dasc_restore_int8(_ptr(codes), _ptr(scales), R, _ptr(offsets), _ptr(unit_index),
                                L, n_units, unit_rows, dv, _ptr(src_slot), _ptr(dst_slot),
                                len(src_slot), _ptr(active_out),
                                S_dst * n_units * unit_rows * dv * 4)
    return active_out


def dasc_refresh_local(scratch, active, local, src_slot, dst_slot):
    """Copy the local units (local uint8 [L, n_units] == 1) of scratch slots into active
    slots, in place; both uint8 [L, S, n_units, unit_bytes]."""
    scratch = np.ascontiguousarray(scratch, np.uint8)
    if not (active.dtype == np.uint8 and active.flags.c_contiguous):
        raise TypeError("active must be C-contiguous uint8")
    L, S_s, n_units, ub = scratch.shape
    S_a = active.shape[1]
    local = np.ascontiguousarray(local, np.uint8)
    src_slot, dst_slot = _i32(src_slot), _i32(dst_slot)
    lib().orc_dasc_refresh_local(_ptr(scratch), S_s * n_units * ub, _ptr(active),
                                 S_a * n_units * ub, L, n_units, ub, _ptr(local),
                                 _ptr(src_slot), _ptr(dst_slot), len(src_slot))
    return active


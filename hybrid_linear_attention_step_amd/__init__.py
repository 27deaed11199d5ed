"""Python binding of libhla.so, the gfx950 HIP library declared in include/hla.h.

Argument marshalling only: every function here checks tensor dtypes, devices and
shapes, passes raw device pointers, sizes and the current HIP stream to the C
entry point of the same name, and raises on a non-zero status.  All arithmetic
runs in the library's kernels.  There is no CPU fallback: if libhla.so is not
built, every call raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

from ._build import LIB as LIB_PATH

HLA_F32, HLA_BF16, HLA_F16 = 0, 1, 2
DECAY_SCALAR, DECAY_VECTOR = 0, 1
DEVERR_SLOT, DEVERR_ACCEPT, DEVERR_PLAN = 1, 2, 4

# ctypes signature of every entry point in include/hla.h
_P, _I, _L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
SIGNATURES = {
    "hla_status_str": ([_I], ctypes.c_char_p),
    "hla_version": ([], _I),
    "gdn_step": ([_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _I, _P, _P], _I),
    "kda_step": ([_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _I, _P, _P], _I),
    "damp_step": ([_P, _P, _P, _I, _P, _I, _I, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I, _P,
                   _I, _P, _P, _I, _P, _P], _I),
    "damp_quantize": ([_P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P], _I),
    "damp_dequantize": ([_P, _P, _P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P], _I),
    "dasc_plan": ([_P, _I, _I, _P, _P, _I, _P, _P], _I),
    "dasc_pack": ([_P, _L, _I, _I, _I, _L, _P, _P, _I, _P, _P, _I, _P, _I, _P, _P], _I),
    "dasc_restore": ([_P, _I, _I, _P, _I, _I, _L, _P, _P, _I, _P, _L, _I, _P, _P], _I),
    "dasc_pack_int8": ([_P, _L, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _I, _P, _P, _I, _P, _P],
                       _I),
    "dasc_restore_int8": ([_P, _P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _I, _P, _L, _I, _P, _P],
                          _I),
    "dasc_static_horizon": ([_P, _P, _I, _I, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                             _P, _P], _I),
    "dasc_replay_window": ([_P, _P, _I, _I, _I, _P, _P], _I),
    "dasc_refresh_local": ([_P, _L, _I, _P, _L, _I, _I, _I, _L, _P, _P, _I, _P, _P, _I, _P, _P],
                           _I),
    "replay_accepted": ([_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, _P, _I,
                         _P, _P], _I),
    "replay_accepted_bonus": ([_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P,
                               _P, _P, _P, _P, _P, _P, _P, _I, _P, _P], _I),
    "verify_drafts": ([_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, _I, _P,
                       _P], _I),
}


class HLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhla.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().hla_status_str(status).decode()


def _call(name: str, *args) -> None:
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise HLAError(name, rc)


# ------------------------------------------------------------------ marshalling

def _torch():
    import torch

    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")
    return t


def _code(dtype) -> int:
    torch = _torch()
    return {torch.float32: HLA_F32, torch.bfloat16: HLA_BF16, torch.float16: HLA_F16}[dtype]


def _in_dtypes():
    torch = _torch()
    return (torch.float32, torch.bfloat16, torch.float16)


def _i32():
    return (_torch().int32,)


def _f32():
    return (_torch().float32,)


def _opt_out(out, shape, device, want_out):
    torch = _torch()
    if out is None and want_out:
        out = torch.empty(shape, dtype=torch.float32, device=device)
    if out is not None:
        _dev(out, "out", _in_dtypes(), len(shape))
    return out


def _step(name, state, q, k, v, alpha, beta, out, slot, err_flag, stream, want_out):
    _dev(state, "state", _f32(), 4)
    S, H, dk, dv = state.shape
    _dev(q, "q", _in_dtypes(), 3)
    B = q.shape[0]
    _dev(k, "k", (q.dtype,), 3)
    _dev(v, "v", (q.dtype,), 3)
    _dev(alpha, "alpha", _f32())
    _dev(beta, "beta", _f32(), 2)
    if slot is not None:
        _dev(slot, "slot", _i32(), 1)
    if err_flag is not None:
        _dev(err_flag, "err_flag", _i32())
    out = _opt_out(out, (B, H, dv), state.device, want_out)
    _call(name, _ptr(state), S, _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
          _code(q.dtype), _ptr(alpha), _ptr(beta), _ptr(out),
          _code(out.dtype) if out is not None else HLA_F32, _ptr(err_flag), _stream(stream))
    return out


def gdn_step(state, q, k, v, alpha, beta, out=None, slot=None, err_flag=None, stream=None,
             want_out=True):
    """GDN decode step in place on `state` [S,H,dk,dv] fp32; returns o [B,H,dv]."""
    return _step("gdn_step", state, q, k, v, alpha, beta, out, slot, err_flag, stream, want_out)


def kda_step(state, q, k, v, alpha, beta, out=None, slot=None, err_flag=None, stream=None,
             want_out=True):
    """KDA decode step (alpha [B,H,dk]) in place on `state`; returns o [B,H,dv]."""
    return _step("kda_step", state, q, k, v, alpha, beta, out, slot, err_flag, stream, want_out)


def replay_accepted(state, q, k, v, alpha, beta, n_accept, decay_kind, out=None, slot=None,
                    err_flag=None, stream=None, want_out=True):
    """Replay the first n_accept[b] of K cached draft projections into each state."""
    _dev(state, "state", _f32(), 4)
    S, H, dk, dv = state.shape
    _dev(q, "q", _in_dtypes(), 4)
    B, K = q.shape[:2]
    _dev(k, "k", (q.dtype,), 4)
    _dev(v, "v", (q.dtype,), 4)
    _dev(alpha, "alpha", _f32())
    _dev(beta, "beta", _f32(), 3)
    _dev(n_accept, "n_accept", _i32(), 1)
    if slot is not None:
        _dev(slot, "slot", _i32(), 1)
    if err_flag is not None:
        _dev(err_flag, "err_flag", _i32())
    out = _opt_out(out, (B, K, H, dv), state.device, want_out)
    _call("replay_accepted", _ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k),
          _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta), _ptr(n_accept),
          _ptr(out), _code(out.dtype) if out is not None else HLA_F32, _ptr(err_flag),
          _stream(stream))
    return out


def _drafts(state, q, k, v, alpha, beta, slot, err_flag):
    """Shared checks of the multi-token entry points; returns (S, H, dk, dv, B, K)."""
    _dev(state, "state", _f32(), 4)
    S, H, dk, dv = state.shape
    _dev(q, "q", _in_dtypes(), 4)
    B, K = q.shape[:2]
    _dev(k, "k", (q.dtype,), 4)
    _dev(v, "v", (q.dtype,), 4)
    _dev(alpha, "alpha", _f32())
    _dev(beta, "beta", _f32(), 3)
    if slot is not None:
        _dev(slot, "slot", _i32(), 1)
    if err_flag is not None:
        _dev(err_flag, "err_flag", _i32())
    return S, H, dk, dv, B, K


def replay_accepted_bonus(state, q, k, v, alpha, beta, n_accept, decay_kind, q_bonus, k_bonus,
                          v_bonus, alpha_bonus, beta_bonus, out=None, out_bonus=None, slot=None,
                          err_flag=None, stream=None, want_out_bonus=True):
    """Replay the first n_accept[b] drafts, then the bonus token ([B, H, .] inputs), in one
    pass over the state.  Returns the bonus token's readout [B, H, dv] (or None)."""
    S, H, dk, dv, B, K = _drafts(state, q, k, v, alpha, beta, slot, err_flag)
    _dev(n_accept, "n_accept", _i32(), 1)
    _dev(q_bonus, "q_bonus", (q.dtype,), 3)
    _dev(k_bonus, "k_bonus", (q.dtype,), 3)
    _dev(v_bonus, "v_bonus", (q.dtype,), 3)
    _dev(alpha_bonus, "alpha_bonus", _f32())
    _dev(beta_bonus, "beta_bonus", _f32(), 2)
    if out is not None:
        _dev(out, "out", _in_dtypes(), 4)
    out_bonus = _opt_out(out_bonus, (B, H, dv), state.device, want_out_bonus)
    if out is not None and out_bonus is not None and out.dtype != out_bonus.dtype:
        raise TypeError("out and out_bonus must have the same dtype")
    od = out_bonus if out_bonus is not None else out
    _call("replay_accepted_bonus", _ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q),
          _ptr(k), _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta),
          _ptr(n_accept), _ptr(out), _ptr(q_bonus), _ptr(k_bonus), _ptr(v_bonus),
          _ptr(alpha_bonus), _ptr(beta_bonus), _ptr(out_bonus),
          _code(od.dtype) if od is not None else HLA_F32, _ptr(err_flag), _stream(stream))
    return out_bonus


def verify_drafts(state, q, k, v, alpha, beta, decay_kind, out=None, slot=None, err_flag=None,
                  stream=None):
    """Readouts at all K draft positions from the committed state (which is only read).
    Returns out [B, K, H, dv]."""
    S, H, dk, dv, B, K = _drafts(state, q, k, v, alpha, beta, slot, err_flag)
    out = _opt_out(out, (B, K, H, dv), state.device, True)
    _call("verify_drafts", _ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k),
          _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta), _ptr(out),
          _code(out.dtype), _ptr(err_flag), _stream(stream))
    return out


def _damp_group(lo_scale, dv):
    """Scale granularity from the scale tensor's shape: [S,H,rows] per row,
    [S,H,rows,dv/group] per group."""
    if lo_scale.dim() == 3:
        return dv
    if lo_scale.dim() == 4 and lo_scale.shape[3] > 0 and dv % lo_scale.shape[3] == 0:
        return dv // lo_scale.shape[3]
    raise ValueError(f"lo_scale shape {tuple(lo_scale.shape)} fits no scale group of dv={dv}")


def _sr_tables(val_perm, val_scale):
    if val_perm is not None:
        _dev(val_perm, "val_perm", _i32(), 2)
    if val_scale is not None:
        _dev(val_scale, "val_scale", _f32(), 2)


def damp_step(hi, lo, lo_scale, key_perm, K_hi, q, k, v, alpha, decay_kind, beta, out=None,
              slot=None, err_flag=None, stream=None, want_out=True, val_perm=None,
              val_scale=None):
    """One fused dequantise -> update -> requantise step on the packed state (in place).
    The scale group (per row or per 32 values) is read off lo_scale's shape; val_perm /
    val_scale [H, dv] select the value transform (None: untransformed)."""
    torch = _torch()
    _dev(hi, "hi", (torch.int16, torch.uint16, torch.float16), 4)
    _dev(lo, "lo", (torch.int8,), 4)
    _dev(lo_scale, "lo_scale", _f32())
    S, H, _, dv = hi.shape
    group = _damp_group(lo_scale, dv)
    _dev(q, "q", _in_dtypes(), 3)
    B, _, dk = q.shape
    _dev(k, "k", (q.dtype,), 3)
    _dev(v, "v", (q.dtype,), 3)
    _dev(alpha, "alpha", _f32())
    _dev(beta, "beta", _f32(), 2)
    if key_perm is not None:
        _dev(key_perm, "key_perm", _i32(), 2)
    _sr_tables(val_perm, val_scale)
    if slot is not None:
        _dev(slot, "slot", _i32(), 1)
    if err_flag is not None:
        _dev(err_flag, "err_flag", _i32())
    if lo.shape[2] != dk - K_hi or hi.shape[2] != K_hi:
        raise ValueError("hi/lo row counts do not match K_hi and dk")
    out = _opt_out(out, (B, H, dv), hi.device, want_out)
    _call("damp_step", _ptr(hi), _ptr(lo), _ptr(lo_scale), S, _ptr(key_perm), K_hi, group,
          _ptr(val_perm), _ptr(val_scale), _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
          _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta), _ptr(out),
          _code(out.dtype) if out is not None else HLA_F32, _ptr(err_flag), _stream(stream))
    return out


def damp_alloc(S, H, dk, dv, K_hi, device="cuda", group=None):
    """Empty packed state; group None or dv: one scale per INT8 row, else per `group`."""
    torch = _torch()
    g = dv if group is None else int(group)
    sc_shape = (S, H, dk - K_hi) if g == dv else (S, H, dk - K_hi, dv // g)
    return (torch.empty((S, H, K_hi, dv), dtype=torch.int16, device=device),
            torch.empty((S, H, dk - K_hi, dv), dtype=torch.int8, device=device),
            torch.empty(sc_shape, dtype=torch.float32, device=device))


def damp_quantize(state, key_perm, K_hi, hi=None, lo=None, lo_scale=None, stream=None,
                  group=None, val_perm=None, val_scale=None):
    _dev(state, "state", _f32(), 4)
    S, H, dk, dv = state.shape
    if hi is None:
        hi, lo, lo_scale = damp_alloc(S, H, dk, dv, K_hi, state.device, group)
    g = _damp_group(lo_scale, dv)
    if group is not None and int(group) != g:
        raise ValueError("lo_scale shape does not match group")
    if key_perm is not None:
        _dev(key_perm, "key_perm", _i32(), 2)
    _sr_tables(val_perm, val_scale)
    _call("damp_quantize", _ptr(state), S, H, dk, dv, _ptr(key_perm), K_hi, g, _ptr(val_perm),
          _ptr(val_scale), _ptr(hi), _ptr(lo), _ptr(lo_scale), _stream(stream))
    return hi, lo, lo_scale


def damp_dequantize(hi, lo, lo_scale, key_perm, K_hi, dk, out=None, stream=None,
                    val_perm=None, val_scale=None):
    torch = _torch()
    S, H, _, dv = hi.shape
    g = _damp_group(lo_scale, dv)
    if out is None:
        out = torch.empty((S, H, dk, dv), dtype=torch.float32, device=hi.device)
    _dev(out, "state", _f32(), 4)
    if key_perm is not None:
        _dev(key_perm, "key_perm", _i32(), 2)
    _sr_tables(val_perm, val_scale)
    _call("damp_dequantize", _ptr(hi), _ptr(lo), _ptr(lo_scale), S, H, dk, dv, _ptr(key_perm),
          K_hi, g, _ptr(val_perm), _ptr(val_scale), _ptr(out), _stream(stream))
    return out


def dasc_plan(mask):
    """Host plan from a uint8 numpy mask [L, n_units]: (offsets, unit_index, unit_pos, R_total)
    as numpy int32 arrays."""
    import numpy as np

    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    L, n = mask.shape
    offsets = np.zeros(L + 1, np.int32)
    unit_index = np.zeros(max(1, L * n), np.int32)
    unit_pos = np.zeros(L * n, np.int32)
    R = ctypes.c_int32(0)
    _call("dasc_plan", mask.ctypes.data, L, n, offsets.ctypes.data, unit_index.ctypes.data,
          unit_index.size, unit_pos.ctypes.data, ctypes.byref(R))
    return offsets, unit_index[:R.value].copy(), unit_pos.reshape(L, n), R.value


def dasc_pack(active, layer_stride_bytes, S_act, L, n_units, unit_bytes, offsets, unit_index,
              R_total, src_slot, dst_slot, packed, S_ckpt, err_flag=None, stream=None):
    """Byte-level pack; `active` and `packed` are device tensors (any dtype)."""
    for t, nm in ((offsets, "offsets"), (src_slot, "src_slot"), (dst_slot, "dst_slot")):
        _dev(t, nm, _i32(), 1)
    _call("dasc_pack", _ptr(active), int(layer_stride_bytes), S_act, L, n_units, int(unit_bytes),
          _ptr(offsets), _ptr(unit_index) if unit_index.numel() else None, R_total,
          _ptr(src_slot), _ptr(dst_slot), src_slot.numel(), _ptr(packed), S_ckpt,
          _ptr(err_flag), _stream(stream))


def dasc_restore(packed, S_ckpt, R_total, unit_pos, L, n_units, unit_bytes, src_slot, dst_slot,
                 active_out, layer_stride_bytes, S_dst, err_flag=None, stream=None):
    for t, nm in ((src_slot, "src_slot"), (dst_slot, "dst_slot")):
        _dev(t, nm, _i32(), 1)
    _dev(unit_pos, "unit_pos", _i32())
    _call("dasc_restore", _ptr(packed), S_ckpt, R_total, _ptr(unit_pos), L, n_units,
          int(unit_bytes), _ptr(src_slot), _ptr(dst_slot), src_slot.numel(), _ptr(active_out),
          int(layer_stride_bytes), S_dst, _ptr(err_flag), _stream(stream))


def dasc_pack_int8(active, layer_stride_bytes, S_act, L, n_units, unit_rows, dv, offsets,
                   unit_index, R_total, src_slot, dst_slot, codes, scales, S_ckpt, err_flag=None,
                   stream=None):
    """Quantise-once pack of the retained units of an FP32 state into (codes, scales)."""
    for t, nm in ((offsets, "offsets"), (src_slot, "src_slot"), (dst_slot, "dst_slot")):
        _dev(t, nm, _i32(), 1)
    torch = _torch()
    _dev(codes, "codes", (torch.int8,))
    _dev(scales, "scales", _f32())
    _call("dasc_pack_int8", _ptr(active), int(layer_stride_bytes), S_act, L, n_units, unit_rows,
          dv, _ptr(offsets), _ptr(unit_index) if unit_index.numel() else None, R_total,
          _ptr(src_slot), _ptr(dst_slot), src_slot.numel(), _ptr(codes), _ptr(scales), S_ckpt,
          _ptr(err_flag), _stream(stream))


def dasc_restore_int8(codes, scales, S_ckpt, R_total, unit_pos, L, n_units, unit_rows, dv,
                      src_slot, dst_slot, active_out, layer_stride_bytes, S_dst, err_flag=None,
                      stream=None):
    """Dequantise-once restore into FP32 active slots, omitted units zero."""
    for t, nm in ((src_slot, "src_slot"), (dst_slot, "dst_slot")):
        _dev(t, nm, _i32(), 1)
    _dev(unit_pos, "unit_pos", _i32())
    _dev(active_out, "active_out", _f32())
    _call("dasc_restore_int8", _ptr(codes), _ptr(scales), S_ckpt, R_total, _ptr(unit_pos), L,
          n_units, unit_rows, dv, _ptr(src_slot), _ptr(dst_slot), src_slot.numel(),
          _ptr(active_out), int(layer_stride_bytes), S_dst, _ptr(err_flag), _stream(stream))


GATE_SOFTPLUS, GATE_BOUNDED = 0, 1


def dasc_static_horizon(A_log, d, gate, a_s, W_max, eps=1e-3):
    """Host: static horizons (float64) and the selection mask (uint8) of numpy float32
    gate parameters of any shape."""
    import numpy as np

    A_log = np.ascontiguousarray(A_log, np.float32)
    d = np.ascontiguousarray(d, np.float32)
    if A_log.shape != d.shape:
        raise ValueError("A_log and d must have the same shape")
    H = np.zeros(A_log.shape, np.float64)
    mask = np.zeros(A_log.shape, np.uint8)
    _call("dasc_static_horizon", A_log.ctypes.data, d.ctypes.data, A_log.size, int(gate),
          float(a_s), float(eps), float(W_max), H.ctypes.data, mask.ctypes.data)
    return H, mask


def dasc_replay_window(H, mask, n_prefix, W_max):
    """Host: (W_replay, W_u int32) of the dasc-wr refresh window."""
    import numpy as np

    H = np.ascontiguousarray(H, np.float64)
    mask = np.ascontiguousarray(mask, np.uint8)
    W_u = np.zeros(H.shape, np.int32)
    W = ctypes.c_int32(0)
    _call("dasc_replay_window", H.ctypes.data, mask.ctypes.data, H.size, int(n_prefix),
          int(W_max), W_u.ctypes.data, ctypes.byref(W))
    return W.value, W_u


def dasc_refresh_local(scratch, scratch_layer_stride_bytes, S_scratch, active,
                       layer_stride_bytes, S_act, L, n_units, unit_bytes, offsets_local,
                       unit_index_local, R_local, src_slot, dst_slot, err_flag=None,
                       stream=None):
    """Copy the local units (plan of the inverted mask) from scratch slots into active
    slots; everything else in the active slots is left alone."""
    for t, nm in ((offsets_local, "offsets"), (src_slot, "src_slot"), (dst_slot, "dst_slot")):
        _dev(t, nm, _i32(), 1)
    _call("dasc_refresh_local", _ptr(scratch), int(scratch_layer_stride_bytes), S_scratch,
          _ptr(active), int(layer_stride_bytes), S_act, L, n_units, int(unit_bytes),
          _ptr(offsets_local), _ptr(unit_index_local) if unit_index_local.numel() else None,
          R_local, _ptr(src_slot), _ptr(dst_slot), src_slot.numel(), _ptr(err_flag),
          _stream(stream))


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
    "dasc_restore_replay": ([_P, _I, _I, _P, _I, _I, _P, _P, _I, _P, _L, _I, _I, _I, _I, _I,
                             _P, _P, _P, _I, _P, _I, _P, _P, _P, _I, _P, _P], _I),
    "dasc_restore_int8_replay": ([_P, _P, _I, _I, _P, _I, _I, _P, _P, _I, _P, _L, _I, _I, _I, _I,
                                  _I, _P, _P, _P, _I, _P, _I, _P, _P, _P, _I, _P, _P], _I),
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


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _in_dtypes():
    torch = _torch()
    return (torch.float32, torch.bfloat16, torch.float16)


def _i32():
    return (_torch().int32,)


def _f32():
    return (_torch().float32,)


def _code(dtype) -> int:
    torch = _torch()
    return {torch.float32: HLA_F32, torch.bfloat16: HLA_BF16, torch.float16: HLA_F16}[dtype]


class _Args:
    """The tensor arguments of one call, checked before anything reaches the library.

    Element type, contiguity and the full shape (or, for byte-level buffers, the size)
    are checked as each tensor is added; devices are checked together by on_gpu() once
    every shape has passed, so that a mis-shaped tensor is reported as such whatever
    device it is on.  The library sizes every access from the sizes it is given, so a
    tensor smaller than those sizes, or one in host memory, would be read or written out
    of bounds by a kernel: both are refused here."""

    def __init__(self, fn: str):
        self.fn = fn
        self.ts = []

    def _fail(self, exc, msg):
        raise exc(f"{self.fn}: {msg}")

    def t(self, x, name, dtypes=None, shape=None, ndim=None, optional=False):
        """A tensor of one of `dtypes` (None: any), contiguous, of exactly `shape` (None
        entries match any size) or with `ndim` dimensions.  Returns x (None when optional
        and absent)."""
        torch = _torch()
        if x is None:
            if optional:
                return None
            self._fail(ValueError, f"{name} is required")
        if not isinstance(x, torch.Tensor):
            self._fail(TypeError, f"{name}: expected a torch.Tensor, got {type(x).__name__}")
        if dtypes is not None and x.dtype not in dtypes:
            self._fail(TypeError, f"{name}: dtype {x.dtype} not in {dtypes}")
        if not x.is_contiguous():
            self._fail(ValueError, f"{name}: must be contiguous")
        if shape is not None:
            ndim = len(shape)
        if ndim is not None and x.dim() != ndim:
            self._fail(ValueError, f"{name}: expected {ndim} dimensions, got shape "
                                   f"{tuple(x.shape)}")
        if shape is not None and any(e is not None and int(e) != int(g)
                                     for e, g in zip(shape, x.shape)):
            want = tuple("*" if e is None else int(e) for e in shape)
            self._fail(ValueError, f"{name}: expected shape {want}, got {tuple(x.shape)}")
        self.ts.append((name, x))
        return x

    def nbytes(self, x, name, need, dtypes=None, optional=False):
        """A contiguous buffer of at least `need` bytes (any shape)."""
        x = self.t(x, name, dtypes, optional=optional)
        if x is not None and need > 0 and x.numel() * x.element_size() < need:
            self._fail(ValueError, f"{name}: {x.numel() * x.element_size()} bytes, the call "
                                   f"addresses {need}")
        return x

    def flag(self, x):
        """The optional device error flag: int32, at least one element."""
        x = self.t(x, "err_flag", _i32(), optional=True)
        if x is not None and x.numel() < 1:
            self._fail(ValueError, "err_flag: needs one int32 element")
        return x

    def on_gpu(self, stream=None):
        """Every tensor on one GPU, the one the launch stream belongs to."""
        torch = _torch()
        for name, x in self.ts:
            if x.device.type != "cuda":
                self._fail(ValueError, f"{name}: must be a GPU tensor, got {x.device}")
        devs = {x.device for _, x in self.ts}
        if len(devs) > 1:
            self._fail(ValueError, f"tensors on several devices: {sorted(map(str, devs))}")
        if devs:
            d = next(iter(devs))
            sd = (stream.device if stream is not None
                  else torch.device("cuda", torch.cuda.current_device()))
            if d != sd:
                self._fail(ValueError, f"tensors on {d}, launch stream on {sd}")

    def stream(self, stream):
        self.on_gpu(stream)
        if stream is None:
            stream = _torch().cuda.current_stream()
        return ctypes.c_void_p(stream.cuda_stream)


def _alpha_shape(lead, decay_kind, dk):
    """Decay shape: one scalar per head, or one per key channel; None (left to the library,
    which refuses the code) for an unknown decay kind."""
    if decay_kind == DECAY_SCALAR:
        return lead
    if decay_kind == DECAY_VECTOR:
        return lead + (dk,)
    return None


def _decay_arg(a, x, name, lead, decay_kind, dk):
    shape = _alpha_shape(lead, decay_kind, dk)
    return a.t(x, name, _f32(), shape=shape) if shape is not None else a.t(x, name, _f32())


def _new_out(out, shape, like):
    if out is None:
        out = _torch().empty(shape, dtype=_torch().float32, device=like.device)
    return out


def _step(name, decay_kind, state, q, k, v, alpha, beta, out, slot, err_flag, stream,
          want_out):
    a = _Args(name)
    a.t(state, "state", _f32(), ndim=4)
    S, H, dk, dv = state.shape
    a.t(q, "q", _in_dtypes(), shape=(None, H, dk))
    B = q.shape[0]
    a.t(k, "k", (q.dtype,), shape=(B, H, dk))
    a.t(v, "v", (q.dtype,), shape=(B, H, dv))
    _decay_arg(a, alpha, "alpha", (B, H), decay_kind, dk)
    a.t(beta, "beta", _f32(), shape=(B, H))
    a.t(slot, "slot", _i32(), shape=(B,), optional=True)
    a.flag(err_flag)
    a.t(out, "out", _in_dtypes(), shape=(B, H, dv), optional=True)
    st = a.stream(stream)
    if want_out:
        out = _new_out(out, (B, H, dv), state)
    _call(name, _ptr(state), S, _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
          _code(q.dtype), _ptr(alpha), _ptr(beta), _ptr(out),
          _code(out.dtype) if out is not None else HLA_F32, _ptr(err_flag), st)
    return out


def gdn_step(state, q, k, v, alpha, beta, out=None, slot=None, err_flag=None, stream=None,
             want_out=True):
    """GDN decode step in place on `state` [S,H,dk,dv] fp32 (alpha [B,H]); returns o
    [B,H,dv]."""
    return _step("gdn_step", DECAY_SCALAR, state, q, k, v, alpha, beta, out, slot, err_flag,
                 stream, want_out)


def kda_step(state, q, k, v, alpha, beta, out=None, slot=None, err_flag=None, stream=None,
             want_out=True):
    """KDA decode step (alpha [B,H,dk]) in place on `state`; returns o [B,H,dv]."""
    return _step("kda_step", DECAY_VECTOR, state, q, k, v, alpha, beta, out, slot, err_flag,
                 stream, want_out)


def _drafts(a, state, q, k, v, alpha, beta, decay_kind, slot, err_flag):
    """Shared checks of the multi-token entry points; returns (S, H, dk, dv, B, K)."""
    a.t(state, "state", _f32(), ndim=4)
    S, H, dk, dv = state.shape
    a.t(q, "q", _in_dtypes(), shape=(None, None, H, dk))
    B, K = q.shape[:2]
    a.t(k, "k", (q.dtype,), shape=(B, K, H, dk))
    a.t(v, "v", (q.dtype,), shape=(B, K, H, dv))
    _decay_arg(a, alpha, "alpha", (B, K, H), decay_kind, dk)
    a.t(beta, "beta", _f32(), shape=(B, K, H))
    a.t(slot, "slot", _i32(), shape=(B,), optional=True)
    a.flag(err_flag)
    return S, H, dk, dv, B, K


def replay_accepted(state, q, k, v, alpha, beta, n_accept, decay_kind, out=None, slot=None,
                    err_flag=None, stream=None, want_out=True):
    """Replay the first n_accept[b] of K cached draft projections into each state."""
    a = _Args("replay_accepted")
    S, H, dk, dv, B, K = _drafts(a, state, q, k, v, alpha, beta, decay_kind, slot, err_flag)
    a.t(n_accept, "n_accept", _i32(), shape=(B,))
    a.t(out, "out", _in_dtypes(), shape=(B, K, H, dv), optional=True)
    st = a.stream(stream)
    if want_out:
        out = _new_out(out, (B, K, H, dv), state)
    _call("replay_accepted", _ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k),
          _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta), _ptr(n_accept),
          _ptr(out), _code(out.dtype) if out is not None else HLA_F32, _ptr(err_flag), st)
    return out


def replay_accepted_bonus(state, q, k, v, alpha, beta, n_accept, decay_kind, q_bonus, k_bonus,
                          v_bonus, alpha_bonus, beta_bonus, out=None, out_bonus=None, slot=None,
                          err_flag=None, stream=None, want_out_bonus=True):
    """Replay the first n_accept[b] drafts, then the bonus token ([B, H, .] inputs), in one
    pass over the state.  Returns the bonus token's readout [B, H, dv] (or None)."""
    a = _Args("replay_accepted_bonus")
    S, H, dk, dv, B, K = _drafts(a, state, q, k, v, alpha, beta, decay_kind, slot, err_flag)
    a.t(n_accept, "n_accept", _i32(), shape=(B,))
    a.t(q_bonus, "q_bonus", (q.dtype,), shape=(B, H, dk))
    a.t(k_bonus, "k_bonus", (q.dtype,), shape=(B, H, dk))
    a.t(v_bonus, "v_bonus", (q.dtype,), shape=(B, H, dv))
    _decay_arg(a, alpha_bonus, "alpha_bonus", (B, H), decay_kind, dk)
    a.t(beta_bonus, "beta_bonus", _f32(), shape=(B, H))
    a.t(out, "out", _in_dtypes(), shape=(B, K, H, dv), optional=True)
    a.t(out_bonus, "out_bonus", _in_dtypes(), shape=(B, H, dv), optional=True)
    if out is not None and out_bonus is not None and out.dtype != out_bonus.dtype:
        raise TypeError("replay_accepted_bonus: out and out_bonus must have the same dtype")
    st = a.stream(stream)
    if want_out_bonus:
        out_bonus = _new_out(out_bonus, (B, H, dv), state)
        if out is not None and out.dtype != out_bonus.dtype:
            raise TypeError("replay_accepted_bonus: out and out_bonus must have the same dtype")
    od = out_bonus if out_bonus is not None else out
    _call("replay_accepted_bonus", _ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q),
          _ptr(k), _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta),
          _ptr(n_accept), _ptr(out), _ptr(q_bonus), _ptr(k_bonus), _ptr(v_bonus),
          _ptr(alpha_bonus), _ptr(beta_bonus), _ptr(out_bonus),
          _code(od.dtype) if od is not None else HLA_F32, _ptr(err_flag), st)
    return out_bonus


def verify_drafts(state, q, k, v, alpha, beta, decay_kind, out=None, slot=None, err_flag=None,
                  stream=None):
    """Readouts at all K draft positions from the committed state (which is only read).
    Returns out [B, K, H, dv]."""
    a = _Args("verify_drafts")
    S, H, dk, dv, B, K = _drafts(a, state, q, k, v, alpha, beta, decay_kind, slot, err_flag)
    a.t(out, "out", _in_dtypes(), shape=(B, K, H, dv), optional=True)
    st = a.stream(stream)
    out = _new_out(out, (B, K, H, dv), state)
    _call("verify_drafts", _ptr(state), S, _ptr(slot), B, H, dk, dv, K, _ptr(q), _ptr(k),
          _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta), _ptr(out),
          _code(out.dtype), _ptr(err_flag), st)
    return out


def _damp_group(lo_scale, dv):
    """Scale granularity from the scale tensor's shape: [S,H,rows] per row,
    [S,H,rows,dv/group] per group."""
    if lo_scale.dim() == 3:
        return dv
    if lo_scale.dim() == 4 and lo_scale.shape[3] > 0 and dv % lo_scale.shape[3] == 0:
        return dv // lo_scale.shape[3]
    raise ValueError(f"lo_scale shape {tuple(lo_scale.shape)} fits no scale group of dv={dv}")


def _hi_dtypes():
    torch = _torch()
    return (torch.int16, torch.uint16, torch.float16)


def _packed(a, hi, lo, lo_scale, S, H, dk, dv, K_hi):
    """The three packed regions of S slots x H heads; returns the scale group."""
    if not 0 <= K_hi <= dk:
        raise ValueError(f"{a.fn}: K_hi = {K_hi} outside [0, dk = {dk}]")
    a.t(hi, "hi", _hi_dtypes(), shape=(S, H, K_hi, dv))
    a.t(lo, "lo", (_torch().int8,), shape=(S, H, dk - K_hi, dv))
    a.t(lo_scale, "lo_scale", _f32())
    g = _damp_group(lo_scale, dv)
    a.t(lo_scale, "lo_scale", _f32(),
        shape=(S, H, dk - K_hi) if g == dv else (S, H, dk - K_hi, dv // g))
    return g


def _plans(a, key_perm, val_perm, val_scale, H, dk, dv):
    a.t(key_perm, "key_perm", _i32(), shape=(H, dk), optional=True)
    a.t(val_perm, "val_perm", _i32(), shape=(H, dv), optional=True)
    a.t(val_scale, "val_scale", _f32(), shape=(H, dv), optional=True)


def damp_step(hi, lo, lo_scale, key_perm, K_hi, q, k, v, alpha, decay_kind, beta, out=None,
              slot=None, err_flag=None, stream=None, want_out=True, val_perm=None,
              val_scale=None):
    """One fused dequantise -> update -> requantise step on the packed state (in place).
    The scale group (per row or per 32 values) is read off lo_scale's shape; val_perm /
    val_scale [H, dv] select the value transform (None: untransformed)."""
    a = _Args("damp_step")
    if not isinstance(hi, _torch().Tensor) or hi.dim() != 4:
        raise ValueError("damp_step: hi must be a 4-dimensional tensor [S, H, K_hi, dv]")
    S, H, _, dv = hi.shape
    a.t(q, "q", _in_dtypes(), shape=(None, H, None))
    B, _, dk = q.shape
    group = _packed(a, hi, lo, lo_scale, S, H, dk, dv, K_hi)
    a.t(k, "k", (q.dtype,), shape=(B, H, dk))
    a.t(v, "v", (q.dtype,), shape=(B, H, dv))
    _decay_arg(a, alpha, "alpha", (B, H), decay_kind, dk)
    a.t(beta, "beta", _f32(), shape=(B, H))
    _plans(a, key_perm, val_perm, val_scale, H, dk, dv)
    a.t(slot, "slot", _i32(), shape=(B,), optional=True)
    a.flag(err_flag)
    a.t(out, "out", _in_dtypes(), shape=(B, H, dv), optional=True)
    st = a.stream(stream)
    if want_out:
        out = _new_out(out, (B, H, dv), hi)
    _call("damp_step", _ptr(hi), _ptr(lo), _ptr(lo_scale), S, _ptr(key_perm), K_hi, group,
          _ptr(val_perm), _ptr(val_scale), _ptr(slot), B, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
          _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta), _ptr(out),
          _code(out.dtype) if out is not None else HLA_F32, _ptr(err_flag), st)
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
    """Pack an FP32 state [S,H,dk,dv] into (hi, lo, lo_scale); the three regions are
    allocated when none is given (group None: one scale per row)."""
    a = _Args("damp_quantize")
    a.t(state, "state", _f32(), ndim=4)
    S, H, dk, dv = state.shape
    given = [x is not None for x in (hi, lo, lo_scale)]
    if any(given) and not all(given):
        raise ValueError("damp_quantize: give all of hi, lo and lo_scale, or none")
    if all(given):
        g = _packed(a, hi, lo, lo_scale, S, H, dk, dv, K_hi)
        if group is not None and int(group) != g:
            raise ValueError("damp_quantize: lo_scale shape does not match group")
    else:
        if not 0 <= K_hi <= dk:
            raise ValueError(f"damp_quantize: K_hi = {K_hi} outside [0, dk = {dk}]")
        g = dv if group is None else int(group)
    _plans(a, key_perm, val_perm, val_scale, H, dk, dv)
    st = a.stream(stream)
    if not all(given):
        if g <= 0 or dv % g:
            raise ValueError(f"damp_quantize: group {g} does not divide dv = {dv}")
        hi, lo, lo_scale = damp_alloc(S, H, dk, dv, K_hi, state.device, g)
    _call("damp_quantize", _ptr(state), S, H, dk, dv, _ptr(key_perm), K_hi, g, _ptr(val_perm),
          _ptr(val_scale), _ptr(hi), _ptr(lo), _ptr(lo_scale), st)
    return hi, lo, lo_scale


def damp_dequantize(hi, lo, lo_scale, key_perm, K_hi, dk, out=None, stream=None,
                    val_perm=None, val_scale=None):
    """Reconstruct the FP32 state [S,H,dk,dv] (original coordinates) from the packed
    regions."""
    a = _Args("damp_dequantize")
    if not isinstance(hi, _torch().Tensor) or hi.dim() != 4:
        raise ValueError("damp_dequantize: hi must be a 4-dimensional tensor [S, H, K_hi, dv]")
    S, H, _, dv = hi.shape
    g = _packed(a, hi, lo, lo_scale, S, H, dk, dv, K_hi)
    _plans(a, key_perm, val_perm, val_scale, H, dk, dv)
    a.t(out, "state", _f32(), shape=(S, H, dk, dv), optional=True)
    st = a.stream(stream)
    out = _new_out(out, (S, H, dk, dv), hi)
    _call("damp_dequantize", _ptr(hi), _ptr(lo), _ptr(lo_scale), S, H, dk, dv, _ptr(key_perm),
          K_hi, g, _ptr(val_perm), _ptr(val_scale), _ptr(out), st)
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


def _span(L, stride, S, n_units, unit_bytes):
    """Bytes a layered state buffer must hold: layer L-1 starts at (L-1)*stride and holds
    S slots of n_units units."""
    if min(L, S, n_units, unit_bytes) <= 0 or stride < 0:
        return 0
    return (L - 1) * stride + S * n_units * unit_bytes


def _pairs(a, src_slot, dst_slot):
    a.t(src_slot, "src_slot", _i32(), ndim=1)
    a.t(dst_slot, "dst_slot", _i32(), shape=(src_slot.numel(),))
    return src_slot.numel()


def _unit_index(a, unit_index, R):
    """The retained-unit list [R]; an empty list is passed as NULL."""
    if unit_index is None or (R == 0 and unit_index.numel() == 0):
        return None
    return a.t(unit_index, "unit_index", _i32(), shape=(R,))


def dasc_pack(active, layer_stride_bytes, S_act, L, n_units, unit_bytes, offsets, unit_index,
              R_total, src_slot, dst_slot, packed, S_ckpt, err_flag=None, stream=None):
    """Byte-level pack; `active` and `packed` are device tensors (any dtype) at least as
    large as the geometry given."""
    a = _Args("dasc_pack")
    a.nbytes(active, "active", _span(L, layer_stride_bytes, S_act, n_units, unit_bytes))
    a.t(offsets, "offsets", _i32(), shape=(max(L, 0) + 1,))
    idx = _unit_index(a, unit_index, R_total)
    N = _pairs(a, src_slot, dst_slot)
    a.nbytes(packed, "packed", max(S_ckpt, 0) * max(R_total, 0) * max(unit_bytes, 0))
    a.flag(err_flag)
    _call("dasc_pack", _ptr(active), int(layer_stride_bytes), S_act, L, n_units, int(unit_bytes),
          _ptr(offsets), _ptr(idx), R_total, _ptr(src_slot), _ptr(dst_slot), N, _ptr(packed),
          S_ckpt, _ptr(err_flag), a.stream(stream))


def dasc_restore(packed, S_ckpt, R_total, unit_pos, L, n_units, unit_bytes, src_slot, dst_slot,
                 active_out, layer_stride_bytes, S_dst, err_flag=None, stream=None):
    """Byte-level restore with zero-fill of the omitted units."""
    a = _Args("dasc_restore")
    a.nbytes(packed, "packed", max(S_ckpt, 0) * max(R_total, 0) * max(unit_bytes, 0))
    a.t(unit_pos, "unit_pos", _i32())
    if unit_pos.numel() != max(L, 0) * max(n_units, 0):
        raise ValueError(f"dasc_restore: unit_pos has {unit_pos.numel()} entries, the plan "
                         f"has L * n_units = {L * n_units}")
    N = _pairs(a, src_slot, dst_slot)
    a.nbytes(active_out, "active_out", _span(L, layer_stride_bytes, S_dst, n_units, unit_bytes))
    a.flag(err_flag)
    _call("dasc_restore", _ptr(packed), S_ckpt, R_total, _ptr(unit_pos), L, n_units,
          int(unit_bytes), _ptr(src_slot), _ptr(dst_slot), N, _ptr(active_out),
          int(layer_stride_bytes), S_dst, _ptr(err_flag), a.stream(stream))


def _restore_replay_units(a, units, name, dtypes, dv, dk):
    """Rows per checkpoint unit from the unit buffer's shape: [S_ckpt, R_total, unit_rows *
    dv] or [S_ckpt, R_total, unit_rows, dv]."""
    a.t(units, name, dtypes)
    if units.dim() == 4 and units.shape[3] == dv:
        unit_rows = int(units.shape[2])
    elif units.dim() == 3 and units.shape[2] % dv == 0:
        unit_rows = int(units.shape[2]) // dv
    else:
        raise ValueError(f"{a.fn}: {name}: expected [S_ckpt, R_total, unit_rows * {dv}] or "
                         f"[S_ckpt, R_total, unit_rows, {dv}], got {tuple(units.shape)}")
    if unit_rows < 1 or unit_rows > dk or unit_rows & (unit_rows - 1):
        raise ValueError(f"{a.fn}: {name}: {unit_rows} rows per unit is not a power of two in "
                         f"[1, {dk}]")
    return unit_rows


def _restore_replay(fn, units, scales, unit_pos, src_slot, dst_slot, active_out, q, k, v, alpha,
                    beta, n_accept, decay_kind, out, err_flag, stream):
    a = _Args(fn)
    a.t(active_out, "active_out", _f32(), ndim=5)
    L, S_dst, H, dk, dv = active_out.shape
    q8 = scales is not None
    unit_rows = _restore_replay_units(a, units, "codes" if q8 else "packed",
                                      (_torch().int8,) if q8 else _f32(), dv, dk)
    S_ckpt, R_total = units.shape[:2]
    if q8:
        a.nbytes(scales, "scales", S_ckpt * R_total * unit_rows * 4, _f32())
        if scales.numel() != S_ckpt * R_total * unit_rows:
            raise ValueError(f"{fn}: scales has {scales.numel()} entries, the checkpoint has "
                             f"{S_ckpt * R_total * unit_rows} rows")
    a.t(unit_pos, "unit_pos", _i32())
    n_units = H * dk // unit_rows
    if unit_pos.numel() != L * n_units:
        raise ValueError(f"{fn}: unit_pos has {unit_pos.numel()} entries, the state has "
                         f"L * H * dk / unit_rows = {L * n_units} units")
    N = _pairs(a, src_slot, dst_slot)
    a.t(q, "q", _in_dtypes(), shape=(L, N, None, H, dk))
    K = q.shape[2]
    a.t(k, "k", (q.dtype,), shape=(L, N, K, H, dk))
    a.t(v, "v", (q.dtype,), shape=(L, N, K, H, dv))
    _decay_arg(a, alpha, "alpha", (L, N, K, H), decay_kind, dk)
    a.t(beta, "beta", _f32(), shape=(L, N, K, H))
    a.t(n_accept, "n_accept", _i32(), shape=(N,))
    a.t(out, "out", _in_dtypes(), shape=(L, N, K, H, dv), optional=True)
    a.flag(err_flag)
    head = ([_ptr(units), _ptr(scales)] if q8 else [_ptr(units)])
    _call(fn, *head, S_ckpt, R_total, _ptr(unit_pos), L, unit_rows, _ptr(src_slot),
          _ptr(dst_slot), N, _ptr(active_out), S_dst * H * dk * dv * 4, S_dst, H, dk, dv, K,
          _ptr(q), _ptr(k), _ptr(v), _code(q.dtype), _ptr(alpha), int(decay_kind), _ptr(beta),
          _ptr(n_accept), _ptr(out), _code(out.dtype) if out is not None else HLA_F32,
          _ptr(err_flag), a.stream(stream))
    return out


def dasc_restore_replay(packed, unit_pos, src_slot, dst_slot, active_out, q, k, v, alpha, beta,
                        n_accept, decay_kind, out=None, err_flag=None, stream=None):
    """Restore a checkpoint into private slots and replay each request's accepted drafts,
    layer by layer, in one pass.

    packed [S_ckpt, R_total, unit_rows * dv] (or [S_ckpt, R_total, unit_rows, dv]) fp32:
    units of unit_rows key channels (dk: whole heads; 1: single channels); unit_pos
    [L, H * dk / unit_rows] (or flat) int32 from dasc_plan of the unit mask; active_out
    [L, S_dst, H, dk, dv] fp32; q, k [L, N, K, H, dk], v [L, N, K, H, dv]; alpha
    [L, N, K, H] (scalar decay) or [L, N, K, H, dk]; beta [L, N, K, H]; n_accept [N]
    int32; out [L, N, K, H, dv] or None (no readout)."""
    return _restore_replay("dasc_restore_replay", packed, None, unit_pos, src_slot, dst_slot,
                           active_out, q, k, v, alpha, beta, n_accept, decay_kind, out,
                           err_flag, stream)


def dasc_restore_int8_replay(codes, scales, unit_pos, src_slot, dst_slot, active_out, q, k, v,
                             alpha, beta, n_accept, decay_kind, out=None, err_flag=None,
                             stream=None):
    """As dasc_restore_replay, from an INT8 checkpoint: codes int8 [S_ckpt, R_total,
    unit_rows, dv] (or [S_ckpt, R_total, unit_rows * dv]) and scales fp32 with one entry
    per checkpoint row (S_ckpt * R_total * unit_rows), as dasc_pack_int8 writes them."""
    return _restore_replay("dasc_restore_int8_replay", codes, scales, unit_pos, src_slot,
                           dst_slot, active_out, q, k, v, alpha, beta, n_accept, decay_kind,
                           out, err_flag, stream)


def dasc_pack_int8(active, layer_stride_bytes, S_act, L, n_units, unit_rows, dv, offsets,
                   unit_index, R_total, src_slot, dst_slot, codes, scales, S_ckpt, err_flag=None,
                   stream=None):
    """Quantise-once pack of the retained units of an FP32 state into (codes, scales)."""
    a = _Args("dasc_pack_int8")
    a.nbytes(active, "active", _span(L, layer_stride_bytes, S_act, n_units, unit_rows * dv * 4),
             _f32())
    a.t(offsets, "offsets", _i32(), shape=(max(L, 0) + 1,))
    idx = _unit_index(a, unit_index, R_total)
    N = _pairs(a, src_slot, dst_slot)
    rows = max(S_ckpt, 0) * max(R_total, 0) * max(unit_rows, 0)
    a.nbytes(codes, "codes", rows * max(dv, 0), (_torch().int8,))
    a.nbytes(scales, "scales", rows * 4, _f32())
    a.flag(err_flag)
    _call("dasc_pack_int8", _ptr(active), int(layer_stride_bytes), S_act, L, n_units, unit_rows,
          dv, _ptr(offsets), _ptr(idx), R_total, _ptr(src_slot), _ptr(dst_slot), N,
          _ptr(codes), _ptr(scales), S_ckpt, _ptr(err_flag), a.stream(stream))


def dasc_restore_int8(codes, scales, S_ckpt, R_total, unit_pos, L, n_units, unit_rows, dv,
                      src_slot, dst_slot, active_out, layer_stride_bytes, S_dst, err_flag=None,
                      stream=None):
    """Dequantise-once restore into FP32 active slots, omitted units zero."""
    a = _Args("dasc_restore_int8")
    rows = max(S_ckpt, 0) * max(R_total, 0) * max(unit_rows, 0)
    a.nbytes(codes, "codes", rows * max(dv, 0), (_torch().int8,))
    a.nbytes(scales, "scales", rows * 4, _f32())
    a.t(unit_pos, "unit_pos", _i32())
    if unit_pos.numel() != max(L, 0) * max(n_units, 0):
        raise ValueError(f"dasc_restore_int8: unit_pos has {unit_pos.numel()} entries, the "
                         f"plan has L * n_units = {L * n_units}")
    N = _pairs(a, src_slot, dst_slot)
    a.nbytes(active_out, "active_out",
             _span(L, layer_stride_bytes, S_dst, n_units, unit_rows * dv * 4), _f32())
    a.flag(err_flag)
    _call("dasc_restore_int8", _ptr(codes), _ptr(scales), S_ckpt, R_total, _ptr(unit_pos), L,
          n_units, unit_rows, dv, _ptr(src_slot), _ptr(dst_slot), N, _ptr(active_out),
          int(layer_stride_bytes), S_dst, _ptr(err_flag), a.stream(stream))


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
    a = _Args("dasc_refresh_local")
    a.nbytes(scratch, "scratch",
             _span(L, scratch_layer_stride_bytes, S_scratch, n_units, unit_bytes))
    a.nbytes(active, "active", _span(L, layer_stride_bytes, S_act, n_units, unit_bytes))
    a.t(offsets_local, "offsets", _i32(), shape=(max(L, 0) + 1,))
    idx = _unit_index(a, unit_index_local, R_local)
    N = _pairs(a, src_slot, dst_slot)
    a.flag(err_flag)
    _call("dasc_refresh_local", _ptr(scratch), int(scratch_layer_stride_bytes), S_scratch,
          _ptr(active), int(layer_stride_bytes), S_act, L, n_units, int(unit_bytes),
          _ptr(offsets_local), _ptr(idx), R_local, _ptr(src_slot), _ptr(dst_slot), N,
          _ptr(err_flag), a.stream(stream))

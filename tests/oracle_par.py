"""The float64 oracle run over whole batches on every host thread (test infrastructure).

Requests are independent in every operation the oracle computes (a request's state,
inputs and readouts touch no other request's), so a batch is split into contiguous
request ranges and each range goes through the unchanged oracle routine on its own
thread.  The oracle is a C library called through ctypes, which releases the GIL for
the call, so the ranges run in parallel; the results are the ones a single call over
the whole batch gives, bit for bit.  The error measures used by the parity tests are
evaluated the same way, range by range."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle


def threads() -> int:
    """Host threads to use: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def ranges(n: int, parts: int | None = None):
    parts = max(1, min(n, threads() if parts is None else parts))
    cuts = np.linspace(0, n, parts + 1).round().astype(int)
    return [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def pmap(fn, n: int):
    """fn(b0, b1) over the request ranges of a batch of n, in parallel; list of results."""
    rs = ranges(n)
    if len(rs) == 1:
        return [fn(*rs[0])]
    with ThreadPoolExecutor(len(rs)) as ex:
        return list(ex.map(lambda r: fn(*r), rs))


def _sl(x: dict, b0: int, b1: int) -> dict:
    return {k: np.ascontiguousarray(v[b0:b1]) for k, v in x.items()}


def delta_step(state64, x64, *, per_channel, want_out=True, live=None):
    """oracle.delta_step over the whole batch: request b owns slot b; with `live` (bool
    [B]) the requests where it is False are padding (skipped, readout NaN)."""
    B = x64["q"].shape[0]
    H, dv = state64.shape[1], state64.shape[3]
    out = np.full((B, H, dv), np.nan) if want_out else None

    def run(b0, b1):
        xs = _sl(x64, b0, b1)
        slot = None
        if live is not None:
            slot = np.where(live[b0:b1], np.arange(b1 - b0), -1).astype(np.int32)
        o = oracle.delta_step(state64[b0:b1], xs["q"], xs["k"], xs["v"], xs["alpha"],
                              xs["beta"], per_channel=per_channel, slot=slot,
                              want_out=want_out)
        if want_out:
            out[b0:b1] = o

    pmap(run, B)
    return out


def replay(state64, x64, n_accept, *, per_channel, want_out=True):
    B, K = x64["q"].shape[:2]
    H, dv = state64.shape[1], state64.shape[3]
    out = np.full((B, K, H, dv), np.nan) if want_out else None

    def run(b0, b1):
        xs = _sl(x64, b0, b1)
        o = oracle.replay(state64[b0:b1], xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"],
                          n_accept[b0:b1], per_channel=per_channel, want_out=want_out)
        if want_out:
            out[b0:b1] = o

    pmap(run, B)
    return out


def verify(state64, x64, *, per_channel):
    B, K = x64["q"].shape[:2]
    H, dv = state64.shape[1], state64.shape[3]
    out = np.full((B, K, H, dv), np.nan)

    def run(b0, b1):
        xs = _sl(x64, b0, b1)
        out[b0:b1] = oracle.verify(state64[b0:b1], xs["q"], xs["k"], xs["v"], xs["alpha"],
                                   xs["beta"], per_channel=per_channel)

    pmap(run, B)
    return out


def replay_bonus(state64, x64, n_accept, xb64, *, per_channel):
    """Returns the bonus token's readout [B, H, dv]; the state is advanced in place."""
    B = x64["q"].shape[0]
    H, dv = state64.shape[1], state64.shape[3]
    out_b = np.full((B, H, dv), np.nan)

    def run(b0, b1):
        xs, bs = _sl(x64, b0, b1), _sl(xb64, b0, b1)
        _, ob = oracle.replay_bonus(state64[b0:b1], xs["q"], xs["k"], xs["v"], xs["alpha"],
                                    xs["beta"], n_accept[b0:b1], bs["q"], bs["k"], bs["v"],
                                    bs["alpha"], bs["beta"], per_channel=per_channel)
        out_b[b0:b1] = ob

    pmap(run, B)
    return out_b


def damp_step(hi, lo, sc, key_perm, K_hi, x64, *, per_channel, val_perm=None,
              val_scale=None):
    """oracle.damp_step over the whole batch, in place on the packed arrays."""
    B = x64["q"].shape[0]
    H, dv = sc.shape[1], x64["v"].shape[-1]
    out = np.full((B, H, dv), np.nan)

    def run(b0, b1):
        xs = _sl(x64, b0, b1)
        out[b0:b1] = oracle.damp_step(hi[b0:b1], lo[b0:b1], sc[b0:b1], key_perm, K_hi,
                                      xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"],
                                      per_channel=per_channel, val_perm=val_perm,
                                      val_scale=val_scale)

    pmap(run, B)
    return out


def damp_dequantize(hi, lo, sc, key_perm, K_hi, dk, val_perm=None, val_scale=None):
    S, H = sc.shape[:2]
    dv = lo.shape[-1] if lo.size else hi.shape[-1]
    out = np.empty((S, H, dk, dv), np.float64)

    def run(b0, b1):
        out[b0:b1] = oracle.damp_dequantize(hi[b0:b1], lo[b0:b1], sc[b0:b1], key_perm, K_hi,
                                            dk, val_perm=val_perm, val_scale=val_scale)

    pmap(run, S)
    return out


def readout_scale(state64, q64, live=None):
    """Per (request, head): max over value columns j of sum_i |S[i][j]| |q_i|, the size of
    the terms of the readout o_j = sum_i S[i][j] q_i.  state64 [B, H, dk, dv], q64
    [B, H, dk]; returns [B, H] (zero where `live`, bool [B], is False)."""
    B, H = state64.shape[:2]
    out = np.zeros((B, H))

    def run(b0, b1):
        rows = np.arange(b0, b1) if live is None else b0 + np.flatnonzero(live[b0:b1])
        if rows.size:
            t = np.matmul(np.abs(q64[rows])[:, :, None, :], np.abs(state64[rows]))
            out[rows] = t[:, :, 0, :].max(axis=-1)

    pmap(run, B)
    return out


def replay_terms(state64, x64, n_accept, *, per_channel):
    """The oracle's replay as n_b single steps per request (oracle.replay is exactly that),
    in place on state64.  Returns the readouts [B, K, H, dv] (NaN for t >= n_b) and, for
    each (b, t, h), the size of the readout's terms, max_j sum_i |S_t[i][j]| |q_t,i|: a
    readout evaluated in FP32 has a rounding error relative to that size, not to its own,
    which cancels whenever q and the state's columns are nearly orthogonal."""
    B, K, H = x64["q"].shape[:3]
    n_accept = np.clip(np.asarray(n_accept), 0, K)
    out = np.full((B, K, H, state64.shape[-1]), np.nan)
    scale = np.zeros((B, K, H))
    for t in range(K):
        live = n_accept > t
        xt = {n: np.ascontiguousarray(a[:, t]) for n, a in x64.items()}
        out[:, t] = delta_step(state64, xt, per_channel=per_channel, live=live)
        scale[:, t] = readout_scale(state64, xt["q"], live)
    return out, scale


def rel_err_tiles(got, ref, tile_dims: int = 2) -> float:
    """max over tiles (the last `tile_dims` axes) of max|got - ref| / max|ref|, the
    denominator floored at 1e-30; NaN anywhere in got counts as an infinite error."""
    n = ref.shape[0]

    def run(b0, b1):
        g = np.asarray(got[b0:b1], np.float64)
        r = np.asarray(ref[b0:b1], np.float64)
        lead = int(np.prod(r.shape[: r.ndim - tile_dims]))
        g = g.reshape(lead, -1)
        r = r.reshape(lead, -1)
        if not np.isfinite(g).all():
            return float("inf")
        num = np.abs(g - r).max(axis=1)
        den = np.maximum(np.abs(r).max(axis=1), 1e-30)
        return float((num / den).max())

    return max(pmap(run, n))


def dasc_pack_int8_all(active, offsets, unit_index):
    """oracle.dasc_pack_int8 of every slot of `active` (float32 [L, S, n_units, unit_rows,
    dv]) into checkpoint slot of the same index, slot range by slot range on every host
    thread.  Returns (codes int8 [S, R, unit_rows, dv], scales float32 [S, R, unit_rows])."""
    L, S, n_units, unit_rows, dv = active.shape
    R = int(offsets[-1])
    codes = np.empty((S, R, unit_rows, dv), np.int8)
    scales = np.empty((S, R, unit_rows), np.float32)

    def run(b0, b1):
        ids = np.arange(b1 - b0, dtype=np.int32)
        c, s = oracle.dasc_pack_int8(np.ascontiguousarray(active[:, b0:b1]), offsets,
                                     unit_index, ids, ids, b1 - b0)
        codes[b0:b1] = c
        scales[b0:b1] = s

    pmap(run, S)
    return codes, scales


def dasc_restore_int8_all(codes, scales, offsets, unit_index, L, n_units, active_out):
    """oracle.dasc_restore_int8 of checkpoint slot s into slot s of active_out (float32
    [L, S, n_units, unit_rows, dv], in place) for every slot, by slot ranges."""
    S = codes.shape[0]

    def run(b0, b1):
        ids = np.arange(b1 - b0, dtype=np.int32)
        part = np.ascontiguousarray(active_out[:, b0:b1])
        oracle.dasc_restore_int8(np.ascontiguousarray(codes[b0:b1]),
                                 np.ascontiguousarray(scales[b0:b1]), offsets, unit_index, L,
                                 n_units, ids, ids, part)
        active_out[:, b0:b1] = part

    pmap(run, S)
    return active_out

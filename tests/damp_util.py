"""Comparison helpers for the mixed-precision (DAMP) GPU parity tests.

Bars: FP32 scales bit-exact when both sides quantise the same FP32 values (else
within 1e-5 relative); INT8 codes differ by at most 1 on at most 0.1% of values;
FP16 rows differ by at most one FP16 ulp; every reconstructed INT8 value within one
code step of the oracle's; the reconstructed state within 1e-3 relative in Frobenius
norm per head; the readout within 1e-3 of max|o| per head."""
import numpy as np

import oracle
from gpu_util import dev

STATE_TOL = 1e-3
CODE_FRAC = 1e-3


def _packed_dev(hi, lo, sc):
    return dev(hi.view(np.int16)), dev(lo), dev(sc)


def _packed_host(hi_d, lo_d, sc_d):
    return (hi_d.cpu().numpy().view(np.uint16).copy(), lo_d.cpu().numpy().copy(),
            sc_d.cpu().numpy().copy())


def _code_stats(lo_g, lo_o):
    d = np.abs(lo_g.astype(np.int32) - lo_o.astype(np.int32))
    return (float((d > 0).mean()) if d.size else 0.0), (int(d.max()) if d.size else 0)


def _per_value(sc, dv):
    """Scale of every INT8 value: [.., rows] (one per row) or [.., rows, groups]."""
    if sc.ndim == 3:
        return np.repeat(sc[..., None], dv, axis=-1)
    return np.repeat(sc, dv // sc.shape[-1], axis=-1)


def _state_bars(g, o, perm, K_hi, dk, val_perm=None, val_scale=None):
    """Compare two packed states (hi, lo, scale) and return the worst statistics."""
    hi_g, lo_g, sc_g = g
    hi_o, lo_o, sc_o = o
    frac, dmax = _code_stats(lo_g, lo_o)
    scale_rel = float((np.abs(sc_g.astype(np.float64) - sc_o) / sc_o).max()) if sc_o.size else 0.0
    if hi_o.size:
        a = hi_g.view(np.float16).astype(np.float64)
        b = hi_o.view(np.float16).astype(np.float64)
        ulp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float16)).astype(np.float64)
        fp16_ulps = float((np.abs(a - b) / ulp).max())
    else:
        fp16_ulps = 0.0
    if lo_o.size:
        dv = lo_o.shape[-1]
        pv_g, pv_o = _per_value(sc_g, dv), _per_value(sc_o, dv)
        dq_g = lo_g.astype(np.float64) * pv_g
        dq_o = lo_o.astype(np.float64) * pv_o
        step = np.maximum(pv_g, pv_o).astype(np.float64)
        steps = float((np.abs(dq_g - dq_o) / step).max())
    else:
        steps = 0.0
    s_g = oracle.damp_dequantize(hi_g, lo_g, sc_g, perm, K_hi, dk, val_perm=val_perm,
                                 val_scale=val_scale)
    s_o = oracle.damp_dequantize(hi_o, lo_o, sc_o, perm, K_hi, dk, val_perm=val_perm,
                                 val_scale=val_scale)
    d = (s_g - s_o).reshape(s_o.shape[0] * s_o.shape[1], -1)
    r = s_o.reshape(d.shape)
    frob = float((np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)).max())
    return dict(frac=frac, dmax=dmax, scale_rel=scale_rel, fp16_ulps=fp16_ulps,
                code_steps=steps, state=frob)


def _assert_bars(w):
    assert w["dmax"] <= 1 and w["frac"] <= CODE_FRAC
    assert w["scale_rel"] <= 1e-5 and w["fp16_ulps"] <= 1.0
    assert w["code_steps"] <= 1.001
    assert w["state"] <= STATE_TOL and w["out"] <= STATE_TOL


def _perm(rng, H, dk):
    return np.stack([rng.permutation(dk) for _ in range(H)]).astype(np.int32)


def state_bars_batch(g, o, perm, K_hi, dk, val_perm=None, val_scale=None):
    """_state_bars over a whole batch, request range by request range on every host
    thread; the code-disagreement fraction is taken over all INT8 values, every other
    figure is the worst over the ranges."""
    import oracle_par

    n = o[2].shape[0]

    def run(b0, b1):
        w = _state_bars(tuple(a[b0:b1] for a in g), tuple(a[b0:b1] for a in o), perm, K_hi, dk,
                        val_perm=val_perm, val_scale=val_scale)
        return w, o[1][b0:b1].size

    parts = oracle_par.pmap(run, n)
    total = sum(c for _, c in parts)
    w = {k: max(p[k] for p, _ in parts) for k in parts[0][0]}
    w["frac"] = sum(p["frac"] * c for p, c in parts) / total if total else 0.0
    return w

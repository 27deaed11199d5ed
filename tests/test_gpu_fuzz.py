"""Seeded random configurations of every state-update entry point against the float64
oracle: head sizes, batch, heads, draft count, input / output types (FP32, bf16,
binary16), decay kind, slot
maps with padding requests, accepted counts and DAMP budgets drawn per case.  Each case
is small (the oracle finishes it in well under a second); the bars are the ones of the
dedicated tests (FP32 1e-5 of max|oracle| per head tile; DAMP the code / scale / state
bars of damp_util)."""
import numpy as np
import pytest

import oracle
import synth
from damp_util import _assert_bars, _packed_dev, _packed_host, _state_bars
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, rel_err_tiles, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")
N_CASES = 12


def _case(i):
    g = np.random.default_rng(9000 + i)
    dk, dv = (int(x) for x in g.choice([64, 128], size=2))
    kind = "kda" if g.random() < 0.5 else "gdn"
    u = g.random()
    in_dtype = "bf16" if u < 0.35 else "f16" if u < 0.55 else "f32"
    B, H, K = int(g.integers(1, 7)), int(g.integers(1, 4)), int(g.integers(1, 17))
    n_slots = B + int(g.integers(0, 4))
    slot = g.permutation(n_slots)[:B].astype(np.int32)
    slot[g.random(B) < 0.2] = -1                       # padding requests
    base = synth.CONFIGS["dasc_gdn"]
    cfg = synth.shrink(base, B=B, H=H, dk=dk, dv=dv, K=K, in_dtype=in_dtype,
                       decay="vector" if kind == "kda" else "scalar", seed=base.seed + 97 * i)
    return g, cfg, kind, n_slots, slot


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_step_replay_verify(i):
    hla = need_gpu()
    g, cfg, kind, n_slots, slot = _case(i)
    per = kind == "kda"
    live = slot >= 0
    S0 = synth.initial_state(cfg, S=n_slots)
    # one step through the slot map
    x = synth.step_inputs(cfg, 0)
    st = dev(S0)
    u = g.random()
    out_dtype = torch.bfloat16 if u < 0.2 else torch.float16 if u < 0.35 else torch.float32
    out = torch.full((cfg.B, cfg.H, cfg.dv), 3.0, device="cuda", dtype=out_dtype)
    fn = hla.kda_step if per else hla.gdn_step
    fn(st, *(dev_inputs(x, cfg.in_dtype)[n] for n in NAMES), out=out, slot=dev(slot))
    S64 = S0.astype(np.float64)
    x64 = f64_inputs(x, cfg.in_dtype)
    o_ref = (oracle.kda_step if per else oracle.gdn_step)(S64, *(x64[n] for n in NAMES),
                                                          slot=slot)
    assert rel_err_tiles(host(st), S64) <= TOL
    o = host(out)
    if live.any() and out_dtype == torch.float32:
        assert rel_err_tiles(o[live], o_ref[live], 1) <= TOL
    elif live.any():  # 2-byte readout: one bf16 / binary16 rounding of the FP32 value
        rel = 2.0 ** -8 if out_dtype == torch.bfloat16 else 2.0 ** -11
        bound = (rel * np.abs(o_ref[live]) + TOL * np.abs(o_ref[live]).max(-1, keepdims=True)
                 + 2.0 ** -24)
        assert (np.abs(o[live] - o_ref[live]) <= bound).all()
    assert (o[~live] == 3.0).all()
    # verify (state only read), then a replay with random accepted counts
    xr = synth.replay_inputs(cfg, 1)
    xd = dev_inputs({n: xr[n] for n in NAMES}, cfg.in_dtype)
    r64 = f64_inputs({n: xr[n] for n in NAMES}, cfg.in_dtype)
    before = host(st).copy()
    ov = hla.verify_drafts(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], int(per),
                           slot=dev(slot))
    assert np.array_equal(host(st), before)
    ov_ref = oracle.verify(S64, r64["q"], r64["k"], r64["v"], r64["alpha"], r64["beta"],
                           per_channel=per, slot=slot)
    if live.any():
        assert rel_err_tiles(host(ov)[live], ov_ref[live], 1) <= TOL
    n_acc = g.integers(0, cfg.K + 1, cfg.B).astype(np.int32)
    orp = hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                              dev(n_acc), int(per), slot=dev(slot))
    or_ref = oracle.replay(S64, r64["q"], r64["k"], r64["v"], r64["alpha"], r64["beta"], n_acc,
                           per_channel=per, slot=slot)
    assert rel_err_tiles(host(st), S64) <= TOL
    o_r = host(orp)
    for b in np.nonzero(live)[0]:
        if n_acc[b]:
            assert rel_err_tiles(o_r[b, :n_acc[b]], or_ref[b, :n_acc[b]], 1) <= TOL


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_damp_step(i):
    hla = need_gpu()
    g, cfg, kind, n_slots, slot = _case(i)
    # any FP16 budget, but at least 32 INT8 rows when there are INT8 rows at all: the
    # code bar (at most 0.1% of codes off by one) needs enough codes for one flip
    K_hi = int(g.integers(0, cfg.dk - 31)) if g.random() < 0.85 else cfg.dk
    group = int(g.choice([32, cfg.dv]))
    cfg = synth.shrink(cfg, K_hi=K_hi, state_sigma=0.05)
    perm = np.stack([g.permutation(cfg.dk) for _ in range(cfg.H)]).astype(np.int32)
    S0 = synth.initial_state(cfg, S=n_slots)
    hi, lo, sc = oracle.damp_quantize(S0.astype(np.float64), perm, K_hi, group=group)
    hi_d, lo_d, sc_d = _packed_dev(hi, lo, sc)
    x = synth.step_inputs(cfg, 0)
    per = kind == "kda"
    o = hla.damp_step(hi_d, lo_d, sc_d, dev(perm), K_hi, *(dev_inputs(x, cfg.in_dtype)[n]
                      for n in ("q", "k", "v", "alpha")), int(per),
                      dev_inputs(x, cfg.in_dtype)["beta"], slot=dev(slot))
    x64 = f64_inputs(x, cfg.in_dtype)
    o_ref = oracle.damp_step(hi, lo, sc, perm, K_hi, x64["q"], x64["k"], x64["v"],
                             x64["alpha"], x64["beta"], per_channel=per, slot=slot)
    w = _state_bars(_packed_host(hi_d, lo_d, sc_d), (hi, lo, sc), perm, K_hi, cfg.dk)
    live = slot >= 0
    w["out"] = rel_err_tiles(host(o)[live], o_ref[live], 1) if live.any() else 0.0
    _assert_bars(w)

"""Every head of the serving-size workloads against the float64 oracle.

The smaller parity tests cover shapes, dtypes and edge cases; these run the workloads
the benchmark times, in its launch configuration, and compare every (request, head)
element by element with the oracle, which runs over the same batch on every host
thread (`oracle_par`: request ranges through the unchanged oracle routines).

* GDN and KDA steps ([DAMP] §3.1 Eq. (1)-(2)): batch 256 x 32 heads x 128 x 128,
  32 consecutive steps, state and readout after every step within 1e-5 of max|oracle|
  per head tile.
* The mixed-precision step ([DAMP] §3.2-§3.3, App. A.4), both layouts (one FP32 scale
  per row; group-32 scales with the value transform of App. A.3): the initial
  quantisation of the whole batch, then 3 teacher-forced steps (before each step the
  GPU's packed state is read back and the oracle takes the same step from it), at the
  bars of the mixed-precision tests (codes within 1 on at most 0.1% of values, FP16
  rows within one ulp, scales, state within 1e-3 per head, readout within 1e-3).
* Replay, verify and replay + bonus ([K3] "Speculative decoding without state
  snapshots") on the checkpoint workload's 512 request states x 32 heads, K = 8
  drafts, accepted counts U{0..8}: state and every readout within 1e-5."""
import numpy as np
import pytest

import oracle
import oracle_par
import synth
from damp_util import _assert_bars, _packed_host, state_bars_batch
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")


@pytest.mark.parametrize("name", ["gdn_serving", "kda_serving"])
def test_step_every_head_32_steps(name):
    hla = need_gpu()
    cfg = synth.CONFIGS[name]
    kda = cfg.decay == "vector"
    fn = hla.kda_step if kda else hla.gdn_step
    S0 = synth.initial_state(cfg)
    st = dev(S0)
    S64 = S0.astype(np.float64)
    del S0
    out = torch.empty((cfg.B, cfg.H, cfg.dv), device="cuda")
    worst_s = worst_o = 0.0
    for step in range(32):
        x = synth.step_inputs(cfg, step)
        xd = dev_inputs(x, cfg.in_dtype)
        fn(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], out=out)
        o_ref = oracle_par.delta_step(S64, f64_inputs(x, cfg.in_dtype), per_channel=kda)
        worst_o = max(worst_o, oracle_par.rel_err_tiles(host(out), o_ref, 1))
        worst_s = max(worst_s, oracle_par.rel_err_tiles(host(st), S64))
        assert worst_s <= TOL and worst_o <= TOL, (step, worst_s, worst_o)
    print(f"{name}: {cfg.B * cfg.H} heads x 32 steps, worst state err {worst_s:.2e}, "
          f"readout err {worst_o:.2e}")


def _damp_setup(hla, cfg):
    group = synth.damp_group(cfg)
    perm = synth.damp_key_perm(cfg)
    vp = vs = None
    if cfg.sr:
        vp, vs = synth.damp_value_plan(cfg)
    tabs = dict(group=group, val_perm=None if vp is None else dev(vp),
                val_scale=None if vs is None else dev(vs))
    return group, perm, vp, vs, tabs


@pytest.mark.parametrize("name", ["damp_kda", "damp_kda_g32sr"])
def test_mixed_precision_every_head_teacher_forced(name):
    hla = need_gpu()
    cfg = synth.CONFIGS[name]
    group, perm, vp, vs, tabs = _damp_setup(hla, cfg)
    perm_d = dev(perm)
    S0 = synth.initial_state(cfg)
    hi_d, lo_d, sc_d = hla.damp_quantize(dev(S0), perm_d, cfg.K_hi, **tabs)
    # the initial quantisation of the whole batch against the oracle's quantiser
    S64 = S0.astype(np.float64)
    del S0
    parts = oracle_par.pmap(lambda b0, b1: oracle.damp_quantize(
        S64[b0:b1], perm, cfg.K_hi, group=group, val_perm=vp, val_scale=vs), cfg.B)
    ref = tuple(np.concatenate([p[i] for p in parts]) for i in range(3))
    del S64, parts
    g0 = _packed_host(hi_d, lo_d, sc_d)
    if not cfg.sr:  # with a value scale the GPU divides in FP32, the oracle in float64
        assert np.array_equal(g0[0], ref[0])  # FP16 rows: the same RNE of the same value
        assert np.array_equal(g0[2], ref[2])  # scales: fl(max / 127) of the same values
    w = state_bars_batch(g0, ref, perm, cfg.K_hi, cfg.dk, val_perm=vp, val_scale=vs)
    w["out"] = 0.0
    print(f"{name} quantise: {w}")
    _assert_bars(w)
    del ref, g0
    worst = {}
    for step in range(3):
        x = synth.step_inputs(cfg, step)
        hi, lo, sc = _packed_host(hi_d, lo_d, sc_d)  # both sides start from these bits
        xd = dev_inputs(x, cfg.in_dtype)
        out = hla.damp_step(hi_d, lo_d, sc_d, perm_d, cfg.K_hi, xd["q"], xd["k"], xd["v"],
                            xd["alpha"], 1, xd["beta"], val_perm=tabs["val_perm"],
                            val_scale=tabs["val_scale"])
        o_ref = oracle_par.damp_step(hi, lo, sc, perm, cfg.K_hi, f64_inputs(x, cfg.in_dtype),
                                     per_channel=True, val_perm=vp, val_scale=vs)
        w = state_bars_batch(_packed_host(hi_d, lo_d, sc_d), (hi, lo, sc), perm, cfg.K_hi,
                             cfg.dk, val_perm=vp, val_scale=vs)
        w["out"] = oracle_par.rel_err_tiles(host(out), o_ref, 1)
        print(f"{name} step {step + 1}: {w}")
        _assert_bars(w)
        for k, v in w.items():
            worst[k] = max(worst.get(k, 0.0), v)
    print(f"{name}: {cfg.B * cfg.H} heads x 3 teacher-forced steps, worst {worst}")


def _replay_setup(cfg, layer=0):
    x = synth.replay_inputs(cfg, layer)
    xd = dev_inputs({n: x[n] for n in NAMES}, cfg.in_dtype)
    x64 = f64_inputs({n: x[n] for n in NAMES}, cfg.in_dtype)
    return x, xd, x64


def _masked_drafts(o, n_accept):
    """Readouts [B, K, H, dv] with rows t >= n_b set to zero."""
    o = np.array(o, np.float64, copy=True)
    K = o.shape[1]
    o[np.arange(K)[None, :] >= n_accept[:, None]] = 0.0
    return o


def test_replay_every_head_checkpoint_workload():
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    x, xd, x64 = _replay_setup(cfg)
    n_acc = x["n_accept"]
    S0 = synth.initial_state(cfg, S=cfg.slots)
    st = dev(S0)
    S64 = S0.astype(np.float64)
    out = torch.full((cfg.B, cfg.K, cfg.H, cfg.dv), 5.0, device="cuda")
    hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], dev(n_acc), 0,
                        out=out)
    o_ref = oracle_par.replay(S64, x64, n_acc, per_channel=False)
    got = host(st)
    assert oracle_par.rel_err_tiles(got, S64) <= TOL
    idle = n_acc == 0
    assert np.array_equal(got[idle], S0[idle])  # n = 0: the state is not touched
    o = host(out)
    rows = np.arange(cfg.K)[None, :] < n_acc[:, None]
    assert (o[~rows] == 5.0).all()               # rows t >= n_b are left alone
    assert oracle_par.rel_err_tiles(_masked_drafts(o, n_acc), _masked_drafts(o_ref, n_acc),
                                    1) <= TOL


def test_verify_every_head_checkpoint_workload():
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    _, xd, x64 = _replay_setup(cfg, layer=1)
    S0 = synth.initial_state(cfg, S=cfg.slots)
    st = dev(S0)
    out = hla.verify_drafts(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], 0)
    o_ref = oracle_par.verify(S0.astype(np.float64), x64, per_channel=False)
    assert np.array_equal(host(st), S0)          # the committed state is only read
    assert oracle_par.rel_err_tiles(host(out), o_ref, 1) <= TOL


def test_replay_bonus_every_head_checkpoint_workload():
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    x, xd, x64 = _replay_setup(cfg, layer=2)
    xb = synth.step_inputs(cfg, 10_002)
    bd = dev_inputs(xb, cfg.in_dtype)
    n_acc = x["n_accept"]
    S0 = synth.initial_state(cfg, S=cfg.slots)
    st = dev(S0)
    S64 = S0.astype(np.float64)
    del S0
    ob = hla.replay_accepted_bonus(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                   dev(n_acc), 0, bd["q"], bd["k"], bd["v"], bd["alpha"],
                                   bd["beta"])
    ob_ref = oracle_par.replay_bonus(S64, x64, n_acc, f64_inputs(xb, cfg.in_dtype),
                                     per_channel=False)
    assert oracle_par.rel_err_tiles(host(st), S64) <= TOL
    assert oracle_par.rel_err_tiles(host(ob), ob_ref, 1) <= TOL

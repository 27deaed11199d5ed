"""GPU parity of the mixed-precision state in the DAMP paper's deployed layout against
the float64 oracle: INT8 rows with one FP32 scale per group of 32 values (App. A.1 /
A.4) and the value scaling and reordering of App. A.3 Eq. (17)-(18).

Bars are those of the per-row layout (tests/damp_util.py).  With a value scale the
GPU divides in FP32 (v / c' as v * rcp(c') in the step, correctly rounded in the
codec) where the oracle divides in float64, so FP16 rows may round one ulp apart and
FP32 scales may differ in the last bit; both are inside the bars."""
import numpy as np
import pytest

import oracle
import synth
from damp_util import _assert_bars, _packed_dev, _packed_host, _perm, _state_bars
from gpu_util import (dev, dev_inputs, f64_inputs, gather_heads, host, need_gpu, rel_err_tiles,
                      sample_heads, torch)

pytestmark = pytest.mark.gpu


def _vplan(rng, H, dv, mode):
    """mode: 'none', 'scale' (order folded into the weights), 'perm', 'both'."""
    perm = np.stack([rng.permutation(dv) for _ in range(H)]).astype(np.int32)
    scale = np.exp(rng.normal(0.0, 0.5, (H, dv))).astype(np.float32)
    return (perm if mode in ("perm", "both") else None,
            scale if mode in ("scale", "both") else None)


def _d(a):
    return None if a is None else dev(a)


@pytest.mark.parametrize("mode", ["none", "both", "scale"])
@pytest.mark.parametrize("dk,dv,K_hi", [(128, 128, 16), (64, 64, 5), (128, 64, 0), (64, 128, 64)])
def test_grouped_quantize_and_dequantize(dk, dv, K_hi, mode):
    hla = need_gpu()
    rng = np.random.default_rng(dk + dv + K_hi + len(mode))
    S_, H = 3, 4
    state = (rng.standard_normal((S_, H, dk, dv)) * 0.05).astype(np.float32)
    state[0, 0, 3] = 0.0                    # a zero row: every group takes the scale floor
    state[1, 2, 7, 5] = 40.0                # an outlier in one group only
    perm = _perm(rng, H, dk)
    vp, vs = _vplan(rng, H, dv, mode)
    hi_d, lo_d, sc_d = hla.damp_quantize(dev(state), dev(perm), K_hi, group=32,
                                         val_perm=_d(vp), val_scale=_d(vs))
    assert tuple(sc_d.shape) == (S_, H, dk - K_hi, dv // 32)
    g = _packed_host(hi_d, lo_d, sc_d)
    o = oracle.damp_quantize(state.astype(np.float64), perm, K_hi, group=32, val_perm=vp,
                             val_scale=vs)
    if mode == "none":
        assert np.array_equal(g[0], o[0])   # FP16 rows: same RNE from the same FP32 value
        assert np.array_equal(g[2], o[2])   # scale = fl(max / 127), bit-exact
    w = _state_bars(g, o, perm, K_hi, dk, vp, vs)
    w["out"] = 0.0
    _assert_bars(w)
    back = host(hla.damp_dequantize(hi_d, lo_d, sc_d, dev(perm), K_hi, dk, val_perm=_d(vp),
                                    val_scale=_d(vs)))
    ref = oracle.damp_dequantize(*g, perm, K_hi, dk, val_perm=vp, val_scale=vs)
    assert rel_err_tiles(back, ref) <= 1e-6


def _teacher_forced(hla, cfg, perm, vp, vs, steps, slot=None, n_slots=None):
    n_slots = cfg.B if n_slots is None else n_slots
    group = synth.damp_group(cfg)
    S0 = synth.initial_state(cfg, S=n_slots).astype(np.float64)
    hi, lo, sc = oracle.damp_quantize(S0, perm, cfg.K_hi, group=group, val_perm=vp,
                                      val_scale=vs)
    per = cfg.decay == "vector"
    worst = {}
    for step in range(steps):
        x = synth.step_inputs(cfg, step)
        hi_d, lo_d, sc_d = _packed_dev(hi, lo, sc)
        xd = dev_inputs(x, cfg.in_dtype)
        out = torch.full((cfg.B, cfg.H, cfg.dv), 3.0, device="cuda")
        hla.damp_step(hi_d, lo_d, sc_d, _d(perm), cfg.K_hi, xd["q"], xd["k"], xd["v"],
                      xd["alpha"], 1 if per else 0, xd["beta"], out=out,
                      slot=None if slot is None else dev(slot), val_perm=_d(vp),
                      val_scale=_d(vs))
        x64 = f64_inputs(x, cfg.in_dtype)
        o_ref = oracle.damp_step(hi, lo, sc, perm, cfg.K_hi, x64["q"], x64["k"], x64["v"],
                                 x64["alpha"], x64["beta"], per_channel=per, slot=slot,
                                 val_perm=vp, val_scale=vs)
        w = _state_bars(_packed_host(hi_d, lo_d, sc_d), (hi, lo, sc), perm, cfg.K_hi, cfg.dk,
                        vp, vs)
        live = np.ones(cfg.B, bool) if slot is None else slot >= 0
        o = host(out)
        w["out"] = rel_err_tiles(o[live], o_ref[live], 1)
        for key, val in w.items():
            worst[key] = max(worst.get(key, 0), val)
        assert (o[~live] == 3.0).all()
    return worst


@pytest.mark.parametrize("mode", ["none", "both", "scale", "perm"])
@pytest.mark.parametrize("decay", ["vector", "scalar"])
@pytest.mark.parametrize("dk,dv,K_hi", [(128, 128, 16), (64, 64, 5), (128, 64, 0),
                                        (64, 128, 64), (128, 128, 37)])
def test_grouped_step_teacher_forced(dk, dv, K_hi, decay, mode):
    hla = need_gpu()
    base = synth.CONFIGS["damp_kda_g32sr"]
    cfg = synth.shrink(base, B=5, H=3, dk=dk, dv=dv, K_hi=K_hi, decay=decay,
                       seed=base.seed + dk + dv + K_hi)
    rng = np.random.default_rng(K_hi + dv)
    perm = _perm(rng, cfg.H, dk)
    vp, vs = _vplan(rng, cfg.H, dv, mode)
    slot = np.array([3, -1, 0, 5, 1], np.int32)
    w = _teacher_forced(hla, cfg, perm, vp, vs, steps=3, slot=slot, n_slots=6)
    print(w)
    _assert_bars(w)


def test_per_row_scales_with_value_transform():
    """The value transform also runs with one scale per row."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda_g32sr"], B=6, H=4, group=0)
    vp, vs = synth.damp_value_plan(cfg)
    w = _teacher_forced(hla, cfg, synth.damp_key_perm(cfg), vp, vs, steps=3)
    print(w)
    _assert_bars(w)


def test_workload_plan_teacher_forced():
    """The deployed-layout workload's own plans (16 FP16 rows per head biased to slow
    decay; seeded value scales with the RMS-sorted order), 32 heads, bf16 inputs."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda_g32sr"], B=8)
    vp, vs = synth.damp_value_plan(cfg)
    w = _teacher_forced(hla, cfg, synth.damp_key_perm(cfg), vp, vs, steps=4)
    print(w)
    _assert_bars(w)


def test_serving_shape_sampled_heads_teacher_forced():
    """Batch 256 x 32 heads in the benchmark's launch configuration of the deployed
    layout: before each of 2 steps the packed state of 24 sampled heads is read back, the
    oracle takes the same step from it, and the GPU's result for those heads is compared."""
    hla = need_gpu()
    cfg = synth.CONFIGS["damp_kda_g32sr"]
    perm = synth.damp_key_perm(cfg)
    vp, vs = synth.damp_value_plan(cfg)
    perm_d, vp_d, vs_d = dev(perm), dev(vp), dev(vs)
    S0 = dev(synth.initial_state(cfg))
    hi_d, lo_d, sc_d = hla.damp_quantize(S0, perm_d, cfg.K_hi, group=32, val_perm=vp_d,
                                         val_scale=vs_d)
    del S0
    pairs = sample_heads(np.random.default_rng(19), cfg.B, cfg.H, 24)
    bi = torch.tensor([b for b, _ in pairs], device="cuda")
    hh = torch.tensor([h for _, h in pairs], device="cuda")
    for step in range(2):
        x = synth.step_inputs(cfg, step)
        before = [a[bi, hh][:, None].cpu().numpy().copy() for a in (hi_d, lo_d, sc_d)]
        before[0] = before[0].view(np.uint16)
        xd = dev_inputs(x, cfg.in_dtype)
        o = hla.damp_step(hi_d, lo_d, sc_d, perm_d, cfg.K_hi, xd["q"], xd["k"], xd["v"],
                          xd["alpha"], 1, xd["beta"], val_perm=vp_d, val_scale=vs_d)
        xs = gather_heads(f64_inputs(x, cfg.in_dtype), pairs)
        after = [a[bi, hh][:, None].cpu().numpy() for a in (hi_d, lo_d, sc_d)]
        after[0] = after[0].view(np.uint16)
        o_g = host(o[bi, hh])
        for i, (b, h) in enumerate(pairs):
            ref = [a[i:i + 1].copy() for a in before]
            xi = {n: xs[n][i:i + 1] for n in xs}
            o_ref = oracle.damp_step(*ref, perm[h:h + 1], cfg.K_hi, xi["q"], xi["k"], xi["v"],
                                     xi["alpha"], xi["beta"], per_channel=True,
                                     val_perm=vp[h:h + 1], val_scale=vs[h:h + 1])
            w = _state_bars(tuple(a[i:i + 1] for a in after), tuple(ref), perm[h:h + 1],
                            cfg.K_hi, cfg.dk, vp[h:h + 1], vs[h:h + 1])
            w["out"] = rel_err_tiles(o_g[i:i + 1], o_ref[0], 1)
            _assert_bars(w)


def test_free_running_drift_deployed_layout():
    """16 free-running steps on both sides from the same packed state: each trajectory's
    drift from the unquantised FP32 recurrence is of the same size on both sides."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda_g32sr"], B=4)
    perm = synth.damp_key_perm(cfg)
    vp, vs = synth.damp_value_plan(cfg)
    S0 = synth.initial_state(cfg).astype(np.float64)
    hi, lo, sc = oracle.damp_quantize(S0, perm, cfg.K_hi, group=32, val_perm=vp, val_scale=vs)
    S_fp = oracle.damp_dequantize(hi, lo, sc, perm, cfg.K_hi, cfg.dk, val_perm=vp,
                                  val_scale=vs)
    hi_d, lo_d, sc_d = _packed_dev(hi, lo, sc)
    perm_d, vp_d, vs_d = dev(perm), dev(vp), dev(vs)
    for step in range(16):
        x = synth.step_inputs(cfg, step)
        xd = dev_inputs(x, cfg.in_dtype)
        o = hla.damp_step(hi_d, lo_d, sc_d, perm_d, cfg.K_hi, xd["q"], xd["k"], xd["v"],
                          xd["alpha"], 1, xd["beta"], val_perm=vp_d, val_scale=vs_d)
        x64 = f64_inputs(x, cfg.in_dtype)
        o_ref = oracle.damp_step(hi, lo, sc, perm, cfg.K_hi, x64["q"], x64["k"], x64["v"],
                                 x64["alpha"], x64["beta"], per_channel=True, val_perm=vp,
                                 val_scale=vs)
        o_fp = oracle.kda_step(S_fp, x64["q"], x64["k"], x64["v"], x64["alpha"], x64["beta"])
    g = _packed_host(hi_d, lo_d, sc_d)
    s_g = oracle.damp_dequantize(*g, perm, cfg.K_hi, cfg.dk, val_perm=vp, val_scale=vs)
    s_o = oracle.damp_dequantize(hi, lo, sc, perm, cfg.K_hi, cfg.dk, val_perm=vp, val_scale=vs)
    nfp = np.linalg.norm(S_fp)
    drift_g, drift_o = np.linalg.norm(s_g - S_fp) / nfp, np.linalg.norm(s_o - S_fp) / nfp
    on = np.linalg.norm(o_fp)
    od_g, od_o = np.linalg.norm(host(o) - o_fp) / on, np.linalg.norm(o_ref - o_fp) / on
    print(dict(drift_gpu=drift_g, drift_oracle=drift_o, out_gpu=od_g, out_oracle=od_o))
    assert drift_g <= 1.5 * drift_o + 1e-4
    assert od_g <= 1.5 * od_o + 1e-4


def test_bad_value_permutation_entry_sets_flag():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda_g32sr"], B=2, H=2)
    vp, vs = synth.damp_value_plan(cfg)
    hi_d, lo_d, sc_d = hla.damp_quantize(dev(synth.initial_state(cfg)), None, cfg.K_hi,
                                         group=32)
    bad = vp.copy()
    bad[1, 7] = 1000
    xd = dev_inputs(synth.step_inputs(cfg, 0), cfg.in_dtype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.damp_step(hi_d, lo_d, sc_d, None, cfg.K_hi, xd["q"], xd["k"], xd["v"], xd["alpha"], 1,
                  xd["beta"], err_flag=err, val_perm=dev(bad), val_scale=dev(vs))
    torch.cuda.synchronize()
    assert int(err.item()) == hla.DEVERR_PLAN

"""GPU parity of the mixed-precision state kernels (damp_quantize, damp_dequantize,
damp_step) against the float64 oracle.

Bars: FP32 scales bit-exact when both sides quantise the same FP32 values (else
within 1e-5 relative: the row maximum comes from an FP32 update on the GPU and a
float64 one in the oracle); INT8 codes differ by at most 1 on at most 0.1% of values
(the quantiser's FP32 rounding decision can land on the other side of a
half-integer); FP16 rows differ by at most one FP16 ulp; every reconstructed value
within one code step of the oracle's; the reconstructed state within 1e-3 relative in
Frobenius norm per head (a single legitimate 1-code flip is a whole quantisation step,
up to 1/127 of the row maximum, so a max-norm bar of 1e-3 could not hold); the
readout within 1e-3 of max|o| per head.  The step is checked teacher-forced (both
sides start every step from the same packed state) and free-running (the statistics
are reported)."""
import numpy as np
import pytest

import oracle
import synth
from damp_util import (CODE_FRAC, STATE_TOL, _assert_bars, _code_stats, _packed_dev,
                       _packed_host, _perm, _state_bars)
from gpu_util import (dev, dev_inputs, f64_inputs, gather_heads, host, need_gpu, rel_err_tiles,
                      sample_heads, torch)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dk,dv,K_hi", [(128, 128, 16), (64, 64, 5), (128, 64, 0), (64, 128, 64)])
def test_quantize_and_dequantize(dk, dv, K_hi):
    hla = need_gpu()
    rng = np.random.default_rng(dk + dv + K_hi)
    S_, H = 3, 4
    state = (rng.standard_normal((S_, H, dk, dv)) * 0.05).astype(np.float32)
    state[0, 0, 3] = 0.0                    # a zero row: scale floor
    state[1, 2, 7, 5] = 40.0                # an outlier
    perm = _perm(rng, H, dk)
    hi_d, lo_d, sc_d = hla.damp_quantize(dev(state), dev(perm), K_hi)
    hi_g, lo_g, sc_g = _packed_host(hi_d, lo_d, sc_d)
    hi_o, lo_o, sc_o = oracle.damp_quantize(state.astype(np.float64), perm, K_hi)
    assert np.array_equal(hi_g, hi_o)       # FP16 rows: same RNE from the same FP32 value
    assert np.array_equal(sc_g, sc_o)       # scale = fl(max / 127), bit-exact
    frac, dmax = _code_stats(lo_g, lo_o)
    assert dmax <= 1 and frac <= CODE_FRAC
    back = host(hla.damp_dequantize(hi_d, lo_d, sc_d, dev(perm), K_hi, dk))
    ref = oracle.damp_dequantize(hi_g, lo_g, sc_g, perm, K_hi, dk)
    assert rel_err_tiles(back, ref) <= 1e-6


def _teacher_forced(hla, cfg, perm, steps, slot=None, n_slots=None):
    rng = np.random.default_rng(cfg.seed)
    n_slots = cfg.B if n_slots is None else n_slots
    S0 = synth.initial_state(cfg, S=n_slots).astype(np.float64)
    hi, lo, sc = oracle.damp_quantize(S0, perm, cfg.K_hi)
    per = cfg.decay == "vector"
    worst = {}
    for step in range(steps):
        x = synth.step_inputs(cfg, step)
        hi_d, lo_d, sc_d = _packed_dev(hi, lo, sc)
        xd = dev_inputs(x, cfg.in_dtype)
        out = torch.full((cfg.B, cfg.H, cfg.dv), 3.0, device="cuda")
        hla.damp_step(hi_d, lo_d, sc_d, dev(perm) if perm is not None else None, cfg.K_hi,
                      xd["q"], xd["k"], xd["v"], xd["alpha"], 1 if per else 0, xd["beta"],
                      out=out, slot=None if slot is None else dev(slot))
        x64 = f64_inputs(x, cfg.in_dtype)
        o_ref = oracle.damp_step(hi, lo, sc, perm, cfg.K_hi, x64["q"], x64["k"], x64["v"],
                                 x64["alpha"], x64["beta"], per_channel=per, slot=slot)
        w = _state_bars(_packed_host(hi_d, lo_d, sc_d), (hi, lo, sc), perm, cfg.K_hi, cfg.dk)
        live = np.ones(cfg.B, bool) if slot is None else slot >= 0
        o = host(out)
        w["out"] = rel_err_tiles(o[live], o_ref[live], 1)
        for key, val in w.items():
            worst[key] = max(worst.get(key, 0), val)
        assert (o[~live] == 3.0).all()
    return worst


@pytest.mark.parametrize("decay", ["vector", "scalar"])
@pytest.mark.parametrize("dk,dv,K_hi,use_perm", [
    (128, 128, 16, True), (128, 128, 16, False), (64, 64, 5, True), (128, 64, 0, True),
    (64, 128, 64, True), (128, 128, 128, False), (128, 128, 37, True)])
def test_step_teacher_forced(decay, dk, dv, K_hi, use_perm):
    hla = need_gpu()
    base = synth.CONFIGS["damp_kda"]
    cfg = synth.shrink(base, B=5, H=3, dk=dk, dv=dv, K_hi=K_hi, decay=decay,
                       seed=base.seed + dk + dv + K_hi)
    perm = _perm(np.random.default_rng(K_hi), cfg.H, dk) if use_perm else None
    slot = np.array([3, -1, 0, 5, 1], np.int32)
    w = _teacher_forced(hla, cfg, perm, steps=4, slot=slot, n_slots=6)
    print(w)
    _assert_bars(w)


@pytest.mark.parametrize("in_dtype", ["f32", "f16"])
def test_step_teacher_forced_input_types(in_dtype):
    """FP32 and IEEE binary16 projections (the serving shape's inputs are bf16) through
    the serving layout (K_hi = 16 of 128, per-channel decay, permuted plan)."""
    hla = need_gpu()
    base = synth.CONFIGS["damp_kda"]
    cfg = synth.shrink(base, B=5, H=3, in_dtype=in_dtype, seed=base.seed + 404)
    perm = _perm(np.random.default_rng(404), cfg.H, cfg.dk)
    slot = np.array([3, -1, 0, 5, 1], np.int32)
    w = _teacher_forced(hla, cfg, perm, steps=4, slot=slot, n_slots=6)
    _assert_bars(w)


def test_workload_plan_teacher_forced():
    """The mixed-precision workload's own plan (16 FP16 rows per head biased to slow
    decay), 32 heads, bf16 inputs, per-channel decay."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=8)
    w = _teacher_forced(hla, cfg, synth.damp_key_perm(cfg), steps=4)
    print(w)
    _assert_bars(w)


def test_many_heads_per_block_teacher_forced():
    """More heads than the GPU holds resident at once (1,280 heads with padding requests):
    workgroups are scheduled in several waves over the chip."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=40)
    slot = np.arange(cfg.B, dtype=np.int32)
    slot[[3, 17, 38]] = -1
    w = _teacher_forced(hla, cfg, synth.damp_key_perm(cfg), steps=2, slot=slot)
    print(w)
    _assert_bars(w)


@pytest.mark.parametrize("K_hi,decay", [(16, 1), (0, 1), (32, 0)])
def test_scale_buffer_alignment_does_not_change_results(K_hi, decay):
    """lo_scale only needs 4-byte alignment: a scale buffer 4 bytes off a 16-byte boundary
    gives the same bits as an aligned one, over 1,280 heads and 3 steps."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=40, K_hi=K_hi,
                       decay="vector" if decay else "scalar")
    perm = dev(synth.damp_key_perm(synth.shrink(cfg, K_hi=max(K_hi, 1))))
    hi0, lo0, sc0 = hla.damp_quantize(dev(synth.initial_state(cfg)), perm, K_hi)
    runs = []
    for misalign in (0, 1):
        hi, lo = hi0.clone(), lo0.clone()
        buf = torch.empty(sc0.numel() + 4, dtype=torch.float32, device="cuda")
        sc = buf[misalign:misalign + sc0.numel()].view(sc0.shape)
        sc.copy_(sc0)
        assert (sc.data_ptr() % 16 == 0) == (misalign == 0)
        outs = []
        for step in range(3):
            xd = dev_inputs(synth.step_inputs(cfg, step), cfg.in_dtype)
            outs.append(hla.damp_step(hi, lo, sc, perm, K_hi, xd["q"], xd["k"], xd["v"],
                                      xd["alpha"], decay, xd["beta"]))
        runs.append((hi, lo, sc.clone(), outs))
    (h0, l0, s0, o0), (h1, l1, s1, o1) = runs
    assert torch.equal(h0, h1) and torch.equal(l0, l1) and torch.equal(s0, s1)
    assert all(torch.equal(a, b) for a, b in zip(o0, o1))


def test_free_running_32_steps_drift():
    """Both sides run 32 steps of the quantised recurrence from the same packed state without
    re-synchronising.  Individual codes drift apart (a flipped code at a row maximum changes
    that row's scale, after which the two trajectories round independently: the error
    accumulation of DAMP section 3.3), so the bar here is statistical: each trajectory's drift
    from the unquantised FP32 recurrence (DAMP Eq. (8)) is of the same size on both sides."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=4)
    perm = synth.damp_key_perm(cfg)
    S0 = synth.initial_state(cfg).astype(np.float64)
    hi, lo, sc = oracle.damp_quantize(S0, perm, cfg.K_hi)
    S_fp = oracle.damp_dequantize(hi, lo, sc, perm, cfg.K_hi, cfg.dk)  # same start, unquantised
    hi_d, lo_d, sc_d = _packed_dev(hi, lo, sc)
    perm_d = dev(perm)
    report = {}
    for step in range(32):
        x = synth.step_inputs(cfg, step)
        xd = dev_inputs(x, cfg.in_dtype)
        o = hla.damp_step(hi_d, lo_d, sc_d, perm_d, cfg.K_hi, xd["q"], xd["k"], xd["v"],
                          xd["alpha"], 1, xd["beta"])
        x64 = f64_inputs(x, cfg.in_dtype)
        o_ref = oracle.damp_step(hi, lo, sc, perm, cfg.K_hi, x64["q"], x64["k"], x64["v"],
                                 x64["alpha"], x64["beta"], per_channel=True)
        o_fp = oracle.kda_step(S_fp, x64["q"], x64["k"], x64["v"], x64["alpha"], x64["beta"])
        if step in (0, 7, 31):
            g = _packed_host(hi_d, lo_d, sc_d)
            w = _state_bars(g, (hi, lo, sc), perm, cfg.K_hi, cfg.dk)
            s_g = oracle.damp_dequantize(*g, perm, cfg.K_hi, cfg.dk)
            s_o = oracle.damp_dequantize(hi, lo, sc, perm, cfg.K_hi, cfg.dk)
            nfp = np.linalg.norm(S_fp)
            w["drift_gpu"] = float(np.linalg.norm(s_g - S_fp) / nfp)
            w["drift_oracle"] = float(np.linalg.norm(s_o - S_fp) / nfp)
            on = np.linalg.norm(o_fp)
            w["out_drift_gpu"] = float(np.linalg.norm(host(o) - o_fp) / on)
            w["out_drift_oracle"] = float(np.linalg.norm(o_ref - o_fp) / on)
            report[step + 1] = w
    print(report)
    first = dict(report[1], out=0.0)
    _assert_bars(first)  # one step from the same state is the teacher-forced case
    for r in report.values():
        assert r["drift_gpu"] <= 1.5 * r["drift_oracle"] + 1e-4
        assert r["out_drift_gpu"] <= 1.5 * r["out_drift_oracle"] + 1e-4


def test_serving_shape_sampled_heads_teacher_forced():
    """Batch 256 x 32 heads in the benchmark's launch configuration: before each of 3
    steps the packed state of 48 sampled heads is read back, the oracle takes the same
    step from it, and the GPU's result for those heads is compared."""
    hla = need_gpu()
    cfg = synth.CONFIGS["damp_kda"]
    perm = synth.damp_key_perm(cfg)
    S0 = dev(synth.initial_state(cfg))
    hi_d, lo_d, sc_d = hla.damp_quantize(S0, dev(perm), cfg.K_hi)
    del S0
    pairs = sample_heads(np.random.default_rng(9), cfg.B, cfg.H, 48)
    bi = torch.tensor([b for b, _ in pairs], device="cuda")
    hh = torch.tensor([h for _, h in pairs], device="cuda")
    perm_d = dev(perm)
    for step in range(3):
        x = synth.step_inputs(cfg, step)
        hi_s, lo_s, sc_s = (hi_d[bi, hh][:, None].cpu().numpy().view(np.uint16).copy(),
                            lo_d[bi, hh][:, None].cpu().numpy().copy(),
                            sc_d[bi, hh][:, None].cpu().numpy().copy())
        xd = dev_inputs(x, cfg.in_dtype)
        o = hla.damp_step(hi_d, lo_d, sc_d, perm_d, cfg.K_hi, xd["q"], xd["k"], xd["v"],
                          xd["alpha"], 1, xd["beta"])
        xs = gather_heads(f64_inputs(x, cfg.in_dtype), pairs)
        # the oracle takes one head per sample, each with its own head's plan
        o_ref = np.zeros((len(pairs), cfg.dv))
        for i, (b, h) in enumerate(pairs):
            hs, ls, ss = hi_s[i:i + 1].copy(), lo_s[i:i + 1].copy(), sc_s[i:i + 1].copy()
            xi = {n: xs[n][i:i + 1] for n in xs}
            o_ref[i] = oracle.damp_step(hs, ls, ss, perm[h:h + 1], cfg.K_hi, xi["q"], xi["k"],
                                        xi["v"], xi["alpha"], xi["beta"], per_channel=True)[0, 0]
            hi_s[i], lo_s[i], sc_s[i] = hs[0], ls[0], ss[0]
        g = (hi_d[bi, hh][:, None].cpu().numpy().view(np.uint16),
             lo_d[bi, hh][:, None].cpu().numpy(), sc_d[bi, hh][:, None].cpu().numpy())
        for i, (b, h) in enumerate(pairs):
            w = _state_bars(tuple(a[i:i + 1] for a in g),
                            (hi_s[i:i + 1], lo_s[i:i + 1], sc_s[i:i + 1]), perm[h:h + 1],
                            cfg.K_hi, cfg.dk)
            w["out"] = 0.0
            _assert_bars(w)
        assert rel_err_tiles(host(o[bi, hh]), o_ref, 1) <= STATE_TOL


def test_bad_plan_entry_sets_flag():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=2, H=2)
    perm = np.tile(np.arange(cfg.dk, dtype=np.int32), (cfg.H, 1))
    perm[1, 3] = 500
    hi_d, lo_d, sc_d = hla.damp_quantize(dev(synth.initial_state(cfg)), None, cfg.K_hi)
    xd = dev_inputs(synth.step_inputs(cfg, 0), cfg.in_dtype)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.damp_step(hi_d, lo_d, sc_d, dev(perm), cfg.K_hi, xd["q"], xd["k"], xd["v"], xd["alpha"],
                  1, xd["beta"], err_flag=err)
    torch.cuda.synchronize()
    assert int(err.item()) == hla.DEVERR_PLAN

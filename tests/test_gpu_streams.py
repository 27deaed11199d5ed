"""The boundary's stream contract on the GPU: every launch goes on the caller's stream
(torch's current stream, or the `stream` argument), so it is ordered after work queued
there before it; and calls are reentrant, so steps of separate states issued on two
streams at once each match the float64 oracle.  Bar as for the step tests: per head
tile, max|gpu - oracle| <= 1e-5 * max|oracle|."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, rel_err_tiles, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")


def _busy(n=3072):
    """A few milliseconds of work on the current stream."""
    a = torch.randn((n, n), device="cuda")
    for _ in range(4):
        a = a @ a * (1.0 / n)
    return a


def test_step_is_ordered_on_the_callers_stream():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["gdn_serving"], B=16)
    S0 = synth.initial_state(cfg)
    src = dev(S0)
    xs = [synth.step_inputs(cfg, t) for t in range(2)]
    xd = [dev_inputs(x, cfg.in_dtype) for x in xs]
    st = torch.empty_like(src)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        st.fill_(float("nan"))
        keep = _busy()                        # delays the upload below on this stream only
        st.copy_(src)
        o1 = hla.gdn_step(st, *(xd[0][n] for n in NAMES))   # torch's current stream: side
    # the second step names the stream explicitly while the current stream is the default
    o2 = torch.empty_like(o1)
    hla.gdn_step(st, *(xd[1][n] for n in NAMES), out=o2, stream=side)
    side.synchronize()
    del keep
    S64 = S0.astype(np.float64)
    r1 = oracle.gdn_step(S64, *(f64_inputs(xs[0], cfg.in_dtype)[n] for n in NAMES))
    r2 = oracle.gdn_step(S64, *(f64_inputs(xs[1], cfg.in_dtype)[n] for n in NAMES))
    assert not np.isnan(host(st)).any()
    assert rel_err_tiles(host(o1), r1, 1) <= TOL
    assert rel_err_tiles(host(o2), r2, 1) <= TOL
    assert rel_err_tiles(host(st), S64) <= TOL


def test_two_streams_update_separate_states_concurrently():
    hla = need_gpu()
    runs = []
    for kind in ("gdn", "kda"):
        base = synth.CONFIGS["kda_serving" if kind == "kda" else "gdn_serving"]
        cfg = synth.shrink(base, B=12, seed=base.seed + 77)
        S0 = synth.initial_state(cfg)
        xs = [synth.step_inputs(cfg, t) for t in range(8)]
        runs.append(dict(kind=kind, cfg=cfg, S0=S0, xs=xs, st=dev(S0),
                         xd=[dev_inputs(x, cfg.in_dtype) for x in xs], outs=[]))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for t in range(8):                         # interleaved issue: both streams in flight
        for r, s in zip(runs, streams):
            fn = hla.kda_step if r["kind"] == "kda" else hla.gdn_step
            with torch.cuda.stream(s):
                r["outs"].append(fn(r["st"], *(r["xd"][t][n] for n in NAMES)))
    for s in streams:
        s.synchronize()
    for r in runs:
        S64 = r["S0"].astype(np.float64)
        fn = oracle.kda_step if r["kind"] == "kda" else oracle.gdn_step
        for t, x in enumerate(r["xs"]):
            o_ref = fn(S64, *(f64_inputs(x, r["cfg"].in_dtype)[n] for n in NAMES))
            assert rel_err_tiles(host(r["outs"][t]), o_ref, 1) <= TOL, (r["kind"], t)
        assert rel_err_tiles(host(r["st"]), S64) <= TOL, r["kind"]


def _case(hla, name):
    """(state tensors the call updates or reads, call(stream) -> outputs) for one entry
    point at a small shape; the state tensors are what the hazard below delays."""
    if name in ("replay", "bonus", "verify"):
        cfg = synth.shrink(synth.CONFIGS["dasc_gdn"], B=6, H=3, K=8)
        x = {k: dev(v) for k, v in synth.replay_inputs(cfg, 0).items()}
        xb = {k: dev(v) for k, v in synth.step_inputs(cfg, 5).items()}
        st = dev(synth.initial_state(cfg))

        def call(s, st=st):
            a = (st, x["q"], x["k"], x["v"], x["alpha"], x["beta"])
            if name == "replay":
                return [hla.replay_accepted(*a, x["n_accept"], 0, stream=s), st]
            if name == "bonus":
                return [hla.replay_accepted_bonus(*a, x["n_accept"], 0, xb["q"], xb["k"],
                                                  xb["v"], xb["alpha"], xb["beta"], stream=s),
                        st]
            return [hla.verify_drafts(*a, 0, stream=s)]
        return [st], call
    if name == "damp":
        cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=6, H=3)
        perm = dev(synth.damp_key_perm(cfg))
        codes = list(hla.damp_quantize(dev(synth.initial_state(cfg)), perm, cfg.K_hi))
        x = dev_inputs(synth.step_inputs(cfg, 1), cfg.in_dtype)

        def call(s, codes=codes):
            o = hla.damp_step(codes[0], codes[1], codes[2], perm, cfg.K_hi, x["q"], x["k"],
                              x["v"], x["alpha"], 1, x["beta"], stream=s)
            return [o] + codes
        return codes, call
    # the fused restore + replay from an INT8 checkpoint (whose codes are the hazard)
    cfg = synth.shrink(synth.CONFIGS["dasc_gdn"], H=3, dk=64, dv=64, K=4, L=2, slots=4)
    _, _, unit_pos, R = hla.dasc_plan(synth.dasc_masks(cfg))
    g = np.random.default_rng(3)
    codes = dev(g.integers(-127, 128, size=(cfg.slots, R, cfg.dk, cfg.dv)).astype(np.int8))
    scales = dev((g.uniform(0.5, 2.0, size=(cfg.slots, R, cfg.dk)) * 4e-4).astype(np.float32))
    xs = [synth.replay_inputs(cfg, l, B=3) for l in range(cfg.L)]
    x = {k: dev(np.stack([xl[k] for xl in xs])) for k in NAMES}
    ids = dev(np.array([2, 0, 3], np.int32))
    n_acc = dev(np.array([4, 0, 2], np.int32))

    def call(s, codes=codes):
        st = torch.full((cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv), 7.0, device="cuda")
        o = torch.zeros((cfg.L, 3, cfg.K, cfg.H, cfg.dv), device="cuda")
        pos = dev(unit_pos.reshape(-1))
        if s is not None:  # the fills and the upload above ran on the current stream
            s.wait_stream(torch.cuda.current_stream())
        hla.dasc_restore_int8_replay(codes, scales, pos, ids, ids, st, x["q"], x["k"], x["v"],
                                     x["alpha"], x["beta"], n_acc, 0, out=o, stream=s)
        return [o, st]
    return [codes], call


@pytest.mark.parametrize("name", ["replay", "bonus", "verify", "damp", "restore_int8_replay"])
def test_entry_points_ordered_on_the_callers_stream(name):
    """Each entry point, called with a side stream while that stream still has to finish a
    few milliseconds of work and then the upload of the operand the call reads, gives the
    same bits as the same call made with everything settled."""
    hla = need_gpu()
    tens, call = _case(hla, name)
    keep = [t.clone() for t in tens]
    ref = [t.clone() for t in call(None)]          # everything settled, default stream
    torch.cuda.synchronize()
    for t, k in zip(tens, keep):
        t.copy_(k)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for t in tens:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        busy = _busy()                              # delays the uploads below on this stream
        for t, k in zip(tens, keep):
            t.copy_(k)
    got = call(side)                               # the stream named explicitly
    side.synchronize()
    del busy
    assert len(got) == len(ref)
    for a, b in zip(got, ref):
        assert torch.equal(a, b), name

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

"""The entry points launched under HIP graph capture (as a decode loop runs them) give the
same results as the same launches issued eagerly: bitwise, on every replay, with eager work
and synchronisations between the replays."""
import numpy as np
import pytest

import synth
from gpu_util import dev, dev_inputs, need_gpu, torch

pytestmark = pytest.mark.gpu
REPLAYS = 4


def _check_replays(launch, eager_state, graph_state):
    """launch(state, i) issues step i on `state`.  The graph holds steps 0 and 1; every
    replay is compared with the eager state after the same steps."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(graph_state, 0)
        launch(graph_state, 1)
    for r in range(REPLAYS):
        g.replay()
        launch(eager_state, 0)  # eager work between replays
        launch(eager_state, 1)
        torch.cuda.synchronize()
        for a, b in zip(eager_state, graph_state):
            assert torch.equal(a, b), f"replay {r} differs from eager"


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_step_graph_replays(kind):
    hla = need_gpu()
    base = synth.CONFIGS["kda_serving" if kind == "kda" else "gdn_serving"]
    cfg = synth.shrink(base, B=9, H=5)
    fn = hla.kda_step if kind == "kda" else hla.gdn_step
    xs = [dev_inputs(synth.step_inputs(cfg, s), cfg.in_dtype) for s in range(2)]
    S0 = synth.initial_state(cfg)
    st_e, st_g = dev(S0), dev(S0)
    out_e = torch.empty((cfg.B, cfg.H, cfg.dv), device="cuda")
    out_g = torch.empty_like(out_e)

    def launch(state, i):
        x = xs[i]
        o = out_e if state[0] is st_e else out_g
        fn(state[0], x["q"], x["k"], x["v"], x["alpha"], x["beta"], out=o)

    _check_replays(launch, [st_e, out_e], [st_g, out_g])


def test_damp_graph_replays():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["damp_kda"], B=6, H=4)
    perm = dev(synth.damp_key_perm(cfg))
    S0 = dev(synth.initial_state(cfg))
    codes_e = list(hla.damp_quantize(S0, perm, cfg.K_hi))
    codes_g = [c.clone() for c in codes_e]
    xs = [dev_inputs(synth.step_inputs(cfg, s), cfg.in_dtype) for s in range(2)]
    out_e = torch.empty((cfg.B, cfg.H, cfg.dv), device="cuda")
    out_g = torch.empty_like(out_e)

    def launch(state, i):
        x = xs[i]
        o = out_e if state[0] is codes_e[0] else out_g
        hla.damp_step(state[0], state[1], state[2], perm, cfg.K_hi, x["q"], x["k"], x["v"],
                      x["alpha"], 1, x["beta"], out=o)

    _check_replays(launch, codes_e + [out_e], codes_g + [out_g])


def test_replay_accepted_graph_replays():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["dasc_gdn"], B=7, H=3)
    x = {k: dev(v) for k, v in synth.replay_inputs(cfg, 0).items()}
    S0 = synth.initial_state(cfg)
    st_e, st_g = dev(S0), dev(S0)
    out_e = torch.zeros((cfg.B, cfg.K, cfg.H, cfg.dv), device="cuda")  # rows past n_accept
    out_g = torch.zeros_like(out_e)                                    # are left as they are

    def launch(state, i):
        o = out_e if state[0] is st_e else out_g
        hla.replay_accepted(state[0], x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                            x["n_accept"], 0, out=o)

    _check_replays(launch, [st_e, out_e], [st_g, out_g])


def test_verify_and_bonus_graph_replays():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["dasc_gdn"], B=5, H=3, decay="vector")
    x = {k: dev(v) for k, v in synth.replay_inputs(cfg, 1).items()}
    xb = {k: dev(v) for k, v in synth.step_inputs(cfg, 30_000).items()}
    S0 = synth.initial_state(cfg)
    st_e, st_g = dev(S0), dev(S0)
    ov_e = torch.zeros((cfg.B, cfg.K, cfg.H, cfg.dv), device="cuda")
    ov_g = torch.zeros_like(ov_e)
    ob_e = torch.zeros((cfg.B, cfg.H, cfg.dv), device="cuda")
    ob_g = torch.zeros_like(ob_e)

    def launch(state, i):
        eager = state[0] is st_e
        st = state[0]
        hla.verify_drafts(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"], 1,
                          out=ov_e if eager else ov_g)
        hla.replay_accepted_bonus(st, x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                  x["n_accept"], 1, xb["q"], xb["k"], xb["v"], xb["alpha"],
                                  xb["beta"], out_bonus=ob_e if eager else ob_g)

    _check_replays(launch, [st_e, ov_e, ob_e], [st_g, ov_g, ob_g])


def test_dasc_int8_graph_replays():
    hla = need_gpu()
    import numpy as np

    g = np.random.default_rng(5)
    L, S_, n_units, dv = 2, 3, 24, 128
    act = dev((g.standard_normal((L, S_, n_units, 1, dv)) * 0.05).astype(np.float32))
    mask = (g.random((L, n_units)) < 0.5).astype(np.uint8)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    ids = dev(np.arange(S_, dtype=np.int32))
    stride = S_ * n_units * dv * 4
    tabs = [dev(offsets), dev(unit_index), dev(unit_pos.reshape(-1))]
    bufs = {}
    for side in ("e", "g"):
        bufs[side] = [torch.zeros((S_, R, 1, dv), dtype=torch.int8, device="cuda"),
                      torch.zeros((S_, R, 1), device="cuda"), torch.zeros_like(act)]

    def launch(state, i):
        codes, scales, out = state
        hla.dasc_pack_int8(act, stride, S_, L, n_units, 1, dv, tabs[0], tabs[1], R, ids, ids,
                           codes, scales, S_)
        hla.dasc_restore_int8(codes, scales, S_, R, tabs[2], L, n_units, 1, dv, ids, ids, out,
                              stride, S_)

    _check_replays(launch, bufs["e"], bufs["g"])


@pytest.mark.parametrize("q8", [False, True])
def test_restore_replay_graph_replays(q8):
    """The fused restore + replay from an FP32 or an INT8 checkpoint, with readouts."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["dasc_gdn"], H=3, dk=64, dv=64, K=4, L=2, slots=4)
    mask = synth.dasc_masks(cfg)
    _, _, unit_pos, R = hla.dasc_plan(mask)
    g = np.random.default_rng(7)
    packed = dev((g.standard_normal((cfg.slots, R, cfg.dk * cfg.dv)) * 0.05).astype(np.float32))
    codes = dev(g.integers(-127, 128, size=(cfg.slots, R, cfg.dk, cfg.dv)).astype(np.int8))
    scales = dev((g.uniform(0.5, 2.0, size=(cfg.slots, R, cfg.dk)) * 4e-4).astype(np.float32))
    pos = dev(unit_pos.reshape(-1))
    src = dev(np.array([2, 0, 3], np.int32))
    dst = dev(np.array([1, 3, 0], np.int32))
    xs = [synth.replay_inputs(cfg, l, B=3) for l in range(cfg.L)]
    x = {k: dev(np.stack([xl[k] for xl in xs])) for k in ("q", "k", "v", "alpha", "beta")}
    n_acc = dev(np.array([4, 0, 2], np.int32))
    bufs = {}
    for side in ("e", "g"):
        bufs[side] = [torch.full((cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv), 7.0, device="cuda"),
                      torch.zeros((cfg.L, 3, cfg.K, cfg.H, cfg.dv), device="cuda")]

    def launch(state, i):
        args = (pos, src, dst, state[0], x["q"], x["k"], x["v"], x["alpha"], x["beta"], n_acc, 0)
        if q8:
            hla.dasc_restore_int8_replay(codes, scales, *args, out=state[1])
        else:
            hla.dasc_restore_replay(packed, *args, out=state[1])

    _check_replays(launch, bufs["e"], bufs["g"])

"""Edge cases of the GPU entry points, checked against the float64 oracle or against what
the definition fixes: empty batches, every request padded, the largest and smallest draft
counts, one head, and degenerate decays (alpha = 0 forgets the state: S = beta k v^T;
alpha = 1 with beta = 0 leaves it unchanged)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, rel_err_tiles, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")


def test_empty_batches_launch_nothing():
    hla = need_gpu()
    st = torch.randn(3, 2, 64, 64, device="cuda")
    before = st.clone()
    z = lambda *s: torch.zeros(*s, device="cuda")  # noqa: E731
    out = hla.gdn_step(st, z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), z(0, 2), z(0, 2))
    assert out.shape == (0, 2, 64)
    hla.kda_step(st, z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), z(0, 2))
    n0 = torch.zeros(0, dtype=torch.int32, device="cuda")
    hla.replay_accepted(st, z(0, 4, 2, 64), z(0, 4, 2, 64), z(0, 4, 2, 64), z(0, 4, 2),
                        z(0, 4, 2), n0, 0)
    hla.verify_drafts(st, z(0, 4, 2, 64), z(0, 4, 2, 64), z(0, 4, 2, 64), z(0, 4, 2),
                      z(0, 4, 2), 0)
    hla.replay_accepted_bonus(st, z(0, 4, 2, 64), z(0, 4, 2, 64), z(0, 4, 2, 64), z(0, 4, 2),
                              z(0, 4, 2), n0, 0, z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), z(0, 2),
                              z(0, 2))
    hi, lo, sc = hla.damp_quantize(st, None, 8)
    hla.damp_step(hi, lo, sc, None, 8, z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), 1,
                  z(0, 2))
    torch.cuda.synchronize()
    assert torch.equal(st, before)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_all_requests_padded(kind):
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["kda_serving" if kind == "kda" else "gdn_serving"], B=4,
                       H=3)
    S0 = synth.initial_state(cfg)
    st = dev(S0)
    xd = dev_inputs(synth.step_inputs(cfg, 0), cfg.in_dtype)
    out = torch.full((cfg.B, cfg.H, cfg.dv), 9.0, device="cuda")
    fn = hla.kda_step if kind == "kda" else hla.gdn_step
    fn(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], out=out,
       slot=dev(np.full(cfg.B, -1, np.int32)))
    assert np.array_equal(host(st), S0) and (host(out) == 9.0).all()


@pytest.mark.parametrize("K", [1, 16])
@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_draft_count_limits(K, kind):
    """K = 1 and the largest supported K = 16: replay (all accepted), verify and the fused
    bonus against the oracle."""
    hla = need_gpu()
    base = synth.CONFIGS["dasc_gdn"]
    cfg = synth.shrink(base, B=3, H=2, K=K, decay="vector" if kind == "kda" else "scalar",
                       seed=base.seed + K)
    x = synth.replay_inputs(cfg, 0)
    xb = synth.step_inputs(cfg, 20_000)
    n_acc = np.full(cfg.B, K, np.int32)
    S0 = synth.initial_state(cfg)
    xd = {n: dev(x[n]) for n in NAMES}
    bd = {n: dev(xb[n]) for n in NAMES}
    x64 = f64_inputs({n: x[n] for n in NAMES}, "f32")
    b64 = f64_inputs(xb, "f32")
    dkind = 1 if kind == "kda" else 0
    per = kind == "kda"
    ov = hla.verify_drafts(dev(S0), xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], dkind)
    ov_ref = oracle.verify(S0.astype(np.float64), x64["q"], x64["k"], x64["v"], x64["alpha"],
                           x64["beta"], per_channel=per)
    assert rel_err_tiles(host(ov), ov_ref, 1) <= TOL
    st = dev(S0)
    ob = hla.replay_accepted_bonus(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                   dev(n_acc), dkind, bd["q"], bd["k"], bd["v"], bd["alpha"],
                                   bd["beta"])
    S64 = S0.astype(np.float64)
    _, ob_ref = oracle.replay_bonus(S64, x64["q"], x64["k"], x64["v"], x64["alpha"],
                                    x64["beta"], n_acc, b64["q"], b64["k"], b64["v"],
                                    b64["alpha"], b64["beta"], per_channel=per)
    assert rel_err_tiles(host(st), S64) <= TOL
    assert rel_err_tiles(host(ob), ob_ref, 1) <= TOL


def test_single_head_smallest_shape():
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["gdn_toy"], B=1, H=1)
    S64 = synth.initial_state(cfg).astype(np.float64)
    st = dev(synth.initial_state(cfg))
    for step in range(5):
        x = synth.step_inputs(cfg, step)
        o = hla.gdn_step(st, *(dev(x[n]) for n in NAMES))
        o_ref = oracle.gdn_step(S64, *(x[n].astype(np.float64) for n in NAMES))
        assert rel_err_tiles(host(o), o_ref, 1) <= TOL
    assert rel_err_tiles(host(st), S64) <= TOL


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_degenerate_decays(kind):
    """alpha = 0: the old state is forgotten, S = beta k v^T and o = beta (q.k) v exactly as
    the oracle computes them; alpha = 1 with beta = 0: nothing changes, bit for bit."""
    hla = need_gpu()
    cfg = synth.shrink(synth.CONFIGS["kda_serving" if kind == "kda" else "gdn_serving"], B=3,
                       H=2, in_dtype="f32")
    fn = hla.kda_step if kind == "kda" else hla.gdn_step
    ofn = oracle.kda_step if kind == "kda" else oracle.gdn_step
    S0 = synth.initial_state(cfg)
    x = synth.step_inputs(cfg, 0)
    x["alpha"] = np.zeros_like(x["alpha"])
    st = dev(S0)
    o = fn(st, *(dev(x[n]) for n in NAMES))
    S64 = S0.astype(np.float64)
    o_ref = ofn(S64, *(x[n].astype(np.float64) for n in NAMES))
    closed = x["beta"][..., None, None] * x["k"][..., :, None].astype(np.float64) * \
        x["v"][..., None, :].astype(np.float64)
    np.testing.assert_allclose(S64, closed, rtol=0, atol=1e-15)
    assert rel_err_tiles(host(st), S64) <= TOL and rel_err_tiles(host(o), o_ref, 1) <= TOL
    x["alpha"] = np.ones_like(x["alpha"])
    x["beta"] = np.zeros_like(x["beta"])
    st = dev(S0)
    fn(st, *(dev(x[n]) for n in NAMES))
    assert np.array_equal(host(st), S0)

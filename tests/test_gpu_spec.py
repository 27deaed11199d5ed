"""GPU parity of the speculative-decoding entry points against the float64 oracle:
verify_drafts (readouts at all K draft positions, committed state only read) and
replay_accepted_bonus (accepted drafts, then the bonus token, in one pass over the state).
Tolerance as the FP32 step: per head tile, max|gpu - oracle| <= 1e-5 * max|oracle|.
Bitwise checks: verify leaves the state's bits alone and the fused bonus equals
replay_accepted followed by one step call; verify's readouts match a full-acceptance
replay's to the FP32 tolerance (verify evaluates the drafts in unrolled form)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (dev, dev_inputs, f64_inputs, gather_heads, host, need_gpu, rel_err_tiles,
                      sample_heads, torch)

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")


def _cfg(kind, dk, dv, in_dtype, B, K, H=3):
    base = synth.CONFIGS["dasc_gdn"]
    return synth.shrink(base, B=B, K=K, H=H, dk=dk, dv=dv, in_dtype=in_dtype,
                        decay="vector" if kind == "kda" else "scalar",
                        seed=base.seed + 5 * dk + dv + (11 if kind == "kda" else 0))


def _bonus(cfg, layer):
    """The bonus token's projections: an ordinary step's inputs ([B, H, .])."""
    return synth.step_inputs(cfg, 10_000 + layer)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_verify_matches_oracle_and_reads_only(kind, in_dtype, dk, dv):
    hla = need_gpu()
    cfg = _cfg(kind, dk, dv, in_dtype, B=5, K=6)
    x = synth.replay_inputs(cfg, 0)
    n_slots = 7
    slot = np.array([6, -1, 2, 0, 4], np.int32)
    S0 = synth.initial_state(cfg, S=n_slots)
    st = dev(S0)
    xd = dev_inputs({n: x[n] for n in NAMES}, in_dtype)
    out = torch.full((cfg.B, cfg.K, cfg.H, dv), 7.0, device="cuda")
    hla.verify_drafts(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                      1 if kind == "kda" else 0, out=out, slot=dev(slot))
    x64 = f64_inputs({n: x[n] for n in NAMES}, in_dtype)
    o_ref = oracle.verify(S0.astype(np.float64), x64["q"], x64["k"], x64["v"], x64["alpha"],
                          x64["beta"], per_channel=(kind == "kda"), slot=slot)
    assert np.array_equal(host(st), S0)  # the committed state is not written
    o = host(out)
    live = slot >= 0
    assert rel_err_tiles(o[live], o_ref[live], 1) <= TOL
    assert (o[~live] == 7.0).all()


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_verify_readouts_match_full_acceptance_replay(kind):
    """The verify pass (unrolled form) and a replay accepting every draft (token by token)
    compute the same readouts from the same state, up to summation order."""
    hla = need_gpu()
    cfg = _cfg(kind, 128, 128, "bf16", B=8, K=8, H=4)
    x = synth.replay_inputs(cfg, 2)
    S0 = synth.initial_state(cfg)
    st = dev(S0)
    xd = dev_inputs({n: x[n] for n in NAMES}, "bf16")
    dk = 1 if kind == "kda" else 0
    o_v = hla.verify_drafts(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], dk)
    assert np.array_equal(host(st), S0)
    full = dev(np.full(cfg.B, cfg.K, np.int32))
    o_r = hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], full, dk)
    assert rel_err_tiles(host(o_v), host(o_r), 1) <= 2 * TOL


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
@pytest.mark.parametrize("K", [4, 12])
def test_replay_bonus_matches_oracle(kind, in_dtype, dk, dv, K):
    """K = 12 takes requests with 7 or more accepted tokens through the path that stages
    their inputs in LDS; K = 4 through the token-by-token loads."""
    hla = need_gpu()
    cfg = _cfg(kind, dk, dv, in_dtype, B=6, K=K)
    x = synth.replay_inputs(cfg, 0)
    xb = _bonus(cfg, 0)
    n_acc = np.array([0, 1, K, K // 2 + 1, K + 5, -3], np.int32)  # K + 5, -3 clamp to K, 0
    S0 = synth.initial_state(cfg)
    S64 = S0.astype(np.float64)
    st = dev(S0)
    xd = dev_inputs({n: x[n] for n in NAMES}, in_dtype)
    bd = dev_inputs(xb, in_dtype)
    out = torch.full((cfg.B, cfg.K, cfg.H, dv), 5.0, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ob = hla.replay_accepted_bonus(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                   dev(n_acc), 1 if kind == "kda" else 0, bd["q"], bd["k"],
                                   bd["v"], bd["alpha"], bd["beta"], out=out, err_flag=err)
    x64, b64 = f64_inputs({n: x[n] for n in NAMES}, in_dtype), f64_inputs(xb, in_dtype)
    o_ref, ob_ref = oracle.replay_bonus(S64, x64["q"], x64["k"], x64["v"], x64["alpha"],
                                        x64["beta"], n_acc, b64["q"], b64["k"], b64["v"],
                                        b64["alpha"], b64["beta"], per_channel=(kind == "kda"),
                                        want_out=True)
    assert int(err.item()) == hla.DEVERR_ACCEPT
    assert rel_err_tiles(host(st), S64) <= TOL
    assert rel_err_tiles(host(ob), ob_ref, 1) <= TOL
    o = host(out)
    for b, n in enumerate(np.clip(n_acc, 0, cfg.K)):
        if n:
            assert rel_err_tiles(o[b, :n], o_ref[b, :n], 1) <= TOL
        assert (o[b, n:] == 5.0).all()


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_fused_bonus_is_bitwise_replay_then_step(kind):
    hla = need_gpu()
    cfg = _cfg(kind, 128, 128, "bf16", B=12, K=8, H=4)
    x = synth.replay_inputs(cfg, 3)
    xb = _bonus(cfg, 3)
    S0 = synth.initial_state(cfg)
    fused, seq = dev(S0), dev(S0)
    xd = dev_inputs({n: x[n] for n in NAMES}, "bf16")
    bd = dev_inputs(xb, "bf16")
    n_acc = dev(x["n_accept"])
    dkind = 1 if kind == "kda" else 0
    ob = hla.replay_accepted_bonus(fused, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                   n_acc, dkind, bd["q"], bd["k"], bd["v"], bd["alpha"],
                                   bd["beta"])
    hla.replay_accepted(seq, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], n_acc, dkind,
                        want_out=False)
    step = hla.kda_step if kind == "kda" else hla.gdn_step
    o1 = step(seq, bd["q"], bd["k"], bd["v"], bd["alpha"], bd["beta"])
    assert torch.equal(fused, seq) and torch.equal(ob, o1)


def test_checkpoint_workload_shape_sampled_heads():
    """512 request states x 32 heads x 128 x 128, K = 8 drafts, accepted counts U{0..8}:
    verify over all drafts, then the fused replay + bonus; 32 sampled heads of each
    against the oracle."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    x = synth.replay_inputs(cfg, 0)
    xb = _bonus(cfg, 0)
    S0 = synth.initial_state(cfg, S=cfg.slots)
    st = dev(S0)
    xd = dev_inputs({n: x[n] for n in NAMES}, cfg.in_dtype)
    bd = dev_inputs(xb, cfg.in_dtype)
    o_v = hla.verify_drafts(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], 0)
    ob = hla.replay_accepted_bonus(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                   dev(x["n_accept"]), 0, bd["q"], bd["k"], bd["v"],
                                   bd["alpha"], bd["beta"])
    pairs = sample_heads(np.random.default_rng(15), cfg.B, cfg.H, 32)
    xs = gather_heads(f64_inputs({n: x[n] for n in NAMES}, cfg.in_dtype), pairs,
                      per_token_axes=2)
    bs = gather_heads(f64_inputs(xb, cfg.in_dtype), pairs)
    S64 = np.stack([S0[b, h:h + 1] for b, h in pairs]).astype(np.float64)
    ov_ref = oracle.verify(S64, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"],
                           per_channel=False)
    n_s = np.array([x["n_accept"][b] for b, _ in pairs], np.int32)
    _, ob_ref = oracle.replay_bonus(S64, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"],
                                    n_s, bs["q"], bs["k"], bs["v"], bs["alpha"], bs["beta"],
                                    per_channel=False)
    bi = torch.tensor([b for b, _ in pairs], device="cuda")
    hi = torch.tensor([h for _, h in pairs], device="cuda")
    assert rel_err_tiles(host(o_v[bi, :, hi]), ov_ref[:, :, 0], 1) <= TOL
    assert rel_err_tiles(host(st[bi, hi]), S64[:, 0]) <= TOL
    assert rel_err_tiles(host(ob[bi, hi]), ob_ref[:, 0], 1) <= TOL

"""GPU parity of replay_accepted against the float64 oracle, and bitwise equality of
the fused replay with the same tokens applied by single gdn_step / kda_step calls."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (dev, dev_inputs, f64_inputs, gather_heads, host, need_gpu, rel_err_tiles,
                      sample_heads, torch)

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _cfg(kind, dk, dv, in_dtype, B, K, H=3):
    base = synth.CONFIGS["dasc_gdn"]
    return synth.shrink(base, B=B, K=K, H=H, dk=dk, dv=dv, in_dtype=in_dtype,
                        decay="vector" if kind == "kda" else "scalar",
                        seed=base.seed + dk + 3 * dv + (7 if kind == "kda" else 0))


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("K", [4, 12])
def test_replay_matches_oracle_with_clamping(kind, in_dtype, dk, dv, K):
    """K = 12 takes requests with 7 or more accepted tokens through the path that stages
    their inputs in LDS; K = 4 through the token-by-token loads."""
    hla = need_gpu()
    cfg = _cfg(kind, dk, dv, in_dtype, B=6, K=K)
    x = synth.replay_inputs(cfg, 0)
    n_acc = np.array([0, 1, K, K // 2 + 1, K + 5, -3], np.int32)  # K + 5, -3 clamp to K, 0
    S0 = synth.initial_state(cfg)
    S64 = S0.astype(np.float64)
    st = dev(S0)
    xd = dev_inputs({n: x[n] for n in ("q", "k", "v", "alpha", "beta")}, in_dtype)
    out = torch.full((cfg.B, cfg.K, cfg.H, dv), 5.0, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], dev(n_acc),
                        1 if kind == "kda" else 0, out=out, err_flag=err)
    x64 = f64_inputs(x, in_dtype)
    o_ref = oracle.replay(S64, x64["q"], x64["k"], x64["v"], x64["alpha"], x64["beta"], n_acc,
                          per_channel=(kind == "kda"))
    assert int(err.item()) == hla.DEVERR_ACCEPT
    assert rel_err_tiles(host(st), S64) <= TOL
    o = host(out)
    n_eff = np.clip(n_acc, 0, cfg.K)
    for b in range(cfg.B):
        n = n_eff[b]
        if n:
            assert rel_err_tiles(o[b, :n], o_ref[b, :n], 1) <= TOL
        assert (o[b, n:] == 5.0).all()
    got = host(st)
    assert np.array_equal(got[0], S0[0]) and np.array_equal(got[5], S0[5])  # n = 0: untouched


@pytest.mark.parametrize("kind", ["gdn", "kda"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 128), (128, 64)])
def test_replay_without_readouts_gives_the_same_state(kind, in_dtype, dk, dv):
    """Without readouts (out NULL) the replay skips the readout terms and q; the state
    must be the same bits as with readouts, for requests loaded token by token and for
    those staged in LDS (7 or more of K = 12 accepted).  The replay + bonus without draft
    readouts: the same state and the same bonus readout as with them."""
    hla = need_gpu()
    cfg = _cfg(kind, dk, dv, in_dtype, B=8, K=12)
    x = synth.replay_inputs(cfg, 2)
    xb = synth.step_inputs(cfg, 77)
    n_acc = dev(np.array([0, 1, 3, 6, 7, 9, 12, 12], np.int32))
    S0 = synth.initial_state(cfg)
    xd = dev_inputs({n: x[n] for n in ("q", "k", "v", "alpha", "beta")}, in_dtype)
    bd = dev_inputs({n: xb[n] for n in ("q", "k", "v", "alpha", "beta")}, in_dtype)
    vec = 1 if kind == "kda" else 0
    with_o, without = dev(S0), dev(S0)
    hla.replay_accepted(with_o, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], n_acc, vec)
    hla.replay_accepted(without, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], n_acc, vec,
                        want_out=False)
    assert torch.equal(with_o, without)
    with_o, without = dev(S0), dev(S0)
    drafts_out = torch.empty((cfg.B, cfg.K, cfg.H, dv), device="cuda")
    ob1 = hla.replay_accepted_bonus(with_o, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                    n_acc, vec, bd["q"], bd["k"], bd["v"], bd["alpha"],
                                    bd["beta"], out=drafts_out)
    ob2 = hla.replay_accepted_bonus(without, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                    n_acc, vec, bd["q"], bd["k"], bd["v"], bd["alpha"],
                                    bd["beta"])
    assert torch.equal(with_o, without) and torch.equal(ob1, ob2)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_fused_replay_is_bitwise_equal_to_single_steps(kind):
    """Token t of every request is applied by one step call whose slot map pads out the
    requests with n_b <= t; the fused replay must give the same bits."""
    hla = need_gpu()
    cfg = _cfg(kind, 128, 128, "bf16", B=12, K=8, H=4)
    x = synth.replay_inputs(cfg, 1)
    n_acc = x["n_accept"]
    S0 = synth.initial_state(cfg)
    fused, seq = dev(S0), dev(S0)
    xd = dev_inputs({n: x[n] for n in ("q", "k", "v", "alpha", "beta")}, "bf16")
    out_f = hla.replay_accepted(fused, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                                dev(n_acc), 1 if kind == "kda" else 0)
    step = hla.kda_step if kind == "kda" else hla.gdn_step
    for t in range(cfg.K):
        slot = dev(np.where(n_acc > t, np.arange(cfg.B), -1).astype(np.int32))
        o_t = step(seq, xd["q"][:, t].contiguous(), xd["k"][:, t].contiguous(),
                   xd["v"][:, t].contiguous(), xd["alpha"][:, t].contiguous(),
                   xd["beta"][:, t].contiguous(), slot=slot)
        live = torch.from_numpy(n_acc > t).cuda()
        assert torch.equal(o_t[live], out_f[:, t][live])
    assert torch.equal(fused, seq)


def test_checkpoint_workload_shape_sampled_heads():
    """512 request states x 32 heads x 128 x 128, K = 8 drafts, accepted counts U{0..8}:
    48 sampled heads against the oracle."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    x = synth.replay_inputs(cfg, 0)
    S0 = synth.initial_state(cfg, S=cfg.slots)
    st = dev(S0)
    xd = dev_inputs({n: x[n] for n in ("q", "k", "v", "alpha", "beta")}, cfg.in_dtype)
    out = torch.zeros((cfg.B, cfg.K, cfg.H, cfg.dv), device="cuda")
    hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                        dev(x["n_accept"]), 0, out=out)
    pairs = sample_heads(np.random.default_rng(5), cfg.B, cfg.H, 48)
    xs = gather_heads(f64_inputs({n: x[n] for n in ("q", "k", "v", "alpha", "beta")},
                                 cfg.in_dtype), pairs, per_token_axes=2)
    n_s = np.array([x["n_accept"][b] for b, _ in pairs], np.int32)
    S64 = np.stack([S0[b, h:h + 1] for b, h in pairs]).astype(np.float64)
    o_ref = oracle.replay(S64, xs["q"], xs["k"], xs["v"], xs["alpha"], xs["beta"], n_s,
                          per_channel=False)
    bi = torch.tensor([b for b, _ in pairs], device="cuda")
    hi = torch.tensor([h for _, h in pairs], device="cuda")
    assert rel_err_tiles(host(st[bi, hi]), S64[:, 0]) <= TOL
    o = host(out[bi, :, hi])  # [48, K, dv]
    for i, n in enumerate(n_s):
        if n:
            assert rel_err_tiles(o[i, :n], o_ref[i, :n, 0], 1) <= TOL

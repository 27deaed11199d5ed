"""States larger than 4 GiB.  The kernels form a head's address in 64-bit arithmetic (and
only offsets inside one head in 32 bits), so requests mapped to slots past the first
4 GiB of a state must update exactly as the oracle says.  Each test allocates one state
above 4 GiB on the device (random values drawn there), maps a few requests to slots on
both sides of the boundary, and compares those heads with the float64 oracle taking the
same step from the same (read-back) values."""
import numpy as np
import pytest

import oracle
import synth
from damp_util import _assert_bars, _state_bars
from gpu_util import dev, dev_inputs, f64_inputs, host, need_gpu, rel_err_tiles, torch

pytestmark = pytest.mark.gpu
TOL = 1e-5
NAMES = ("q", "k", "v", "alpha", "beta")
GIB4 = 1 << 32


def _slots_across(n_slots, slot_bytes, n_far=2):
    """Slot ids on both sides of the 4 GiB boundary, plus the first and the last."""
    b = GIB4 // slot_bytes
    ids = [0, b - 1, b, b + 1, n_slots - 1] + [b + 2 + i for i in range(n_far)]
    ids = sorted(set(i for i in ids if 0 <= i < n_slots))
    assert ids[-1] * slot_bytes >= GIB4
    return np.array(ids, np.int32)


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_step_verify_replay_beyond_4gib(kind):
    hla = need_gpu()
    base = synth.CONFIGS["kda_serving" if kind == "kda" else "gdn_serving"]
    H, dk, dv = base.H, base.dk, base.dv
    slot_bytes = H * dk * dv * 4
    n_slots = GIB4 // slot_bytes + 32                     # 2080 slots, 4.36 GB
    gen = torch.Generator(device="cuda").manual_seed(5)
    st = torch.randn((n_slots, H, dk, dv), device="cuda", generator=gen) * 0.05
    slots = _slots_across(n_slots, slot_bytes)
    B = len(slots)
    sd = dev(slots)
    S64 = host(st[sd.long()]).astype(np.float64)
    per = kind == "kda"

    # one step through the slot map
    cfg = synth.shrink(base, B=B)
    x = synth.step_inputs(cfg, 0)
    fn = hla.kda_step if per else hla.gdn_step
    o = fn(st, *(dev_inputs(x, cfg.in_dtype)[n] for n in NAMES), slot=sd)
    x64 = f64_inputs(x, cfg.in_dtype)
    o_ref = (oracle.kda_step if per else oracle.gdn_step)(S64, *(x64[n] for n in NAMES))
    assert rel_err_tiles(host(st[sd.long()]), S64) <= TOL
    assert rel_err_tiles(host(o), o_ref, 1) <= TOL

    # verify (the state only read) and a replay, K = 8 drafts, same slots
    dcfg = synth.shrink(synth.CONFIGS["dasc_gdn"], B=B, H=H,
                        decay="vector" if per else "scalar", seed=base.seed + 31)
    xr = synth.replay_inputs(dcfg, 0)
    xd = {n: dev(xr[n]) for n in NAMES}
    before = host(st[sd.long()])
    ov = hla.verify_drafts(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], int(per),
                           slot=sd)
    assert np.array_equal(host(st[sd.long()]), before)
    r64 = {n: xr[n].astype(np.float64) for n in NAMES}
    ov_ref = oracle.verify(S64, r64["q"], r64["k"], r64["v"], r64["alpha"], r64["beta"],
                           per_channel=per)
    assert rel_err_tiles(host(ov), ov_ref, 1) <= TOL
    hla.replay_accepted(st, xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"],
                        dev(xr["n_accept"]), int(per), slot=sd)
    oracle.replay(S64, r64["q"], r64["k"], r64["v"], r64["alpha"], r64["beta"], xr["n_accept"],
                  per_channel=per)
    assert rel_err_tiles(host(st[sd.long()]), S64) <= TOL


def test_damp_step_beyond_4gib():
    """The packed INT8 rows of the mixed-precision state span more than 4 GiB (9,400
    slots x 32 heads x 14,336 B); random codes, scales and FP16 rows drawn on the device."""
    hla = need_gpu()
    cfg0 = synth.CONFIGS["damp_kda"]
    H, dk, dv, K_hi = cfg0.H, cfg0.dk, cfg0.dv, cfg0.K_hi
    lo_slot = H * (dk - K_hi) * dv
    n_slots = GIB4 // lo_slot + 38                        # 9,400 slots
    gen = torch.Generator(device="cuda").manual_seed(6)
    hi_d = (torch.randn((n_slots, H, K_hi, dv), device="cuda", generator=gen) * 0.05
            ).half().view(torch.int16)
    lo_d = torch.randint(-127, 128, (n_slots, H, dk - K_hi, dv), device="cuda",
                         generator=gen, dtype=torch.int8)
    sc_d = torch.rand((n_slots, H, dk - K_hi), device="cuda", generator=gen) * 4e-4 + 1e-4
    slots = _slots_across(n_slots, lo_slot)
    sd = dev(slots)
    B = len(slots)
    cfg = synth.shrink(cfg0, B=B)
    perm = synth.damp_key_perm(cfg)
    x = synth.step_inputs(cfg, 0)
    take = lambda t: t[sd.long()].cpu().numpy().copy()  # noqa: E731
    hi_s, lo_s, sc_s = take(hi_d).view(np.uint16), take(lo_d), take(sc_d)
    xd = dev_inputs(x, cfg.in_dtype)
    o = hla.damp_step(hi_d, lo_d, sc_d, dev(perm), K_hi, xd["q"], xd["k"], xd["v"],
                      xd["alpha"], 1, xd["beta"], slot=sd)
    x64 = f64_inputs(x, cfg.in_dtype)
    o_ref = oracle.damp_step(hi_s, lo_s, sc_s, perm, K_hi, x64["q"], x64["k"], x64["v"],
                             x64["alpha"], x64["beta"], per_channel=True)
    g = (take(hi_d).view(np.uint16), take(lo_d), take(sc_d))
    w = _state_bars(g, (hi_s, lo_s, sc_s), perm, K_hi, dk)
    w["out"] = rel_err_tiles(host(o), o_ref, 1)
    _assert_bars(w)


def test_restore_replay_beyond_4gib():
    """The fused restore + replay into a private state of 2 layers x 2,080 slots (8.7 GB):
    pairs land on both sides of the 4 GiB boundary of each layer, and the second layer
    starts past it."""
    import oracle_par

    hla = need_gpu()
    base = synth.CONFIGS["dasc_gdn"]
    H, dk, dv = base.H, base.dk, base.dv
    slot_bytes = H * dk * dv * 4
    n_slots = GIB4 // slot_bytes + 32
    cfg = synth.shrink(base, L=2, slots=3, seed=base.seed + 41)
    mask = synth.dasc_masks(cfg)
    _, _, unit_pos, R = hla.dasc_plan(mask)
    packed = synth.initial_state(synth.shrink(cfg, H=R), S=cfg.slots).reshape(cfg.slots, R, -1)
    dst = _slots_across(n_slots, slot_bytes)
    N = len(dst)
    src = (np.arange(N) % cfg.slots).astype(np.int32)
    xs = [synth.replay_inputs(cfg, l, B=N) for l in range(cfg.L)]
    x = {n: np.stack([xl[n] for xl in xs]) for n in NAMES}
    n_acc = xs[0]["n_accept"]
    st = torch.full((cfg.L, n_slots, H, dk, dv), 7.0, device="cuda")
    out = hla.dasc_restore_replay(dev(packed), dev(unit_pos.reshape(-1)), dev(src), dev(dst), st,
                                  *(dev(x[n]) for n in NAMES), dev(n_acc), 0,
                                  out=torch.full((cfg.L, N, cfg.K, H, dv), 5.0, device="cuda"))
    got = host(st[:, torch.from_numpy(dst).long().cuda()])
    o = host(out)
    x64 = {n: a.astype(np.float64) for n, a in x.items()}
    for l in range(cfg.L):
        S64 = np.zeros((N, H, dk, dv))
        for h in range(H):
            if unit_pos[l, h] >= 0:
                S64[:, h] = packed[src, unit_pos[l, h]].reshape(N, dk, dv)
        o_ref, scale = oracle_par.replay_terms(S64, {n: x64[n][l] for n in NAMES}, n_acc,
                                               per_channel=False)
        assert rel_err_tiles(got[l], S64) <= TOL
        rows = np.arange(cfg.K)[None, :] < n_acc[:, None]
        e = np.where(rows[:, :, None, None], np.abs(o[l] - o_ref), 0.0).max(axis=-1)
        assert float((e / np.maximum(scale, 1e-30)).max()) <= TOL
        assert (o[l][~rows] == 5.0).all()
    # slots no pair names keep their contents, on both sides of the boundary
    others = [s for s in range(int(dst[1]) - 2, int(dst[-1]) + 3)
              if s not in set(dst.tolist()) and 0 <= s < n_slots]
    assert (host(st[:, others]) == 7.0).all()

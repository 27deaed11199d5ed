"""GPU parity of the INT8-composed checkpoints (dasc_pack_int8 / dasc_restore_int8) and
of the dasc-wr copy-back (dasc_refresh_local) against the float64 oracle.

Bars: restore and copy-back bit-exact (q * s is one FP32 rounding on both sides; copies
are copies); pack: FP32 scales bit-exact (the same FP32 row maximum divided by 127),
codes differ by at most 1 on at most 0.1% of values (the quantiser's rounding decision
is taken on x * rcp(s) on the GPU and on fl(x / s) in the oracle)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, host, need_gpu, torch

pytestmark = pytest.mark.gpu
CODE_FRAC = 1e-3


def _stride(S_, n_units, unit_rows, dv):
    return S_ * n_units * unit_rows * dv * 4


@pytest.mark.parametrize("unit_rows,dv,n_units,p_keep", [
    (1, 128, 40, 0.3),      # KDA channel rows
    (1, 64, 33, 0.6),
    (128, 128, 5, 0.5),     # GDN heads
    (4, 64, 9, 0.7),
])
def test_pack_and_restore_int8(unit_rows, dv, n_units, p_keep):
    hla = need_gpu()
    g = np.random.default_rng(unit_rows * 100 + dv + n_units)
    L, S_ = 3, 5
    act = (g.standard_normal((L, S_, n_units, unit_rows, dv)) * 0.05).astype(np.float32)
    act[0, 1, 2, 0] = 0.0                      # a zero row
    act[2, 3, 1, 0, 7] = 25.0                  # an outlier
    mask = (g.random((L, n_units)) < p_keep).astype(np.uint8)
    mask[1] = 0                                # an empty layer
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    S_ckpt = S_ + 1
    src = g.permutation(S_)[:4].astype(np.int32)
    dst = g.permutation(S_ckpt)[:4].astype(np.int32)
    codes = torch.full((S_ckpt, R, unit_rows, dv), 99, dtype=torch.int8, device="cuda")
    scales = torch.full((S_ckpt, R, unit_rows), -1.0, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.dasc_pack_int8(dev(act), _stride(S_, n_units, unit_rows, dv), S_, L, n_units, unit_rows,
                       dv, dev(offsets), dev(unit_index), R, dev(src), dev(dst), codes, scales,
                       S_ckpt, err_flag=err)
    c_o, s_o = oracle.dasc_pack_int8(act, offsets, unit_index, src, dst, S_ckpt)
    c_g, s_g = host(codes), host(scales)
    for d_ in dst:
        assert np.array_equal(s_g[d_], s_o[d_])
        diff = np.abs(c_g[d_].astype(int) - c_o[d_].astype(int))
        assert diff.max(initial=0) <= 1 and (diff > 0).mean() <= CODE_FRAC
    others = [s for s in range(S_ckpt) if s not in dst]
    assert (c_g[others] == 99).all() and (s_g[others] == -1.0).all()
    # restore the oracle's checkpoint into sentinel-filled private slots: bit-exact
    S_dst = S_ + 2
    dst2 = g.permutation(S_dst)[:4].astype(np.int32)
    out0 = np.full((L, S_dst, n_units, unit_rows, dv), 3.5, np.float32)
    out = dev(out0)
    hla.dasc_restore_int8(dev(c_o), dev(s_o), S_ckpt, R, dev(unit_pos.reshape(-1)), L, n_units,
                          unit_rows, dv, dev(dst), dev(dst2), out,
                          _stride(S_dst, n_units, unit_rows, dv), S_dst, err_flag=err)
    ref = oracle.dasc_restore_int8(c_o, s_o, offsets, unit_index, L, n_units, dst, dst2,
                                   out0.copy())
    assert np.array_equal(host(out), ref)
    assert int(err.item()) == 0


@pytest.mark.parametrize("unit_rows,dv,n_units", [
    (1, 128, 384),   # channel rows, three heads per layer
    (2, 64, 192),    # units of 2-8 rows: restored by blocks of 128 rows
    (4, 128, 96),
    (8, 128, 48),
    (32, 64, 12),
    (128, 128, 3),   # whole heads
    (1, 64, 200),    # 200 rows per layer: not whole blocks of 128
])
def test_restore_int8_sparse_checkpoints(unit_rows, dv, n_units):
    """Sparse checkpoints (a quarter of the units retained) over unit sizes from single
    channels to whole heads (units of 2-8 rows take the restore by blocks of 128 rows,
    the rest the row kernel): bit-exact against the oracle's restore into sentinel-filled
    slots, with a plan entry past the packed rows (that unit zero, HLA_DEVERR_PLAN) and a
    pair whose destination is past S_dst (skipped, HLA_DEVERR_SLOT); the same restore with
    unit_pos and scales at 4-byte but not 16-byte alignment (the row kernel) gives the same
    bits; an empty checkpoint restores zeros."""
    hla = need_gpu()
    g = np.random.default_rng(7100 + unit_rows * 10 + dv)
    L, S_ = 3, 5
    act = (g.standard_normal((L, S_, n_units, unit_rows, dv)) * 0.05).astype(np.float32)
    mask = (g.random((L, n_units)) < 0.25).astype(np.uint8)
    mask[0, 0] = 1
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    assert 0 < 8 * R <= 3 * L * n_units
    S_ckpt, S_dst = S_, S_ + 2
    c_o, s_o = oracle.dasc_pack_int8(act, offsets, unit_index, np.arange(S_, dtype=np.int32),
                                     np.arange(S_, dtype=np.int32), S_ckpt)
    bad_pos = unit_pos.reshape(-1).copy()
    bad_pos[0] = R + 3                          # layer 0, unit 0: retained
    src = np.array([3, 0, 4, 1], np.int32)
    dst = np.array([6, 1, S_dst + 2, 0], np.int32)
    out0 = np.full((L, S_dst, n_units, unit_rows, dv), 3.5, np.float32)
    stride = _stride(S_dst, n_units, unit_rows, dv)
    ok = dst < S_dst
    ref = oracle.dasc_restore_int8(c_o, s_o, offsets, unit_index, L, n_units, src[ok], dst[ok],
                                   out0.copy())
    ref[0, dst[ok], 0] = 0.0                    # the unit with the bad position reads as zeros

    def restore(pos_t, scales_t):
        out = dev(out0)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        hla.dasc_restore_int8(dev(c_o), scales_t, S_ckpt, R, pos_t, L, n_units, unit_rows, dv,
                              dev(src), dev(dst), out, stride, S_dst, err_flag=err)
        assert int(err.item()) == hla.DEVERR_PLAN | hla.DEVERR_SLOT
        return host(out)

    def shifted(x):  # the same values, 4 bytes past a 16-byte boundary
        buf = torch.zeros(x.size + 4, dtype=torch.from_numpy(x[:0]).dtype, device="cuda")
        view = buf[1:1 + x.size]
        view.copy_(dev(x.reshape(-1)))
        assert view.data_ptr() % 16 == 4
        return view

    assert np.array_equal(restore(dev(bad_pos), dev(s_o)), ref)
    assert np.array_equal(restore(shifted(bad_pos), shifted(s_o)), ref)
    # an empty checkpoint: every unit omitted, every destination unit zero
    none = np.full(L * n_units, -1, np.int32)
    out = dev(out0)
    hla.dasc_restore_int8(torch.zeros(16, dtype=torch.int8, device="cuda"),
                          torch.zeros(4, device="cuda"), S_ckpt, 0, dev(none), L, n_units,
                          unit_rows, dv, dev(src[ok]), dev(dst[ok]), out, stride, S_dst)
    want = out0.copy()
    want[:, dst[ok]] = 0.0
    assert np.array_equal(host(out), want)


def _every_pair_against_oracle(hla, act_h, codes, scales, offsets, unit_index, unit_pos, R):
    """All 512 pairs of a full-size checkpoint workload: the GPU's pack against the oracle's
    (scales bit-exact, codes within one step on at most 0.1%), then the oracle's checkpoint
    restored on the GPU against the oracle's restore, every byte of the 4 GiB."""
    import oracle_par

    L, S_, nu, ur, dv = act_h.shape
    c_o, s_o = oracle_par.dasc_pack_int8_all(act_h, offsets, unit_index)
    assert np.array_equal(host(scales).reshape(s_o.shape), s_o)
    c_g = codes.cpu().numpy().reshape(c_o.shape)
    diff = np.abs(c_g.astype(np.int16) - c_o.astype(np.int16))
    assert diff.max() <= 1 and (diff > 0).mean() <= CODE_FRAC, (diff.max(), (diff > 0).mean())
    del c_g, diff
    ids = dev(np.arange(S_, dtype=np.int32))
    out = torch.full((L, S_, nu, ur, dv), float("nan"), device="cuda")
    hla.dasc_restore_int8(dev(c_o), dev(s_o), S_, R, dev(unit_pos.reshape(-1)), L, nu, ur, dv,
                          ids, ids, out, S_ * nu * ur * dv * 4, S_)
    ref = np.full(act_h.shape, np.nan, np.float32)
    oracle_par.dasc_restore_int8_all(c_o, s_o, offsets, unit_index, L, nu, ref)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_kda_checkpoint_workload_static_horizon_selection():
    """4 layers x 512 request states x 32 heads x 128 key channels, one unit per channel
    row (512 B), selected by static horizons (softplus gate, a_s = -0.3, W_max = 16) from
    the synthetic gate parameters: INT8 pack of all 512 states, restore into 512 private
    slots.  Over the whole 4 GiB state: every retained value within half a quantisation
    step of the original (plus the rounding slack of the GPU quantiser), every omitted
    value zero; every pair against the oracle (pack at the quantiser bars, restore of the
    oracle's checkpoint bit for bit)."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_kda"]
    A, d = synth.gate_params(cfg)
    _, mask3 = hla.dasc_static_horizon(A, d, hla.GATE_SOFTPLUS, cfg.a_s, cfg.W_max)
    mask = mask3.reshape(cfg.L, cfg.H * cfg.dk)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    L, S_, nu, dv = cfg.L, cfg.slots, cfg.H * cfg.dk, cfg.dv
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    act = torch.randn((L, S_, nu, dv), device="cuda", generator=gen) * 0.05
    codes = torch.empty((S_, R, 1, dv), dtype=torch.int8, device="cuda")
    scales = torch.empty((S_, R, 1), device="cuda")
    ids = dev(np.arange(S_, dtype=np.int32))
    stride = S_ * nu * dv * 4
    hla.dasc_pack_int8(act, stride, S_, L, nu, 1, dv, dev(offsets), dev(unit_index), R, ids, ids,
                       codes, scales, S_)
    out = torch.full_like(act, float("nan"))
    hla.dasc_restore_int8(codes, scales, S_, R, dev(unit_pos.reshape(-1)), L, nu, 1, dv, ids,
                          ids, out, stride, S_)
    keep = torch.from_numpy(mask.astype(bool)).cuda()[:, None, :, None]
    step = act.abs().amax(-1, keepdim=True) / 127
    # half a step, widened by the rounding decision taken on x * rcp(s) (it can fall on
    # the other side of a half-integer within ~2e-5 of it) and the FP32 rounding of q * s
    bound = (0.5 + 5e-5) * step + act.abs() * 2.0 ** -23
    assert bool(((out - act).abs() <= bound)[keep.expand_as(act)].all())
    assert bool((out[~keep.expand_as(act)] == 0).all())
    _every_pair_against_oracle(hla, act.cpu().numpy().reshape(L, S_, nu, 1, dv), codes, scales,
                               offsets, unit_index, unit_pos, R)


def test_refresh_local_bit_exact():
    hla = need_gpu()
    g = np.random.default_rng(41)
    L, S_s, S_a, n_units, ub = 3, 4, 6, 37, 512
    scratch = g.integers(0, 256, size=(L, S_s, n_units, ub), dtype=np.uint8)
    active = g.integers(0, 256, size=(L, S_a, n_units, ub), dtype=np.uint8)
    mask = (g.random((L, n_units)) < 0.4).astype(np.uint8)   # 1 = global
    local = 1 - mask
    offsets, unit_index, _, R_local = hla.dasc_plan(local)
    src = np.array([2, 0, 3], np.int32)
    dst = np.array([5, 1, 2], np.int32)
    act_d = dev(active.reshape(-1))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    hla.dasc_refresh_local(dev(scratch.reshape(-1)), S_s * n_units * ub, S_s, act_d,
                           S_a * n_units * ub, S_a, L, n_units, ub, dev(offsets),
                           dev(unit_index), R_local, dev(src), dev(dst), err_flag=err)
    ref = oracle.dasc_refresh_local(scratch, active.copy(), local, src, dst)
    assert np.array_equal(host(act_d).reshape(active.shape), ref)
    assert int(err.item()) == 0


@pytest.mark.parametrize("kind", ["gdn", "kda"])
def test_dasc_wr_flow(kind):
    """The whole dasc-wr load path on the GPU: restore the checkpoint with zero-filled
    local units, replay the refresh window from a zero scratch state with the ordinary
    step, copy the refreshed local units back.  Global units end exactly at their
    checkpoint values, local units exactly at the scratch replay's values."""
    hla = need_gpu()
    base = synth.CONFIGS["dasc_kda" if kind == "kda" else "dasc_gdn"]
    cfg = synth.shrink(base, B=3, H=4, dk=64, dv=64, slots=3, L=2)
    L, S_, H, dk, dv = cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv
    g = np.random.default_rng(7)
    if kind == "kda":
        A, d = synth.gate_params(cfg)
        Hs, m = hla.dasc_static_horizon(A, d, hla.GATE_SOFTPLUS, cfg.a_s, cfg.W_max)
        mask, unit_rows, n_units = m.reshape(L, H * dk), 1, H * dk
    else:
        Hs = g.uniform(2, 64, (L, H))
        mask, unit_rows, n_units = (Hs > 16).astype(np.uint8), dk, H
    ub = unit_rows * dv * 4
    W, _ = hla.dasc_replay_window(Hs.reshape(-1), mask.reshape(-1), 48, 16)
    assert 4 <= W <= 16
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    lo_off, lo_idx, _, R_loc = hla.dasc_plan(1 - mask)
    ckpt_state = (g.standard_normal((L, S_, H, dk, dv)) * 0.05).astype(np.float32)
    ids = dev(np.arange(S_, dtype=np.int32))
    stride = S_ * H * dk * dv * 4
    packed = torch.empty((S_, R, ub // 4), device="cuda")
    hla.dasc_pack(dev(ckpt_state), stride, S_, L, n_units, ub, dev(offsets), dev(unit_index), R,
                  ids, ids, packed, S_)
    active = torch.full((L, S_, H, dk, dv), float("nan"), device="cuda")
    hla.dasc_restore(packed, S_, R, dev(unit_pos.reshape(-1)), L, n_units, ub, ids, ids, active,
                     stride, S_)
    scratch = torch.zeros_like(active)
    step = hla.kda_step if kind == "kda" else hla.gdn_step
    rep = synth.shrink(cfg, B=S_)
    for t in range(W):
        for l in range(L):
            x = synth.step_inputs(rep, 100 * l + t)
            xd = {n: dev(a) for n, a in x.items()}
            step(scratch[l], xd["q"], xd["k"], xd["v"], xd["alpha"], xd["beta"], want_out=False)
    hla.dasc_refresh_local(scratch, stride, S_, active, stride, S_, L, n_units, ub,
                           dev(lo_off), dev(lo_idx), R_loc, ids, ids)
    glob = torch.from_numpy(mask.astype(bool)).cuda()
    shape = (L, S_, n_units, unit_rows * dv)
    a2, c2, s2 = (active.reshape(shape), dev(ckpt_state).reshape(shape), scratch.reshape(shape))
    gm = glob[:, None, :, None].expand(shape)
    assert torch.equal(a2[gm], c2[gm])
    assert torch.equal(a2[~gm], s2[~gm])


def test_gdn_checkpoint_workload_head_units():
    """4 layers x 512 request states x 32 heads of 128 x 128 FP32 (4 GiB), the seeded
    ragged head selection (64 of 128 heads): INT8 pack of all 512 states, restore into
    512 private slots.  Every retained value within half a quantisation step (plus the
    GPU quantiser's rounding slack), every omitted head zero; every pair against the
    oracle (pack at the quantiser bars, restore of the oracle's checkpoint bit for bit)."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_gdn"]
    mask = synth.dasc_masks(cfg)
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    L, S_, nu, ur, dv = cfg.L, cfg.slots, cfg.H, cfg.dk, cfg.dv
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed)
    act = torch.randn((L, S_, nu, ur, dv), device="cuda", generator=gen) * 0.05
    codes = torch.empty((S_, R, ur, dv), dtype=torch.int8, device="cuda")
    scales = torch.empty((S_, R, ur), device="cuda")
    ids = dev(np.arange(S_, dtype=np.int32))
    stride = S_ * nu * ur * dv * 4
    hla.dasc_pack_int8(act, stride, S_, L, nu, ur, dv, dev(offsets), dev(unit_index), R, ids, ids,
                       codes, scales, S_)
    out = torch.full_like(act, float("nan"))
    hla.dasc_restore_int8(codes, scales, S_, R, dev(unit_pos.reshape(-1)), L, nu, ur, dv, ids,
                          ids, out, stride, S_)
    keep = torch.from_numpy(mask.astype(bool)).cuda()[:, None, :, None, None].expand_as(act)
    step = act.abs().amax(-1, keepdim=True) / 127
    bound = (0.5 + 5e-5) * step + act.abs() * 2.0 ** -23
    assert bool(((out - act).abs() <= bound)[keep].all())
    assert bool((out[~keep] == 0).all())
    _every_pair_against_oracle(hla, act.cpu().numpy(), codes, scales, offsets, unit_index,
                               unit_pos, R)


def test_kda_refresh_local_workload():
    """The dasc-wr copy-back at the KDA checkpoint workload (512 states, 12,260 local
    channel rows of 16,384 over 4 layers): local rows take the scratch values, global
    rows keep theirs, bit for bit, over the whole 4 GiB."""
    hla = need_gpu()
    cfg = synth.CONFIGS["dasc_kda"]
    A, d = synth.gate_params(cfg)
    _, m3 = hla.dasc_static_horizon(A, d, hla.GATE_SOFTPLUS, cfg.a_s, cfg.W_max)
    mask = m3.reshape(cfg.L, cfg.H * cfg.dk)
    lo_off, lo_idx, _, R_loc = hla.dasc_plan(1 - mask)
    L, S_, nu, dv = cfg.L, cfg.slots, cfg.H * cfg.dk, cfg.dv
    gen = torch.Generator(device="cuda").manual_seed(cfg.seed + 1)
    scratch = torch.randn((L, S_, nu, dv), device="cuda", generator=gen)
    active = torch.randn((L, S_, nu, dv), device="cuda", generator=gen)
    before = active.clone()
    ids = dev(np.arange(S_, dtype=np.int32))
    stride = S_ * nu * dv * 4
    hla.dasc_refresh_local(scratch, stride, S_, active, stride, S_, L, nu, dv * 4, dev(lo_off),
                           dev(lo_idx), R_loc, ids, ids)
    loc = torch.from_numpy((1 - mask).astype(bool)).cuda()[:, None, :, None].expand_as(active)
    assert torch.equal(active[loc], scratch[loc])
    assert torch.equal(active[~loc], before[~loc])


@pytest.mark.parametrize("unit_rows", [1, 128])
def test_int8_device_errors(unit_rows):
    """Bad device-side indices in the INT8 checkpoint kernels: a source or destination
    slot past its bound sets HLA_DEVERR_SLOT and skips that pair only; a unit_index entry
    past the units sets HLA_DEVERR_PLAN; a unit_pos entry past the packed rows sets
    HLA_DEVERR_PLAN and that unit is restored as zeros, every other unit as the oracle's
    restore (channel rows and head units take different kernel paths)."""
    hla = need_gpu()
    g = np.random.default_rng(4400 + unit_rows)
    L, S_, n_units, dv = 2, 3, 6, 128
    act = (g.standard_normal((L, S_, n_units, unit_rows, dv)) * 0.05).astype(np.float32)
    mask = np.ones((L, n_units), np.uint8)
    mask[0, 2] = 0
    offsets, unit_index, unit_pos, R = hla.dasc_plan(mask)
    stride = _stride(S_, n_units, unit_rows, dv)
    codes = torch.zeros((S_, R, unit_rows, dv), dtype=torch.int8, device="cuda")
    scales = torch.zeros((S_, R, unit_rows), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    # pack: pair 1 names a source slot past S_act; pair 0 is packed as the oracle packs it
    hla.dasc_pack_int8(dev(act), stride, S_, L, n_units, unit_rows, dv, dev(offsets),
                       dev(unit_index), R, dev(np.array([1, 9], np.int32)),
                       dev(np.array([0, 2], np.int32)), codes, scales, S_, err_flag=err)
    assert int(err.item()) == hla.DEVERR_SLOT
    c_o, s_o = oracle.dasc_pack_int8(act, offsets, unit_index, np.array([1], np.int32),
                                     np.array([0], np.int32), S_)
    assert np.array_equal(host(scales)[0], s_o[0])
    assert (host(codes)[2] == 0).all() and (host(scales)[2] == 0).all()
    err.zero_()
    bad_index = unit_index.copy()
    bad_index[1] = n_units + 3
    hla.dasc_pack_int8(dev(act), stride, S_, L, n_units, unit_rows, dv, dev(offsets),
                       dev(bad_index), R, dev(np.array([0], np.int32)),
                       dev(np.array([1], np.int32)), codes, scales, S_, err_flag=err)
    assert int(err.item()) == hla.DEVERR_PLAN
    # that packed position is left as it was (zeros here); the others hold the pack
    c1, s1 = oracle.dasc_pack_int8(act, offsets, unit_index, np.array([0], np.int32),
                                   np.array([1], np.int32), S_)
    s1[1, 1] = 0.0
    c1[1, 1] = 0
    assert np.array_equal(host(scales)[1], s1[1])
    assert (host(codes)[1, 1] == 0).all()
    # restore of the oracle's checkpoint with one unit_pos entry past R_total, and a second
    # pair whose destination slot is past S_dst
    c_o, s_o = oracle.dasc_pack_int8(act, offsets, unit_index, np.array([1], np.int32),
                                     np.array([0], np.int32), S_)
    bad_pos = unit_pos.reshape(-1).copy()
    bad_u = n_units + 4                        # layer 1, unit 4: retained
    assert bad_pos[bad_u] >= 0
    bad_pos[bad_u] = R + 7
    out0 = np.full((L, S_, n_units, unit_rows, dv), 3.5, np.float32)
    out = dev(out0)
    err.zero_()
    hla.dasc_restore_int8(dev(c_o), dev(s_o), S_, R, dev(bad_pos), L, n_units, unit_rows, dv,
                          dev(np.array([0, 0], np.int32)), dev(np.array([2, 5], np.int32)), out,
                          stride, S_, err_flag=err)
    assert int(err.item()) == hla.DEVERR_PLAN | hla.DEVERR_SLOT
    ref = oracle.dasc_restore_int8(c_o, s_o, offsets, unit_index, L, n_units,
                                   np.array([0], np.int32), np.array([2], np.int32), out0.copy())
    ref[1, 2, 4] = 0.0                          # the unit with the bad position reads as zeros
    assert np.array_equal(host(out), ref)

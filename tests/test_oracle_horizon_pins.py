"""Pins for the oracle's static retention horizons, selection masks and dasc-wr refresh
window (dasc paper §3.3 Eq. (2)-(3), §4.1, §4.2 Eq. (7)) and its INT8-composed
checkpoints (App. E.1 Eq. (8), App. E.2).

The horizon is pinned by closed forms at the gates' zero crossing (softplus(0) = ln 2,
sigmoid(0) = 1/2), by numpy's log-add-exp and scipy's logistic function on random parameters, by the
bounded gate's floor and by monotonicity; the window by hand-worked cases of Eq. (7);
the INT8 checkpoint by its composition from two separately pinned oracle pieces (the row
quantiser and the byte pack) and by the quantiser's error bound after a round trip."""
import math

import numpy as np
import pytest

rng = np.random.default_rng


def test_horizon_closed_forms_at_zero_gate_input(orc):
    # a_s + d = 0, A_log = 0: softplus gate g = -ln 2, bounded gate g = -5/2
    A = np.zeros(3)
    d = np.full(3, 0.3)
    H0 = orc.static_horizon(A, d, orc.GATE_SOFTPLUS, -0.3)
    H1 = orc.static_horizon(A, d, orc.GATE_BOUNDED, -0.3)
    np.testing.assert_allclose(H0, math.log(1e3) / math.log(2.0), rtol=1e-15)  # log2(1000)
    np.testing.assert_allclose(H1, math.log(1e3) / 2.5, rtol=1e-15)
    # eps enters only through ln(eps)
    H2 = orc.static_horizon(A, d, orc.GATE_SOFTPLUS, -0.3, eps=1e-6)
    np.testing.assert_allclose(H2, 2 * H0, rtol=1e-15)


def test_horizon_matches_numpy_on_random_parameters(orc):
    g = rng(70)
    A = g.normal(0, 1.0, 2000)
    d = g.normal(0, 1.5, 2000)
    a_s = -0.3
    g0 = -np.exp(A) * np.logaddexp(0.0, a_s + d)
    np.testing.assert_allclose(orc.static_horizon(A, d, orc.GATE_SOFTPLUS, a_s),
                               np.log(1e-3) / g0, rtol=1e-13)
    from scipy.special import expit  # an independent logistic sigmoid

    g1 = -5.0 * expit(np.exp(A) * (0.8 + d))
    np.testing.assert_allclose(orc.static_horizon(A, d, orc.GATE_BOUNDED, 0.8),
                               np.log(1e-3) / g1, rtol=1e-12)


def test_horizon_monotone_and_bounded_gate_floor(orc):
    g = rng(71)
    A = g.normal(0, 1, 500)
    d = np.sort(g.normal(0, 2, 500))
    # larger bias -> faster decay -> shorter horizon (softplus gate, fixed A_log)
    H = orc.static_horizon(np.zeros(500), d, orc.GATE_SOFTPLUS, -0.3)
    assert (np.diff(H) <= 0).all()
    # larger log-scale -> shorter horizon
    Hs = orc.static_horizon(np.sort(A), np.zeros(500), orc.GATE_SOFTPLUS, -0.3)
    assert (np.diff(Hs) <= 0).all()
    # the bounded gate never decays faster than l = -5 per step (it reaches -5 only
    # where the sigmoid saturates to 1 in float64)
    Hb = orc.static_horizon(A, g.normal(0, 5, 500), orc.GATE_BOUNDED, 0.8)
    assert (Hb >= math.log(1e3) / 5.0).all()
    assert (orc.static_horizon(np.zeros(50), np.linspace(-3, 3, 50), orc.GATE_BOUNDED, 0.0)
            > math.log(1e3) / 5.0).all()


def test_mask_is_strict_cutoff(orc):
    H = np.array([0.5, 15.999, 16.0, 16.001, 1e6])
    assert orc.static_mask(H, 16).tolist() == [0, 0, 0, 1, 1]


@pytest.mark.parametrize("H,mask,n_p,W_max,expect_W,expect_u", [
    # next_pow2 rounds up to a power of two, clamped to [4, W_max]
    ([3.0, 4.0, 4.5, 9.0, 0.5], [0, 0, 0, 0, 0], 100, 16, 16, [4, 4, 8, 16, 4]),
    # the window is the largest local unit's; global units do not count
    ([3.0, 9.0, 40.0], [0, 0, 1], 100, 16, 16, [4, 16, 16]),
    ([3.0, 5.0, 40.0], [0, 0, 1], 100, 16, 8, [4, 8, 16]),
    # capped by the cached prefix
    ([3.0, 9.0, 40.0], [0, 0, 1], 7, 16, 7, [4, 16, 16]),
    # nothing omitted: no refresh
    ([30.0, 40.0], [1, 1], 100, 16, 0, [16, 16]),
    # H = 0 maps to 4
    ([0.0], [0], 100, 64, 4, [4]),
    # exact powers of two stay
    ([32.0, 64.0], [0, 0], 1000, 64, 64, [32, 64]),
])
def test_replay_window_cases(orc, H, mask, n_p, W_max, expect_W, expect_u):
    W, W_u = orc.replay_window(np.array(H), np.array(mask, np.uint8), n_p, W_max)
    assert W == expect_W and W_u.tolist() == expect_u


def _kda_units(g, L, S_, n_units, unit_rows, dv):
    return (g.standard_normal((L, S_, n_units, unit_rows, dv)) * 0.05).astype(np.float32)


@pytest.mark.parametrize("unit_rows,dv", [(1, 32), (4, 16)])
def test_int8_pack_is_row_quantise_then_byte_pack(orc, unit_rows, dv):
    """Quantise-once-at-store: the INT8 checkpoint of the retained units equals the row
    quantiser applied to every row of the active state, moved by the byte pack."""
    g = rng(72 + unit_rows)
    L, S_, n_units = 3, 4, 6
    act = _kda_units(g, L, S_, n_units, unit_rows, dv)
    act[1, 2, 3, 0] = 0.0  # a zero row takes the scale floor
    mask = (g.random((L, n_units)) < 0.5).astype(np.uint8)
    offsets, unit_index = orc.dasc_plan(mask)
    src = np.array([2, 0, 3], np.int32)
    dst = np.array([1, 4, 0], np.int32)
    codes, scales = orc.dasc_pack_int8(act, offsets, unit_index, src, dst, 5)
    # reference: quantise every row, then move bytes with the byte pack
    qc = np.zeros(act.shape, np.int8)
    qs = np.zeros(act.shape[:-1], np.float32)
    for idx in np.ndindex(*act.shape[:-1]):
        qc[idx], qs[idx] = orc.quantize_row_int8(act[idx].astype(np.float64))
    ref_c = orc.dasc_pack(qc.view(np.uint8).reshape(L, S_, n_units, -1), offsets, unit_index,
                          src, dst, 5)
    ref_s = orc.dasc_pack(qs.view(np.uint8).reshape(L, S_, n_units, -1), offsets, unit_index,
                          src, dst, 5)
    R = int(offsets[-1])
    assert np.array_equal(codes.view(np.uint8).reshape(5, R, -1), ref_c)
    assert np.array_equal(scales.view(np.uint8).reshape(5, R, -1), ref_s)


def test_int8_restore_round_trip_bound_and_zero_fill(orc):
    g = rng(74)
    L, S_, n_units, unit_rows, dv = 2, 3, 8, 2, 64
    act = _kda_units(g, L, S_, n_units, unit_rows, dv)
    mask = (g.random((L, n_units)) < 0.6).astype(np.uint8)
    mask[0, 0], mask[1, 5] = 1, 0
    offsets, unit_index = orc.dasc_plan(mask)
    ids = np.arange(S_, dtype=np.int32)
    codes, scales = orc.dasc_pack_int8(act, offsets, unit_index, ids, ids, S_)
    out = np.full(act.shape, 7.0, np.float32)
    orc.dasc_restore_int8(codes, scales, offsets, unit_index, L, n_units, ids, ids, out)
    for l in range(L):
        for u in range(n_units):
            if not mask[l, u]:
                assert (out[l, :, u] == 0).all()
                continue
            x = act[l, :, u].astype(np.float64)
            s = np.abs(act[l, :, u]).max(-1, keepdims=True) / np.float32(127)
            assert (np.abs(out[l, :, u] - x) <= 0.5 * s * (1 + 1e-6) + 1e-12).all()
    # the dequantised value is the FP32 product of code and scale
    p = int(offsets[0 + 1]) - 1 if offsets[1] > 0 else None
    if p is not None:
        u = unit_index[p]
        np.testing.assert_array_equal(out[0, 1, u], (codes[1, p].astype(np.float32) *
                                                     scales[1, p][:, None]))


def test_int8_checkpoint_bytes_closed_form(orc):
    """Payload of an INT8 checkpoint row: dv codes + one FP32 scale, vs 4 dv bytes in FP32:
    a ratio of 4 dv / (dv + 4) (3.879 at dv = 128), before the ragged gain."""
    L, S_, n_units, unit_rows, dv = 2, 2, 4, 1, 128
    act = np.ones((L, S_, n_units, unit_rows, dv), np.float32)
    mask = np.ones((L, n_units), np.uint8)
    offsets, unit_index = orc.dasc_plan(mask)
    codes, scales = orc.dasc_pack_int8(act, offsets, unit_index, np.arange(2), np.arange(2), 2)
    ratio = act.nbytes / (codes.nbytes + scales.nbytes)
    assert ratio == 4 * dv / (dv + 4)
    assert round(ratio, 2) == 3.88


def test_refresh_local_copies_local_units_only(orc):
    """dasc-wr copy-back: local units take the scratch values, global units keep theirs,
    and an all-global mask copies nothing."""
    g = rng(75)
    L, S_, n_units, ub = 3, 4, 6, 32
    scratch = g.integers(0, 256, size=(L, S_, n_units, ub), dtype=np.uint8)
    active = g.integers(0, 256, size=(L, S_ + 1, n_units, ub), dtype=np.uint8)
    mask = (g.random((L, n_units)) < 0.5).astype(np.uint8)  # 1 = global (retained)
    local = 1 - mask
    src = np.array([3, 1], np.int32)
    dst = np.array([0, 4], np.int32)
    out = orc.dasc_refresh_local(scratch, active.copy(), local, src, dst)
    for n in range(2):
        for l in range(L):
            for u in range(n_units):
                want = scratch[l, src[n], u] if local[l, u] else active[l, dst[n], u]
                assert np.array_equal(out[l, dst[n], u], want)
    untouched = [s for s in range(S_ + 1) if s not in dst]
    assert np.array_equal(out[:, untouched], active[:, untouched])
    out2 = orc.dasc_refresh_local(scratch, active.copy(), np.zeros_like(local), src, dst)
    assert np.array_equal(out2, active)


def test_refresh_local_all_local_is_a_slot_copy(orc):
    """With every unit local the copy-back is a whole-slot copy from scratch into the
    active slot (numpy slice assignment), per layer; other slots untouched."""
    g = rng(76)
    L, S_, n_units, ub = 2, 3, 5, 48
    scratch = g.integers(0, 256, size=(L, S_, n_units, ub), dtype=np.uint8)
    active = g.integers(0, 256, size=(L, S_ + 2, n_units, ub), dtype=np.uint8)
    local = np.ones((L, n_units), np.uint8)
    src = np.array([2, 0], np.int32)
    dst = np.array([4, 1], np.int32)
    want = active.copy()
    want[:, dst] = scratch[:, src]
    assert np.array_equal(orc.dasc_refresh_local(scratch, active.copy(), local, src, dst), want)

"""Pins for the oracle's GDN / KDA step and replay, independent of the oracle itself.

Each test checks the oracle against something the pages or the mathematics fix:
closed forms, exact rational brute force of the literal matrix form, the other
page's orientation of the same equation, and structural invariants.  Sources:
DAMP paper section 3.1 Eq. (1)-(4), dasc paper section 3.1 Eq. (1), and the
"Serving recurrent attention" explainer (replay of accepted draft projections).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth

rng = np.random.default_rng


def _unit(g, *shape):
    x = g.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_step(g, B, H, dk, dv, per_channel):
    q, k = _unit(g, B, H, dk), _unit(g, B, H, dk)
    v = g.standard_normal((B, H, dv))
    alpha = g.uniform(0.8, 0.999, (B, H, dk) if per_channel else (B, H))
    beta = 1 / (1 + np.exp(-g.standard_normal((B, H))))
    return q, k, v, alpha, beta


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("per_channel", [False, True])
def test_first_step_from_zero_state_closed_form(orc, per_channel):
    """From S_0 = 0: S_1 = beta k v^T and o_1 = beta (q.k) v (DAMP Eq. (1)-(2))."""
    g = rng(1)
    B, H, dk, dv = 2, 3, 64, 64
    q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, per_channel)
    S = np.zeros((B, H, dk, dv))
    o = orc.delta_step(S, q, k, v, alpha, beta, per_channel=per_channel)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(S[b, h], beta[b, h] * np.outer(k[b, h], v[b, h]),
                                       rtol=0, atol=1e-15)
            np.testing.assert_allclose(o[b, h], beta[b, h] * (q[b, h] @ k[b, h]) * v[b, h],
                                       rtol=0, atol=1e-14)


def test_toy_config_first_step_closed_form(orc):
    """The toy workload's first step (zero state, fp32 inputs) matches the closed form."""
    cfg = synth.CONFIGS["gdn_toy"]
    x = synth.step_inputs(cfg, 0)
    S = synth.initial_state(cfg).astype(np.float64)
    assert not S.any()
    q, k, v = (synth.stored_to_f64(x[n], cfg.in_dtype) for n in "qkv")
    a, bt = x["alpha"].astype(np.float64), x["beta"].astype(np.float64)
    o = orc.gdn_step(S, q, k, v, a, bt)
    expect = bt[..., None, None] * k[..., :, None] * v[..., None, :]
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o, (bt * np.sum(q * k, -1))[..., None] * v, rtol=0, atol=1e-14)


@pytest.mark.parametrize("per_channel", [False, True])
def test_beta_zero_is_pure_decay(orc, per_channel):
    """beta = 0 removes the delta rule: S_T = (prod_t Lambda_t) S_0."""
    g = rng(2)
    B, H, dk, dv, T = 2, 2, 64, 64, 7
    S0 = g.standard_normal((B, H, dk, dv))
    S = S0.copy()
    prod = np.ones((B, H, dk))
    for _ in range(T):
        q, k, v, alpha, _ = _rand_step(g, B, H, dk, dv, per_channel)
        orc.delta_step(S, q, k, v, alpha, np.zeros((B, H)), per_channel=per_channel)
        prod = prod * (alpha if per_channel else alpha[..., None])
    np.testing.assert_allclose(S, prod[..., None] * S0, rtol=1e-14, atol=0)


def test_unit_key_full_strength_overwrites(orc):
    """||k|| = 1, beta = 1, no decay: the state now maps k to v exactly, S_t^T k = v."""
    g = rng(3)
    B, H, dk, dv = 2, 2, 128, 128
    S = g.standard_normal((B, H, dk, dv))
    q, k, v, _, _ = _rand_step(g, B, H, dk, dv, False)
    orc.gdn_step(S, q, k, v, np.ones((B, H)), np.ones((B, H)))
    got = np.einsum("bhij,bhi->bhj", S, k)
    np.testing.assert_allclose(got, v, rtol=0, atol=1e-13)


@pytest.mark.parametrize("per_channel", [False, True])
def test_directions_orthogonal_to_key_untouched(orc, per_channel):
    """For w orthogonal to k, S_t^T w = (Lambda S_{t-1})^T w: the correction acts along k only."""
    g = rng(4)
    B, H, dk, dv = 1, 2, 64, 64
    S = g.standard_normal((B, H, dk, dv))
    q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, per_channel)
    lam = alpha if per_channel else np.broadcast_to(alpha[..., None], (B, H, dk))
    Sdec = lam[..., None] * S
    orc.delta_step(S, q, k, v, alpha, beta, per_channel=per_channel)
    for h in range(H):
        w = g.standard_normal(dk)
        w -= (w @ k[0, h]) * k[0, h]
        np.testing.assert_allclose(S[0, h].T @ w, Sdec[0, h].T @ w, rtol=0, atol=1e-12)


@pytest.mark.parametrize("per_channel", [False, True])
def test_increment_is_rank_one(orc, per_channel):
    g = rng(5)
    B, H, dk, dv = 1, 3, 64, 128
    S = g.standard_normal((B, H, dk, dv))
    q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, per_channel)
    lam = alpha if per_channel else np.broadcast_to(alpha[..., None], (B, H, dk))
    Sdec = lam[..., None] * S
    orc.delta_step(S, q, k, v, alpha, beta, per_channel=per_channel)
    for h in range(H):
        sv = np.linalg.svd(S[0, h] - Sdec[0, h], compute_uv=False)
        assert sv[1] <= 1e-12 * sv[0]


def test_kda_constant_vector_equals_gdn(orc):
    g = rng(6)
    B, H, dk, dv = 2, 2, 64, 64
    S1 = g.standard_normal((B, H, dk, dv))
    S2 = S1.copy()
    q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, False)
    o1 = orc.gdn_step(S1, q, k, v, alpha, beta)
    o2 = orc.kda_step(S2, q, k, v, np.repeat(alpha[..., None], dk, -1), beta)
    assert np.array_equal(S1, S2) and np.array_equal(o1, o2)


# ---------------------------------------------------------------- brute force

def _frac_matrix_step(S, q, k, v, a, beta):
    """Literal DAMP Eq. (3)-(4) in exact rationals: A = (I - beta k k^T) diag(a);
    S_t = A S_{t-1} + beta k v^T; o = S_t^T q."""
    dk, dv = len(S), len(S[0])
    A = [[((1 if i == m else 0) - beta * k[i] * k[m]) * a[m] for m in range(dk)]
         for i in range(dk)]
    Sn = [[sum((A[i][m] * S[m][j] for m in range(dk)), Fraction(0)) + beta * k[i] * v[j]
           for j in range(dv)] for i in range(dk)]
    o = [sum((Sn[i][j] * q[i] for i in range(dk)), Fraction(0)) for j in range(dv)]
    return Sn, o


def _dyadic(g, shape, scale=64):
    """Random values that are exact in float64 (small dyadic rationals)."""
    return g.integers(-scale, scale + 1, size=shape) / scale


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("dk,dv", [(2, 3), (4, 4), (3, 2)])
def test_exact_rational_brute_force(orc, per_channel, dk, dv):
    """Oracle vs exact rational arithmetic of the transition-matrix form over 5 steps."""
    g = rng(7 + dk * 10 + dv)
    H, T = 2, 5
    S = _dyadic(g, (1, H, dk, dv))
    Sf = [[[Fraction(x) for x in row] for row in S[0, h]] for h in range(H)]
    for _ in range(T):
        q, k, v = _dyadic(g, (1, H, dk)), _dyadic(g, (1, H, dk)), _dyadic(g, (1, H, dv))
        alpha = (g.integers(32, 65, size=(1, H, dk) if per_channel else (1, H)) / 64)
        beta = g.integers(1, 65, size=(1, H)) / 64
        o = orc.delta_step(S, q, k, v, alpha, beta, per_channel=per_channel)
        for h in range(H):
            a = [Fraction(x) for x in (alpha[0, h] if per_channel else [alpha[0, h]] * dk)]
            Sf[h], of = _frac_matrix_step(Sf[h], [Fraction(x) for x in q[0, h]],
                                          [Fraction(x) for x in k[0, h]],
                                          [Fraction(x) for x in v[0, h]], a,
                                          Fraction(beta[0, h]))
            exact = np.array([[float(x) for x in row] for row in Sf[h]])
            scale = max(1.0, np.abs(exact).max())
            assert np.abs(S[0, h] - exact).max() <= 1e-14 * scale
            assert np.abs(o[0, h] - np.array([float(x) for x in of])).max() <= 1e-14 * scale


@pytest.mark.parametrize("per_channel", [False, True])
def test_dasc_orientation_is_the_transpose(orc, per_channel):
    """dasc Eq. (1) keeps the state as dv x dk: S_t = S_{t-1} Diag(a)(I - beta k k^T) + beta v k^T,
    read by o = S_t q.  Run it in float64 with numpy on 8 x 8 and on serving-size heads and
    compare with the oracle's dk x dv state transposed."""
    g = rng(8)
    for dk, dv in ((8, 8), (5, 7), (128, 128)):
        B, H = 1, 2
        S = g.standard_normal((B, H, dk, dv))
        P = np.transpose(S, (0, 1, 3, 2)).copy()  # dv x dk
        for _ in range(4):
            q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, per_channel)
            o = orc.delta_step(S, q, k, v, alpha, beta, per_channel=per_channel)
            for h in range(H):
                a = alpha[0, h] if per_channel else np.full(dk, alpha[0, h])
                kk = k[0, h]
                P[0, h] = P[0, h] @ np.diag(a) @ (np.eye(dk) - beta[0, h] * np.outer(kk, kk)) \
                    + beta[0, h] * np.outer(v[0, h], kk)
                np.testing.assert_allclose(o[0, h], P[0, h] @ q[0, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(S, np.transpose(P, (0, 1, 3, 2)), rtol=0, atol=1e-12)


def test_error_propagation_is_homogeneous_and_contractive(orc):
    """Two trajectories with the same inputs: DeltaS_t = A_t DeltaS_{t-1} (DAMP Eq. (12) with
    R = 0), and with ||k|| <= 1, a <= 1 the transition never grows the difference."""
    g = rng(9)
    B, H, dk, dv = 1, 2, 32, 32
    S1 = g.standard_normal((B, H, dk, dv))
    S2 = S1 + 1e-3 * g.standard_normal(S1.shape)
    for _ in range(6):
        q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, True)
        d_prev = S2 - S1
        orc.kda_step(S1, q, k, v, alpha, beta)
        orc.kda_step(S2, q, k, v, alpha, beta)
        for h in range(H):
            A = (np.eye(dk) - beta[0, h] * np.outer(k[0, h], k[0, h])) @ np.diag(alpha[0, h])
            np.testing.assert_allclose(S2[0, h] - S1[0, h], A @ d_prev[0, h], rtol=0, atol=1e-13)
            assert np.linalg.norm(S2[0, h] - S1[0, h]) <= np.linalg.norm(d_prev[0, h]) * (1 + 1e-12)


def test_slot_mapping_and_padding(orc):
    """Request b updates state slot slot[b]; a negative slot is padding and touches nothing."""
    g = rng(10)
    S_slots, B, H, dk, dv = 5, 3, 2, 16, 16
    S = g.standard_normal((S_slots, H, dk, dv))
    ref = S.copy()
    q, k, v, alpha, beta = _rand_step(g, B, H, dk, dv, False)
    slot = np.array([4, -1, 1], np.int32)
    o = orc.gdn_step(S, q, k, v, alpha, beta, slot=slot)
    for b, s in enumerate(slot):
        if s < 0:
            assert np.isnan(o[b]).all()
            continue
        one = ref[s:s + 1].copy()
        o1 = orc.gdn_step(one, q[b:b + 1], k[b:b + 1], v[b:b + 1], alpha[b:b + 1], beta[b:b + 1])
        assert np.array_equal(one[0], S[s]) and np.array_equal(o1[0], o[b])
    for s in (0, 2, 3):
        assert np.array_equal(S[s], ref[s])


# ---------------------------------------------------------------- replay

def test_replay_matches_exact_sequential_steps(orc):
    """Replay of the first n accepted drafts = n exact-rational steps, per request; n = 0
    leaves the state untouched; n is clamped to [0, K]."""
    g = rng(11)
    B, K, H, dk, dv = 4, 3, 2, 3, 2
    S = _dyadic(g, (B, H, dk, dv))
    S0 = S.copy()
    q, k, v = _dyadic(g, (B, K, H, dk)), _dyadic(g, (B, K, H, dk)), _dyadic(g, (B, K, H, dv))
    alpha = g.integers(32, 65, size=(B, K, H)) / 64
    beta = g.integers(1, 65, size=(B, K, H)) / 64
    n_acc = np.array([0, 2, 3, 7], np.int32)  # 7 > K is clamped to K
    out = orc.replay(S, q, k, v, alpha, beta, n_acc, per_channel=False)
    assert np.array_equal(S[0], S0[0]) and np.isnan(out[0]).all()
    for b in range(1, B):
        n = min(int(n_acc[b]), K)
        for h in range(H):
            Sf = [[Fraction(x) for x in row] for row in S0[b, h]]
            for t in range(n):
                Sf, of = _frac_matrix_step(Sf, [Fraction(x) for x in q[b, t, h]],
                                           [Fraction(x) for x in k[b, t, h]],
                                           [Fraction(x) for x in v[b, t, h]],
                                           [Fraction(alpha[b, t, h])] * dk, Fraction(beta[b, t, h]))
                np.testing.assert_allclose(out[b, t, h], [float(x) for x in of], rtol=0, atol=1e-14)
            np.testing.assert_allclose(S[b, h], [[float(x) for x in r] for r in Sf], rtol=0,
                                       atol=1e-14)
            assert np.isnan(out[b, n:, h]).all()


def test_replay_equals_repeated_single_steps(orc):
    g = rng(12)
    B, K, H, dk, dv = 3, 4, 2, 16, 16
    S = g.standard_normal((B, H, dk, dv))
    S_seq = S.copy()
    q, k = _unit(g, B, K, H, dk), _unit(g, B, K, H, dk)
    v = g.standard_normal((B, K, H, dv))
    alpha = g.uniform(0.8, 1.0, (B, K, H, dk))
    beta = g.uniform(0, 1, (B, K, H))
    n_acc = np.array([1, 4, 2], np.int32)
    orc.replay(S, q, k, v, alpha, beta, n_acc, per_channel=True)
    for b in range(B):
        for t in range(n_acc[b]):
            orc.kda_step(S_seq[b:b + 1], q[b:b + 1, t], k[b:b + 1, t], v[b:b + 1, t],
                         alpha[b:b + 1, t], beta[b:b + 1, t])
    assert np.array_equal(S, S_seq)

"""Pins for the oracle's speculative-decoding pieces ("Serving recurrent attention",
part "Speculative decoding without state snapshots"): the verify pass (readouts at every
draft position, committed state untouched) and the fused replay of accepted drafts
followed by the target model's bonus token.

They are tied to exact-rational arithmetic of the transition-matrix form (DAMP Eq. (3)-
(4), written out in this file) and to the properties a verify pass must have: causality
(a draft only affects the readouts at and after its position) and no state change."""
from fractions import Fraction

import numpy as np
import pytest

rng = np.random.default_rng


def _frac_step(S, q, k, v, a, beta):
    """(I - beta k k^T) diag(a) S + beta k v^T and its readout, in exact rationals."""
    dk, dv = len(S), len(S[0])
    A = [[((1 if i == m else 0) - beta * k[i] * k[m]) * a[m] for m in range(dk)]
         for i in range(dk)]
    Sn = [[sum((A[i][m] * S[m][j] for m in range(dk)), Fraction(0)) + beta * k[i] * v[j]
           for j in range(dv)] for i in range(dk)]
    o = [sum((Sn[i][j] * q[i] for i in range(dk)), Fraction(0)) for j in range(dv)]
    return Sn, o


def _dyadic(g, shape, scale=64):
    return g.integers(-scale, scale + 1, size=shape) / scale


def _F(x):
    return [Fraction(float(y)) for y in x]


def _drafts(g, B, K, H, dk, dv, per_channel):
    q, k, v = _dyadic(g, (B, K, H, dk)), _dyadic(g, (B, K, H, dk)), _dyadic(g, (B, K, H, dv))
    alpha = g.integers(32, 65, size=(B, K, H, dk) if per_channel else (B, K, H)) / 64
    beta = g.integers(1, 65, size=(B, K, H)) / 64
    return q, k, v, alpha, beta


def _decay(alpha, idx, dk, per_channel):
    return _F(alpha[idx]) if per_channel else [Fraction(float(alpha[idx]))] * dk


@pytest.mark.parametrize("per_channel", [False, True])
def test_verify_matches_exact_steps_and_leaves_state(orc, per_channel):
    g = rng(60)
    B, K, H, dk, dv = 2, 4, 2, 3, 2
    S = _dyadic(g, (B, H, dk, dv))
    S0 = S.copy()
    q, k, v, alpha, beta = _drafts(g, B, K, H, dk, dv, per_channel)
    out = orc.verify(S, q, k, v, alpha, beta, per_channel=per_channel)
    assert np.array_equal(S, S0)
    for b in range(B):
        for h in range(H):
            Sf = [[Fraction(float(x)) for x in row] for row in S0[b, h]]
            for t in range(K):
                Sf, of = _frac_step(Sf, _F(q[b, t, h]), _F(k[b, t, h]), _F(v[b, t, h]),
                                    _decay(alpha, (b, t, h), dk, per_channel),
                                    Fraction(float(beta[b, t, h])))
                np.testing.assert_allclose(out[b, t, h], [float(x) for x in of], rtol=0,
                                           atol=1e-14)


def test_verify_from_zero_state_first_position_closed_form(orc):
    """From S = 0 the first draft's readout is beta (q.k) v."""
    g = rng(61)
    B, K, H, dk, dv = 3, 5, 2, 8, 6
    S = np.zeros((B, H, dk, dv))
    q, k = g.standard_normal((B, K, H, dk)), g.standard_normal((B, K, H, dk))
    v = g.standard_normal((B, K, H, dv))
    alpha = g.uniform(0.5, 1.0, (B, K, H))
    beta = g.uniform(0.1, 1.0, (B, K, H))
    out = orc.verify(S, q, k, v, alpha, beta, per_channel=False)
    ref = beta[:, 0, :, None] * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0])[..., None] * v[:, 0]
    np.testing.assert_allclose(out[:, 0], ref, rtol=1e-13, atol=1e-15)


def test_verify_is_causal(orc):
    """Changing draft j changes the readouts at positions >= j only."""
    g = rng(62)
    B, K, H, dk, dv = 2, 6, 3, 16, 8
    S = g.standard_normal((B, H, dk, dv))
    q, k, v, alpha, beta = (g.standard_normal((B, K, H, dk)), g.standard_normal((B, K, H, dk)),
                            g.standard_normal((B, K, H, dv)), g.uniform(0.8, 1, (B, K, H, dk)),
                            g.uniform(0, 1, (B, K, H)))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    out = orc.verify(S, q, k, v, alpha, beta, per_channel=True)
    j = 3
    v2 = v.copy()
    v2[:, j] += 1.0
    out2 = orc.verify(S, q, k, v2, alpha, beta, per_channel=True)
    assert np.array_equal(out[:, :j], out2[:, :j])
    assert (np.abs(out[:, j:] - out2[:, j:]).max(axis=(0, 2, 3)) > 0).all()


def test_verify_then_full_acceptance_replays_the_same_readouts(orc):
    """Accepting every draft: replay reproduces the verify readouts bit for bit (both run
    the same steps in the same order) and commits the state verify left alone."""
    g = rng(63)
    B, K, H, dk, dv = 3, 4, 2, 16, 16
    S = g.standard_normal((B, H, dk, dv))
    q, k, v, alpha, beta = (g.standard_normal((B, K, H, dk)), g.standard_normal((B, K, H, dk)),
                            g.standard_normal((B, K, H, dv)), g.uniform(0.8, 1, (B, K, H)),
                            g.uniform(0, 1, (B, K, H)))
    out_v = orc.verify(S, q, k, v, alpha, beta, per_channel=False)
    out_r = orc.replay(S, q, k, v, alpha, beta, np.full(B, K, np.int32), per_channel=False)
    assert np.array_equal(out_v, out_r)


@pytest.mark.parametrize("per_channel", [False, True])
def test_replay_bonus_matches_exact_steps(orc, per_channel):
    """n accepted drafts then the bonus token = n + 1 exact-rational steps; the bonus is
    applied also when nothing is accepted; n is clamped to [0, K]."""
    g = rng(64)
    B, K, H, dk, dv = 4, 3, 2, 3, 2
    S = _dyadic(g, (B, H, dk, dv))
    S0 = S.copy()
    q, k, v, alpha, beta = _drafts(g, B, K, H, dk, dv, per_channel)
    qb, kb, vb = _dyadic(g, (B, H, dk)), _dyadic(g, (B, H, dk)), _dyadic(g, (B, H, dv))
    ab = g.integers(32, 65, size=(B, H, dk) if per_channel else (B, H)) / 64
    bb = g.integers(1, 65, size=(B, H)) / 64
    n_acc = np.array([0, 2, 3, 9], np.int32)
    _, ob = orc.replay_bonus(S, q, k, v, alpha, beta, n_acc, qb, kb, vb, ab, bb,
                             per_channel=per_channel)
    for b in range(B):
        n = min(int(n_acc[b]), K)
        for h in range(H):
            Sf = [[Fraction(float(x)) for x in row] for row in S0[b, h]]
            for t in range(n):
                Sf, _ = _frac_step(Sf, _F(q[b, t, h]), _F(k[b, t, h]), _F(v[b, t, h]),
                                   _decay(alpha, (b, t, h), dk, per_channel),
                                   Fraction(float(beta[b, t, h])))
            Sf, of = _frac_step(Sf, _F(qb[b, h]), _F(kb[b, h]), _F(vb[b, h]),
                                _decay(ab, (b, h), dk, per_channel), Fraction(float(bb[b, h])))
            np.testing.assert_allclose(S[b, h], [[float(x) for x in r] for r in Sf], rtol=0,
                                       atol=1e-14)
            np.testing.assert_allclose(ob[b, h], [float(x) for x in of], rtol=0, atol=1e-14)


def test_replay_bonus_with_nothing_accepted_is_one_step(orc):
    g = rng(65)
    B, K, H, dk, dv = 2, 4, 3, 16, 8
    S = g.standard_normal((B, H, dk, dv))
    S1 = S.copy()
    q, k, v = (g.standard_normal((B, K, H, dk)), g.standard_normal((B, K, H, dk)),
               g.standard_normal((B, K, H, dv)))
    alpha, beta = g.uniform(0.8, 1, (B, K, H)), g.uniform(0, 1, (B, K, H))
    qb, kb, vb = g.standard_normal((B, H, dk)), g.standard_normal((B, H, dk)), g.standard_normal((B, H, dv))
    ab, bb = g.uniform(0.8, 1, (B, H)), g.uniform(0, 1, (B, H))
    _, ob = orc.replay_bonus(S, q, k, v, alpha, beta, np.zeros(B, np.int32), qb, kb, vb, ab, bb,
                             per_channel=False)
    o1 = orc.gdn_step(S1, qb, kb, vb, ab, bb)
    assert np.array_equal(S, S1) and np.array_equal(ob, o1)

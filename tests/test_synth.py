"""The seeded generators: same seed -> same bits, and draws that follow the stated recipes."""
import numpy as np

import synth


def test_steps_are_deterministic_and_distinct():
    cfg = synth.shrink(synth.CONFIGS["gdn_serving"], B=4)
    a, b, c = synth.step_inputs(cfg, 3), synth.step_inputs(cfg, 3), synth.step_inputs(cfg, 4)
    for n in a:
        assert a[n].dtype == b[n].dtype and np.array_equal(a[n], b[n])
    assert not np.array_equal(a["q"], c["q"])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0  # tie -> even (down)
    assert back[2] == 1.0 + 2 ** -6          # tie -> even (up)
    assert back[3] == -2.5
    ref = np.array([float(np.float32(v)) for v in x])
    assert np.all(np.abs(back - ref) <= np.abs(ref) * 2 ** -8)


def test_serving_recipe_shapes_ranges_and_norms():
    cfg = synth.shrink(synth.CONFIGS["kda_serving"], B=8)
    x = synth.step_inputs(cfg, 0)
    assert x["q"].dtype == np.uint16 and x["q"].shape == (8, 32, 128)
    assert x["alpha"].shape == (8, 32, 128) and x["beta"].shape == (8, 32)
    q = synth.stored_to_f64(x["q"], "bf16")
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=2e-2)
    assert (x["alpha"] > 0).all() and (x["alpha"] <= 1).all()
    assert (x["beta"] > 0).all() and (x["beta"] < 1).all()
    g = synth.step_inputs(synth.shrink(synth.CONFIGS["gdn_serving"], B=64), 0)
    assert g["alpha"].min() >= 0.90 and g["alpha"].max() <= 0.9999
    toy = synth.step_inputs(synth.CONFIGS["gdn_toy"], 0)
    assert toy["q"].dtype == np.float32 and toy["alpha"].min() >= 0.80


def test_kda_decay_spans_fast_and_slow_channels():
    cfg = synth.shrink(synth.CONFIGS["kda_serving"], B=16)
    a = synth.step_inputs(cfg, 0)["alpha"]
    assert (a < 0.5).mean() > 0.01 and (a > 0.99).mean() > 0.2


def test_initial_state_recipe():
    cfg = synth.shrink(synth.CONFIGS["gdn_serving"], B=2)
    s = synth.initial_state(cfg)
    assert s.dtype == np.float32 and s.shape == (2, 32, 128, 128)
    assert abs(float(s.std()) - 0.05) < 1e-3
    assert not synth.initial_state(synth.CONFIGS["gdn_toy"]).any()


def test_damp_plan_is_a_permutation_biased_to_slow_decay():
    cfg = synth.CONFIGS["damp_kda"]
    perm = synth.damp_key_perm(cfg)
    assert perm.shape == (32, 128) and perm.dtype == np.int32
    for h in range(32):
        assert np.array_equal(np.sort(perm[h]), np.arange(128))
        assert np.all(np.diff(perm[h, :16]) > 0) and np.all(np.diff(perm[h, 16:]) > 0)
    assert np.array_equal(perm, synth.damp_key_perm(cfg))


def test_dasc_masks_are_ragged_with_the_stated_total():
    cfg = synth.CONFIGS["dasc_gdn"]
    m = synth.dasc_masks(cfg)
    r = m.sum(1)
    assert m.shape == (4, 32) and r.sum() == 64 and r.min() >= 8 and r.max() <= 24
    assert len(set(r.tolist())) > 1


def test_replay_inputs():
    cfg = synth.CONFIGS["dasc_gdn"]
    d = synth.replay_inputs(cfg, 0, B=64)
    assert d["q"].shape == (64, 8, 32, 128) and d["alpha"].shape == (64, 8, 32)
    assert d["n_accept"].min() >= 0 and d["n_accept"].max() <= 8


def test_damp_value_plan():
    cfg = synth.CONFIGS["damp_kda_g32sr"]
    perm, scale = synth.damp_value_plan(cfg)
    assert perm.shape == (cfg.H, cfg.dv) and scale.shape == (cfg.H, cfg.dv)
    assert perm.dtype == np.int32 and scale.dtype == np.float32
    for h in range(cfg.H):
        assert sorted(perm[h].tolist()) == list(range(cfg.dv))
    assert (scale > 0).all()
    # stored order: largest RMS after scaling first, i.e. ascending scale
    assert (np.diff(scale, axis=1) >= 0).all()
    p2, s2 = synth.damp_value_plan(cfg)
    assert np.array_equal(perm, p2) and np.array_equal(scale, s2)
    assert synth.damp_group(cfg) == 32 and synth.damp_group(synth.CONFIGS["damp_kda"]) == 128


def test_gate_params():
    cfg = synth.CONFIGS["dasc_kda"]
    A, d = synth.gate_params(cfg)
    assert A.shape == d.shape == (cfg.L, cfg.H, cfg.dk) and A.dtype == np.float32
    A2, d2 = synth.gate_params(cfg)
    assert np.array_equal(A, A2) and np.array_equal(d, d2)
    # layers differ in their typical bias
    assert np.ptp(d.mean(axis=(1, 2))) > 0.3

"""Host-side contract of bench.py (no GPU): the single-GPU refusal, the algorithmic byte
counts the roofline divides by (recounted here from the per-head layouts), and the rule
that a counter-derived traffic figure is only used for the kernel source it was taken on."""
import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_unknown_only_names_are_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--only", "gdn,dmap"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "dmap" in p.stderr and p.stdout == ""


def test_step_bytes_recounted_per_head():
    # batch 256 x 32 heads x 128 x 128 FP32 state, bf16 q/k/v, fp32 decay/beta/readout
    heads = 256 * 32
    state = 128 * 128 * 4                      # 65,536 B per head, read and written
    inputs = 3 * 128 * 2                       # q, k, v in bf16
    gdn = heads * (2 * state + inputs + 4 + 4 + 128 * 4)
    kda = heads * (2 * state + inputs + 128 * 4 + 4 + 128 * 4)
    assert bench.step_bytes(256, 32, 128, 128, 2, False) == gdn == 1_084_293_120
    assert bench.step_bytes(256, 32, 128, 128, 2, True) == kda == 1_088_454_656


def test_damp_bytes_recounted_per_head():
    heads = 256 * 32
    # K_hi = 16 FP16 rows, 112 INT8 rows with one FP32 scale each: 18,880 B per head
    packed = 16 * 128 * 2 + 112 * 128 + 112 * 4
    assert packed == 18_880
    per_row = heads * (2 * packed + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4)
    assert bench.damp_bytes(256, 32, 128, 128, 16, 2, True) == per_row == 324_042_752
    # group-32 scales (4 per INT8 row) and the value tables (c' and pi, 32 x 128 x 8 B once)
    packed32 = 16 * 128 * 2 + 112 * (128 + 4 * 4)
    g32 = heads * (2 * packed32 + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 4) + 32 * 128 * 8
    assert bench.damp_bytes(256, 32, 128, 128, 16, 2, True, 32, True) == g32


def test_speculative_bytes_recounted():
    n = np.array([0, 3, 8, 1], np.int32)
    H, dk, dv = 2, 64, 32
    tok_in = (2 * dk + dv) * 4 + 4 + 4           # fp32 q, k, v, scalar decay, beta
    tok_nr = (dk + dv) * 4 + 4 + 4               # no readout: q not read
    # replay: states with at least one accepted token read + written, accepted tokens'
    # inputs read and readouts written
    assert bench.replay_bytes(n, H, dk, dv, 4) == 3 * H * 2 * dk * dv * 4 + 12 * H * (tok_in + dv * 4)
    assert bench.replay_bytes(n, H, dk, dv, 4, False) == 3 * H * 2 * dk * dv * 4 + 12 * H * tok_nr
    # verify: every state read once, every draft's inputs read and readout written
    assert bench.verify_bytes(4, 8, H, dk, dv, 4) == 4 * H * dk * dv * 4 + 4 * 8 * H * (tok_in + dv * 4)
    # replay + bonus: every state read + written, accepted inputs read, bonus in + out
    assert bench.bonus_bytes(n, H, dk, dv, 4) == (4 * H * 2 * dk * dv * 4 + 12 * H * tok_in
                                                  + 4 * H * (tok_in + dv * 4))


def test_fused_restore_replay_bytes_recounted():
    n = np.array([0, 3, 8, 1], np.int32)
    S, R, L, H, dk, dv = 4, 5, 3, 2, 64, 32
    head = dk * dv * 4
    tok_in = (dk + dv) * 4 + 4 + 4               # k, v, scalar decay, beta: no readout
    # retained checkpoint heads read once, every private head written once, each layer's
    # accepted tokens' inputs read
    want = S * R * head + L * S * H * head + L * 12 * H * tok_in
    assert bench.restore_replay_bytes(n, S, R, L, H, dk, dv, 4, readout=True) == (
        want + L * 12 * H * (dk * 4 + dv * 4))
    assert bench.restore_replay_bytes(n, S, R, L, H, dk, dv, 4) == want
    # the separate calls move every live state (3 of 4 requests) once more per layer, in
    # and out
    two = (S * R * head + L * S * H * head) + L * bench.replay_bytes(n, H, dk, dv, 4, False)
    assert two - want == L * 3 * H * 2 * head
    # units of single key channels (R of them), per-channel decay read with each token
    tok_kda = (dk + dv) * 4 + dk * 4 + 4
    assert bench.restore_replay_bytes(n, S, R, L, H, dk, dv, 4, unit_rows=1,
                                      vector_decay=True) == (S * R * dv * 4 + L * S * H * head
                                                             + L * 12 * H * tok_kda)
    # an INT8 checkpoint: each retained row's dv codes and its FP32 scale
    assert bench.restore_replay_bytes(n, S, R, L, H, dk, dv, 4, unit_rows=1, vector_decay=True,
                                      int8=True) == (S * R * (dv + 4) + L * S * H * head
                                                     + L * 12 * H * tok_kda)
    assert bench.replay_bytes(n, H, dk, dv, 4, False, vector_decay=True) == (
        3 * H * 2 * head + 12 * H * tok_kda)


def test_traffic_only_for_the_profiled_source():
    assert bench.traffic_from_profile("gdn_step", ["bench.py"]) is None
    assert bench.traffic_from_profile("no_such_kernel", bench.STEP_SOURCES) is None


def test_cpu_baseline_runs_the_oracle_on_the_gpu_inputs():
    """The CPU baseline's fields, on the input sets the caller names (the benchmark passes
    the ones its first timed GPU steps use); a short budget keeps this test quick."""
    import synth

    r = bench.cpu_baseline(synth, 0.4, (3, 4))
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "GB/s" and r["value"] > 0
    assert "input sets [3, 4]" in r["sample"]
    assert r["host_cpus"] >= 1 and r["cpu_model"]
    if "all_cores" in r:
        assert r["all_cores"]["cores"] == bench.host_threads() and r["all_cores"]["value"] > 0


def test_free_running_figures_only_for_the_recorded_source(tmp_path, monkeypatch):
    """The benchmark quotes the recorded free-running figures only when they were taken on
    the current mixed-precision kernel source."""
    import json

    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.drift_vs_oracle("damp_kda") is None
    rec = {"1": {"code_frac": 1e-6, "drift_gpu": 0.007, "drift_oracle": 0.007, "other": 1}}
    for h, want in (("0" * 16, None), (bench.source_hash(bench.DAMP_SOURCES), "match")):
        (tmp_path / "damp_free_running_damp_kda.json").write_text(
            json.dumps({"source_hash": h, "at": rec}))
        got = bench.drift_vs_oracle("damp_kda")
        if want is None:
            assert got is None
        else:
            assert got == {"1": {"code_frac": 1e-6, "drift_gpu": 0.007, "drift_oracle": 0.007}}


def test_input_copies_span_the_last_level_cache():
    """Timed launches rotate over copies of their checkpoint / draft inputs: together the
    copies span at least three times the 256 MB last-level cache, so at least twice the
    cache is read between two reads of one copy; an input above the cache needs none."""
    llc = 256 << 20
    assert bench.LLC_BYTES == llc
    for nbytes, want in [(266 << 20, 3), (528 << 20, 2), (201_326_592, 4), (2 << 30, 1),
                         (llc, 3), (1, 3 * llc)]:
        n = bench.n_copies(nbytes)
        assert n == want, (nbytes, n)
        assert n * nbytes >= 3 * llc or n == 1
        if nbytes <= llc:
            assert (n - 1) * nbytes >= 2 * llc

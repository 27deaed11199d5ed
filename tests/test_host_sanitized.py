"""The library's host-only code (argument checks, ragged plans, static horizons, replay
windows) and the float64 oracle, each built with AddressSanitizer and
UndefinedBehaviorSanitizer (gcc / g++, no GPU code) and driven with ordinary and
adversarial arguments (for the host checks, sizes whose products do not fit in 64 bits):
any sanitizer report or failed invariant fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "hybrid_linear_attention_step_amd", "csrc"),
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(ROOT, "hybrid_linear_attention_step_amd", "csrc", "hla_host.cpp"),
           "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    """Every oracle entry point on small ragged shapes with exactly sized heap buffers
    (tests/oracle_sanitize_driver.cpp)."""
    san = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
    obj, exe = tmp_path / "oracle.o", tmp_path / "oracle_driver"
    c = subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *san, "-c",
                        os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(obj)],
                       capture_output=True, text=True, timeout=300)
    assert c.returncode == 0, c.stderr
    b = subprocess.run(["g++", "-std=c++17", *san,
                        os.path.join(ROOT, "tests", "oracle_sanitize_driver.cpp"), str(obj),
                        "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr

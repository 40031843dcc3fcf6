"""The CPU oracle (oracle/*.c) and the input generator (synth/synth.c) built
with AddressSanitizer and UndefinedBehaviorSanitizer, driven over every entry
point on small ragged shapes by tests/sanitize_driver.c (host code only).
Any out-of-bounds access, use after free or undefined operation aborts the
driver; so does a documented bad-size return that is not taken."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "sanitize_driver.c"), os.path.join(ROOT, "oracle", "q4k_oracle.c"),
           os.path.join(ROOT, "oracle", "mixer_oracle.c"), os.path.join(ROOT, "synth", "synth.c")]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("san") / "sanitize_driver")
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.check_call(["gcc"] + flags + ["-o", exe] + SOURCES + ["-lm"])
    return exe


def test_oracle_and_generator_clean_under_asan_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=24",
               OMP_NUM_THREADS="3")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "runs clean" in r.stdout

"""The C oracle built with gcc's address and undefined-behaviour sanitizers and
run over small and edge shapes (empty and one-token sequences, ragged last
chunks, chunk sizes 1 and wider than the stream, M = 1..4, strided rows,
absent optional inputs and outputs).  Any out-of-bounds access, leak or
undefined operation fails the run; the values are pinned elsewhere."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


def _build(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", os.path.join(ORACLE, "gdp_oracle.c"), os.path.join(ORACLE, "sanitize_check.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr or "ubsan" in r.stderr):
        pytest.skip("gcc has no sanitizer runtime here: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"

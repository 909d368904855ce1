"""The C oracle under AddressSanitizer and UBSan (with OpenMP threads).

tests/native/oracle_sanitize.c calls every oracle entry over exact-size heap
buffers: ragged groups, one- and two-sided rotations, row subsets, T = 0,
every fp16/bf16 pattern through the conversions and every block size of the
transform.  The build is gcc only and never touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "nl_oracle.c"), os.path.join(ROOT, "tests", "native", "oracle_sanitize.c"),
           "-lm", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    if b.returncode != 0 and "asan" in (b.stderr or "").lower():
        pytest.skip("gcc has no sanitizer runtime here: " + b.stderr[-300:])
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "oracle sanitize: ok" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]

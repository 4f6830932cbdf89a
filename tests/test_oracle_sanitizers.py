"""The CPU oracle under the host AddressSanitizer and UndefinedBehaviorSanitizer:
oracle/sanitize_check.c runs every oracle entry point (per-token casts in both
orientations, every group size, scale format and input type; per-block casts;
the GEMM reference in full and sampled form; the element-wise helpers) on
ragged shapes with exactly sized buffers, built with gcc
-fsanitize=address,undefined -fno-sanitize-recover=all."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "sanitize_check")
    src = os.path.join(ROOT, "oracle", "sanitize_check.c")
    build = subprocess.run([gcc, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            "-fno-omit-frame-pointer", "-ffp-contract=off", "-fopenmp", "-I",
                            os.path.join(ROOT, "oracle"), src, "-o", exe, "-lm"], capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("gcc without sanitizer runtimes: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ran clean" in run.stdout

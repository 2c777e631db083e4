"""AddressSanitizer + UndefinedBehaviorSanitizer build of the fp64 oracle and
the seeded input generator (CPU only).

tests/sanitize/san_driver.c calls every exported routine of both on small
shapes (NVFP4 with W4A4, BF16 and MXFP8 expert sets; B = 1 and a ragged
B = 5) with buffers of exactly the sizes their contracts state, so any
access past a buffer, any leak and any undefined operation fails the run.
"""
import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "san_driver"
    cmd = [gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-fopenmp", "-o", str(exe),
           str(ROOT / "tests" / "sanitize" / "san_driver.c"), str(ROOT / "oracle" / "moe_oracle.c"),
           str(ROOT / "testgen" / "testgen.c"), "-lm"]
    built = subprocess.run(cmd, capture_output=True, text=True)
    if built.returncode != 0 and "asan" in built.stderr.lower():
        pytest.skip("the sanitizer runtimes are not installed: " + built.stderr[-300:])
    assert built.returncode == 0, built.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "OK" in run.stdout

"""The W4A4 quantiser's division through a correctly rounded reciprocal
(CPU only).

The single-launch kernel's Four Over Six quantiser divides each of a
block's 16 values by the block's two candidate divisors.  Rather than 32
correctly rounded divisions it forms each divisor's correctly rounded
reciprocal once and takes q = RN(v y) plus one FMA residual step, which is
the correctly rounded quotient by Markstein's theorem.  tests/recip/recip_div.c
checks that claim against IEEE division on the host: bit for bit for every
bf16 significand against every fp32 divisor significand, and, over every
bf16 value and divisors across [2^-64, 2^64] (the range the kernel takes
this path for), equal E2M1 codes for every quotient the quantiser can meet;
and every bf16 block maximum divided by 6 the same way, bit for bit.
"""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_reciprocal_division_is_correctly_rounded(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "recip_div"
    cmd = [gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-o", str(exe),
           str(ROOT / "tests" / "recip" / "recip_div.c"), "-lm"]
    built = subprocess.run(cmd, capture_output=True, text=True)
    assert built.returncode == 0, built.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "mismatches 0 0 0" in run.stdout

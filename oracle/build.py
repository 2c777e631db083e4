"""Compile the fp64 CPU oracle (plain C, OpenMP) in place.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg load the library this builds.
"""
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
LIB = HERE / "libmoe_oracle.so"


def build() -> pathlib.Path:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-o", str(LIB), str(HERE / "moe_oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build())

"""Compile the seeded input generator (plain C, OpenMP) in place."""
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
LIB = HERE / "libtestgen.so"


def build() -> pathlib.Path:
    cmd = ["gcc", "-O3", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-o", str(LIB), str(HERE / "testgen.c"), "-lm"]
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build())

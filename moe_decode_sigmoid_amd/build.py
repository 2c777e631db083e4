"""Compile the gfx950 HIP library (libmoe_decode.so) in place with hipcc."""
import os
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
CSRC = HERE / "csrc"
LIB = HERE / "libmoe_decode.so"
SOURCES = ["capi.hip", "decode.hip", "decode_fused.hip", "prefill.hip", "gemv.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: ordinary fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(HERE.parent / "include"),
]


def build(verbose: bool = False) -> pathlib.Path:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc, *FLAGS, "-o", str(tmp), *[str(CSRC / s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Compile the gfx950 HIP library (libmoe_decode.so) in place with hipcc:
each source to an object in parallel (the single-launch decode kernels'
instances are spread over several sources, one weight format each), then
one link."""
import concurrent.futures
import os
import pathlib
import subprocess

HERE = pathlib.Path(__file__).resolve().parent
CSRC = HERE / "csrc"
OBJ = HERE / "_build"
LIB = HERE / "libmoe_decode.so"
SOURCES = ["capi.hip", "decode.hip", "decode_fused.hip", "decode_fused_nv.hip",
           "decode_fused_bf.hip", "decode_fused_ns2.hip", "decode_fused_a4.hip", "decode_stack.hip", "decode_chain_nv.hip", "decode_chain_bf.hip",
           "decode_general.hip", "prefill.hip", "gemv.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off: ordinary fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", str(HERE.parent / "include"),
]


def build(verbose: bool = False) -> pathlib.Path:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    OBJ.mkdir(exist_ok=True)
    objs = [OBJ / (pathlib.Path(s).stem + ".o") for s in SOURCES]

    def compile_one(src_obj):
        src, obj = src_obj
        cmd = [hipcc, *FLAGS, "-c", "-o", str(obj), str(CSRC / src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        list(pool.map(compile_one, zip(SOURCES, objs)))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds the HIP library ``_lib/libmoe_step.so`` in-tree for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "moe_step.hip")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libmoe_step.so")
BENCH_SRC = os.path.join(HERE, "csrc", "moe_step_bench.cpp")
BENCH = os.path.join(OUT_DIR, "moe_step_bench")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep hand-written and compiler-formed packed fp32 arithmetic out of the code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB)
    # C++ driver of the ABI (profiling runs without Python)
    tmpb = BENCH + ".tmp"
    cmdb = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-x", "hip", BENCH_SRC, "-o", tmpb,
            "-L" + OUT_DIR, "-lmoe_step", "-Wl,-rpath,$ORIGIN"]
    res = subprocess.run(cmdb, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc (bench driver) failed:\n" + res.stdout + res.stderr)
    os.replace(tmpb, BENCH)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

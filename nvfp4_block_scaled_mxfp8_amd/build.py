"""Builds libgmlp.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m nvfp4_block_scaled_mxfp8_amd.build

Compiles every source under csrc/ with hipcc into one shared library next to
this file.  Flags: -O3, gfx950 only, no fast-math (correctly rounded fp32
division is relied on by the NVFP4 cast), fp contraction off (bit-reproducible
epilogues), and packed-fp32 instructions disabled.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgmlp.so")
SOURCES = ["quant.hip", "gemm.hip", "static_ws.hip", "api.cpp"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-variable",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the gmlp library needs ROCm's hipcc to build")
    return exe


def build(verbose=True, extra_flags=()):
    """Compile libgmlp.so; raises on a compiler error."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "unknown target feature"           # host pass does not know the packed-fp32 feature
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l and "packed-fp32" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    print("built", LIB)

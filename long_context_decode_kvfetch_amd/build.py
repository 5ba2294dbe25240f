"""Build libverkv.so (HIP kernels + C ABI) for gfx950 with hipcc, in the package dir.

    python -m long_context_decode_kvfetch_amd.build        # or build() from Python
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libverkv.so")
SOURCES = ["k_compress.hip", "k_sketch.hip", "k_quant.hip", "k_decide.hip", "k_attend.hip",
           "k_prefetch.hip", "verkv_api.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                  # every fused multiply-add is written explicitly
    "-munsafe-fp-atomics",                # LDS float64 atomic adds as ds_add_f64
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *FLAGS, "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libverkv.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

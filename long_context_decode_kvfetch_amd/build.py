"""Build libverkv.so (HIP kernels + C ABI) for gfx950 with hipcc, in the package dir.

    python -m long_context_decode_kvfetch_amd.build        # or build() from Python
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libverkv.so")
SOURCES = ["k_compress.hip", "k_append.hip", "k_sketch.hip", "k_quant.hip", "k_decide.hip", "k_resolve.hip", "k_attend.hip",
           "k_prefetch.hip", "verkv_api.cpp"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",                  # every fused multiply-add is written explicitly
    "-munsafe-fp-atomics",                # LDS float64 atomic adds as ds_add_f64
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


HEADER = os.path.join(os.path.dirname(HERE), "include", "verkv.h")

# A second build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
# only (the C ABI's argument checks, layouts and launch set-up; the GPU code is built
# as usual).  It needs the sanitizer runtime preloaded into the process that loads it
# (tests/test_host_sanitizers.py does that for the host ABI tests).
SANITIZED_LIB = os.path.join(HERE, "libverkv_hostsan.so")
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-shared-libsan",
]


def source_hash() -> str:
    """SHA-256 over every file under csrc/, the public header and the compiler flags: the
    identity of a build, compiled into the library (verkv_source_hash) so a loaded
    libverkv.so can be checked against the sources it claims to come from."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC))
    for name in files:
        h.update(name.encode() + b"\0")
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(HEADER, "rb") as f:
        h.update(f.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def sanitizer_runtime() -> str:
    """The AddressSanitizer runtime of the compiler that builds SANITIZED_LIB."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return found[-1]


def build(verbose: bool = False, sanitize_host: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = SANITIZED_LIB if sanitize_host else LIB
    tmp = out + ".tmp"
    extra = HOST_SANITIZE if sanitize_host else []
    cmd = [hipcc, *FLAGS, *extra, f'-DVERKV_SOURCE_HASH="{source_hash()}"', "-x", "hip",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libverkv.so")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

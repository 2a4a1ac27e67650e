"""Builds libpkv.so (the HIP kernels and the C ABI of include/pkv.h) for gfx950.

    python -m paged_kv_attention_scatter_amd.build      # or build() from Python

Always recompiles. The library lands next to this file, inside the package,
so it travels with the source tree."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpkv.so")
# The same library with its host code built under AddressSanitizer and
# UndefinedBehaviorSanitizer (device code as usual): tests/test_abi_sanitized.py
# runs the host-side ABI tests against it.
SAN_LIB = os.path.join(HERE, "libpkv_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan", "-g"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed FP32 VALU ops stay off: hipcc must not emit v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def sanitizer_runtime() -> str:
    """The clang ASan runtime the sanitized build links against (to preload)."""
    import glob
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    found = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("no clang ASan runtime under " + rocm)
    return found[-1]


def build(verbose: bool = False, sanitized: bool = False) -> str:
    out = SAN_LIB if sanitized else LIB
    tmp = out + ".tmp"
    flags = [*HIPCC_FLAGS, *SAN_FLAGS] if sanitized else HIPCC_FLAGS
    cmd = [hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, "pkv.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    if "--sanitized" in sys.argv:
        print(build(verbose=True, sanitized=True))

"""Build the HIP library ``libkvq.so`` for gfx950 in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.hip", "kvq_append.hip", "kvq_decode.hip", "kvq_prefill.hip", "kvq_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep fp32 division and rounding IEEE: the quantizer's codes must match the oracle's bits
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math", "-ffp-contract=off",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in VGPRs: the decode loop's rare rescale then needs no AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # the first 16 kernel-argument dwords arrive in SGPRs with the wave (the decode and merge
    # kernels lead with the scalars of their first memory accesses)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-result",
]


# The host half of the library built with AddressSanitizer and UndefinedBehaviorSanitizer (the
# device code is unchanged): the CPU tests of argument validation and planning run against it.
SANITIZED_LIB = os.path.join(HERE, "libkvq_san.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


# The device-side range-check build (kernels also report corrected page ids and slots; see
# kvq_debug_errors in include/kvq.h).
DEBUG_LIB = os.path.join(HERE, "libkvq_debug.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc's host compiler (to LD_PRELOAD into a
    Python process that loads the sanitized library)."""
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    return found[-1]


def build(verbose: bool = False, extra: list[str] | None = None, out: str = LIB,
          sanitize: bool = False, debug: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    if sanitize:
        extra = [*(extra or []), *HOST_SANITIZE]
        out = SANITIZED_LIB if out == LIB else out
    if debug:
        extra = [*(extra or []), "-DKVQ_DEBUG"]
        out = DEBUG_LIB if out == LIB else out
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", out + ".tmp", *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature and says so; that is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, debug=True))

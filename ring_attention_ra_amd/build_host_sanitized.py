"""Build a copy of libra.so whose HOST code carries AddressSanitizer and
UndefinedBehaviorSanitizer, for running the library's argument validation
(size arithmetic, limit checks, error-message formatting) under both.

The device code is compiled exactly as in the product build; every sanitizer
flag is given to the host pass only (each one right after -Xarch_host), so no
GPU code is instrumented. The result goes to _build/host_sanitized/libra.so
and is loaded through RA_LIB by a process started with the ASan runtime in
LD_PRELOAD (Python itself is not instrumented). It is a test build: nothing in
the product loads it.

Usage: python -m ring_attention_ra_amd.build_host_sanitized
"""

from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from ring_attention_ra_amd import build as _build

OUT = os.path.join(_build.BUILD, "host_sanitized")

_HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address",
                  "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the shared ASan runtime of the ROCm clang that hipcc drives."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    flags = [f for f in _build.HIP_FLAGS if f != "-O3"]
    cmd = [_build.hipcc(), "-O1", "-g", *flags, *_HOST_SANITIZE, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source with host-side sanitizers and link; returns the path."""
    os.makedirs(OUT, exist_ok=True)
    srcs = _build.sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    lib = os.path.join(OUT, "libra.so")
    cmd = [_build.hipcc(), f"--offload-arch={_build.ARCH}", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan",
           "-o", lib, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True)

"""Build libkvsel.so (gfx950) in-tree with hipcc.

Every source under csrc/ is compiled to an object (in parallel) and linked
into ``attention_score_guided_amd/libkvsel.so``.  Run as a script or call
``build()``; it always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkvsel.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for every device pass.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-result", "-I", os.path.join(HERE, "..", "include")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkvsel.so")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


# Host-side AddressSanitizer for the CPU tests of the C ABI: only the host
# pass is instrumented (the device code is built as usual).
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_OUT = os.path.join(HERE, "_build_asan", "libkvsel_asan.so")


def _compile(src: str, build_dir: str = BUILD_DIR, defines=(), extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *extra, *[f"-D{d}" for d in defines], "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = OUT, build_dir: str = BUILD_DIR, defines=(),
          host_asan: bool = False) -> str:
    """Compile every source and link ``out``.  ``defines`` are extra -D
    tuning macros (the defaults in the sources are the shipped values).
    ``host_asan`` instruments the host code with AddressSanitizer (a test
    build: load it with the sanitizer runtime preloaded)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    extra = HOST_ASAN if host_asan else []
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, defines, extra), srcs))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""The host code of the C ABI under AddressSanitizer (CPU only): the library
is rebuilt with the host pass instrumented and tests/test_abi.py runs against
it in a subprocess with the sanitizer runtime preloaded.  Every validation
path (NULL pointers, bad sizes, strides, workspaces, the allocation-free
entry point's size check) then runs with out-of-bounds and use-after-free
detection on the host side."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_asan():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_kvsel_build", os.path.join(ROOT, "attention_score_guided_amd",
                                                                             "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    out = b.ASAN_OUT
    newest = max(os.path.getmtime(p) for p in b.sources() + glob.glob(os.path.join(ROOT, "include", "*.h")))
    if not os.path.exists(out) or os.path.getmtime(out) < newest:
        b.build(out=out, build_dir=os.path.dirname(out), host_asan=True)
    return out


def test_abi_under_host_asan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    lib = _build_asan()
    env = dict(os.environ, KVSEL_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail

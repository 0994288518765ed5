"""CPU: the host side of the C ABI under AddressSanitizer and UBSan.

The API layer (api.hip: argument checks, workspace sizing, dispatch) is
compiled with the sanitizers on its host code only, linked with the other
objects of the in-tree build, and the whole ABI test module (every
validation path, no kernel launch) runs against that library in a child
process with the sanitizer runtime preloaded.  Any report makes the child
fail (UBSan without recovery, ASan halting on its first error)."""
import glob
import os
import subprocess
import sys

import pytest

import kv_cache_selection_sp_amd as sp
from kv_cache_selection_sp_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    out = subprocess.run([B._hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_checks_under_host_sanitizers(tmp_path):
    objs = sorted(glob.glob(os.path.join(B.BUILD_DIR, "*.hip.o")))
    others = [o for o in objs if not o.endswith("api.hip.o")]
    assert others, "in-tree build objects missing: python -m kv_cache_selection_sp_amd.build"
    rt = _asan_runtime()
    assert rt, "the clang AddressSanitizer runtime is not installed with hipcc"
    hipcc = B._hipcc()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in B.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    api_o = str(tmp_path / "api_san.o")
    lib = str(tmp_path / "libspdecode.so")
    r = subprocess.run([hipcc, *flags, *san, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *san, "-shared-libsan",
                        "-o", lib, api_o, *others], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    # the child loads the sanitized library first (binding cache), then runs
    # the ABI tests, whose fixture then uses it
    code = ("import sys, pytest\n"
            "import kv_cache_selection_sp_amd as sp\n"
            f"sp.load({lib!r})\n"
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))\n")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail

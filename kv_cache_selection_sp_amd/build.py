"""Build libspdecode.so for gfx950 with hipcc (in-tree, no JIT cache).

Each HIP source is compiled to an object in parallel, then linked into
``kv_cache_selection_sp_amd/libspdecode.so``.  Usage: ``python -m
kv_cache_selection_sp_amd.build`` or ``build()`` from Python.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libspdecode.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # keep packed fp32 VALU ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the online-softmax rescale of the
    # output tiles then needs no accumulator-register copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Per-source additions.  The prompt-scoring sweeps take maxima of MFMA
# results, which are never signalling NaNs: without NaN semantics the compiler
# drops the quieting max in front of every fmaxf (a fifth of the normaliser
# sweep's vector instructions, which compete with its MFMAs for issue).
FILE_FLAGS = {
    "k_snapkv.hip": ["-fno-honor-nans"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link the shared library.
    Always recompiles.  Returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = (r.stdout + r.stderr).strip()
        # hipcc's host pass does not know the GPU target feature: harmless noise
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out:
            print(out, file=sys.stderr)
        return obj

    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)

"""CPU guard for the direct global-to-LDS loads: a direct load writes a whole
wave's 64 dwords, so every LDS region a direct-load loop fills must cover that
loop's write extent, for every shape the entry points accept.  The layouts
are compiled from the kernels' own header (csrc/lds_layout.h) into a host
program (tests/lds/lds_layout_check.cpp) that restates each loop."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_selection_sp_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "lds", "lds_layout_check.cpp")


def test_direct_load_regions_cover_their_loops(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "lds_layout_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", f"-I{CSRC}", SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed" in r.stdout

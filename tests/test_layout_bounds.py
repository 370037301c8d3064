"""CPU check of the lifted-workspace layout and the direct global -> LDS tile
copies: tests/layout_bounds.cpp is compiled for the host from the library's
own headers (the offset functions and copy arithmetic the kernels use) and
run here.  It covers every tile size the kernels copy, the 64-bit address
join with bit 31 of the low half set, and the layout of the benchmark
configurations and of ragged and odd shapes (see the program's header)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_layout_and_copy_bounds(tmp_path):
    exe = tmp_path / "layout_bounds"
    cmd = [HIPCC, "-std=c++17", "-O1", "-x", "hip", "--offload-host-only",
           os.path.join(HERE, "layout_bounds.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "checks ok" in r.stdout

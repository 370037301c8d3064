"""Build libflashipa.so for gfx950 with hipcc (in-tree, next to this file)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libflashipa.so")
SOURCES = ["abi.cpp", "lift.hip", "flash_f32.hip", "flash_mfma.hip", "epilogue.hip", "diag.hip", "knn.hip", "backward.hip", "flashbias.hip", "noalloc.hip"]
ARCH = os.environ.get("FLASHIPA_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # no packed fp32 VALU instructions anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str, obj_dir: str, csrc: str = CSRC) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, csrc: str = CSRC, out: str = OUT, obj_dir: str = None) -> str:
    """Compile the HIP sources in `csrc` into the shared library `out`."""
    obj_dir = obj_dir or os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, csrc), SOURCES))
    tmp = out + ".tmp"
    # roctx ranges over the ABI calls (rocprofv3 --marker-trace)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

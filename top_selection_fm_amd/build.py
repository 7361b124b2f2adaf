"""Build libfm.so (HIP, gfx950) in-tree with hipcc.

    python -m top_selection_fm_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection turned
off (-packed-fp32-ops), and linked into top_selection_fm_amd/libfm.so next to this file.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libfm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str = SO, defines=()) -> str:
    """Compile every csrc/*.hip into `out`; `defines` are extra -D options (tuning knobs)."""
    srcs = sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
           *[f"-D{d}" for d in defines], *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

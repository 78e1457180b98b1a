"""Build libls_replay.so (the HIP/C ABI library) in-tree for gfx950.

    python -m response_replay_attention_amd.build      (or: python response_replay_attention_amd/build.py)

Every HIP source is compiled with packed-FP32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass prints a
harmless "not a recognized feature" warning for it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libls_replay.so")
BUILD = os.path.join(PKG, "_build")

SOURCES = ["ls_fwd.hip", "ls_bwd.hip", "ls_merge.hip", "ls_static.hip", "ls_calib.hip", "ls_api.cpp"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


# Per-source additions.  ls_bwd.hip: MFMA results in VGPR form.  The response
# dK/dV kernel needs more than 256 registers per wave; left to choose, the
# compiler keeps its accumulators in AGPRs and copies values between the two
# register files around every block (hundreds of moves per block).  The prompt
# kernels of that file compile to the same code either way.
EXTRA_FLAGS = {"ls_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # resolve every symbol now, so a missing kernel launch stub fails the build
    import ctypes
    ctypes.CDLL(tmp, mode=os.RTLD_NOW)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Build the HIP library ``libeta.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libeta.so")
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libeta_probe.so")  # measurement aid (bench.py)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
# atomic optimizer off: for an atomic issued by one lane, the optimizer broadcasts
# the returned value to the wave at once, so the wave waits for the atomic's round
# trip where it is issued; the attention fetches its next work item's ticket at an
# item's start and reads it only at the item's end.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
             "-Wall", "-Wno-unused-command-line-argument"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc(srcs: list[str], out: str, verbose: bool) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_lib(out: str = LIB_PATH, verbose: bool = False) -> str:
    """Compile every ``csrc/*.hip`` into one shared library, and the read probe
    ``csrc/probe/*.hip`` into its own (always recompiles both)."""
    _hipcc(sources(), out, verbose)
    _hipcc(sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))), PROBE_LIB_PATH, verbose)
    return out


def ensure_built() -> str:
    """Build the libraries only if one is absent (tests and benchmarks use this)."""
    if not os.path.exists(LIB_PATH) or not os.path.exists(PROBE_LIB_PATH):
        build_lib()
    return LIB_PATH

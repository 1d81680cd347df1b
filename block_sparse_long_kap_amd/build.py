"""Build the gfx950 shared library ``libcosa.so`` in-tree with hipcc.

Usage: ``python -m block_sparse_long_kap_amd.build`` (or ``build_library()``).
The library is written next to this file; the Python binding loads it from
there and fails loudly if it is missing.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libcosa.so")
SOURCES = ["cosa_api.hip", "attn_fwd.hip", "kap.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand) and shutil.which(cand) is None:
        raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")
    return cand


def compile_command(out: str = LIB_PATH, extra=()) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden",
            # packed-FP32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}", *extra,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build_library(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))

"""Builds libgdn2.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage:  python -m gated_delta_rule_gdn_amd.build      (or build() from Python)
The library lands in gated_delta_rule_gdn_amd/_build/libgdn2.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(OUT_DIR, "libgdn2.so")
SOURCES = ["gdn2_api.cpp", "gdn2_decode.hip", "gdn2_chunk.hip", "gdn2_gates.hip", "gdn2_bwd.hip",
           "gdn2_noalloc.hip", "gdn2_prep.hip", "gdn2_state.hip", "gdn2_bwd16.hip"]
ARCH = "gfx950"
# Packed-fp32 VALU forms are kept out of generated code (hipcc's host pass warns that it
# does not know the feature; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdn2)")


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link libgdn2.so. Returns its path."""
    hipcc = _hipcc()
    os.makedirs(OUT_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT_DIR, src + ".o")
        cmd = [hipcc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

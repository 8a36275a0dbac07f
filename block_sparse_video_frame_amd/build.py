"""Builds libbsvf.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: ``python -m block_sparse_video_frame_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsvf.so")
SOURCES = ["bsvf_host.cpp", "attn_norms.hip", "attn_qk_prep.hip", "attn_fwd.hip"]
ARCH = os.environ.get("BSVF_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-I", INCLUDE, "-I", CSRC,
        # packed FP32 VALU forms stay off
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 into ``libbsvf.so`` (always recompiles)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for s in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, s), "-o", obj]
        if s.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and l.strip())
        if verbose and out:
            print(out, file=sys.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {s}:\n{out}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

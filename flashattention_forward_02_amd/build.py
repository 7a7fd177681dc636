"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: ``python -m flashattention_forward_02_amd.build`` or ``build()`` from Python.
Objects go to ``_build/`` at the repository root; the library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["fa_api.hip", "fwd_mfma.hip", "fwd_f32.hip", "decode.hip", "merge.hip", "bwd.hip", "probe.hip"]
# Packed fp32 VALU instructions are disabled for every device pass.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = [ln for ln in p.stdout.splitlines() if "packed-fp32-ops" not in ln]
    return p.returncode, "\n".join(lines)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source for gfx950 and link libfa.so; returns the library path. Raises on failure."""
    os.makedirs(BUILD, exist_ok=True)
    flags = COMMON + list(extra_flags or [])

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        rc, out = _run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        return src, obj, rc, out

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for src, _, rc, out in results:
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [r[1] for r in results])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])

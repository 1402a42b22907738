"""Compile the HIP library for gfx950, in-tree: decode_step_05_amd/liblfdecode.so."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblfdecode.so")
SOURCES = [os.path.join(CSRC, "lfdecode.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("lf_device.h", "lf_kernels.h", "lf_exchange.h", "lf_prefill.h", "lf_sample.h", "lf_batch.h")] + [os.path.join(ROOT, "include", "lfdecode.h")]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_cmd(out: str, extra=()) -> list:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 instructions stay off for all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *extra, *SOURCES, "-o", out]


def build(verbose: bool = False) -> str:
    """Always recompiles; writes the library atomically."""
    tmp = LIB + ".tmp"
    r = subprocess.run(compile_cmd(tmp), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds libstmat.so in-tree with hipcc for gfx950 (cross-compiles; no GPU needed)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libstmat.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: IEEE semantics (no contraction, no fast-math, fp32 subnormals kept) and no
# packed-fp32 instructions.
DEVICE = ["-O3", f"--offload-arch={ARCH}", "-ffp-contract=off", "-fno-fast-math",
          "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # kernel arguments arrive in SGPRs instead of through a scalar load
          "-mllvm", "-amdgpu-kernarg-preload-count=8"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}")
    return r.stdout


def build(verbose: bool = False, extra_device_flags=(), out: str = LIB, defines=(), build_dir: str = BUILD) -> str:
    """Compile every source and link libstmat.so; returns its path.  ``defines`` (e.g.
    "STK_WORDS_FP8=4") override the compile-time work-unit geometry in every source."""
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    objs = []
    # host-only sources
    for src in ("index.cpp", "stream_plan.cpp"):
        o = os.path.join(build_dir, src + ".o")
        _run(["g++", "-O2", *COMMON, *dflags, "-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    # sources that call the HIP runtime or hold kernels
    for src in ("stage.cpp", "materialize.hip"):
        o = os.path.join(build_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC, *lang, *COMMON, *DEVICE, *dflags, *extra_device_flags, "-c", os.path.join(CSRC, src), "-o", o], verbose)
        objs.append(o)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Builds libkda.so (the gfx950 kernels and the C ABI of include/kda.h) in-tree
with hipcc. Every HIP source is compiled with packed-fp32 instructions turned
off (the compiler still vectorises ordinary float code, without them)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_prefill.hip", "kda_layer.hip", "kda_backward.hip"]
# measured device ceilings for the benchmark's roofline figures (include/kda_calib.h)
CALIB_LIB = os.path.join(PKG, "libkda_calib.so")
CALIB_SOURCES = ["kda_calib.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# -disable-promote-alloca-to-vector: register tiles held in small arrays
# (state slices, accumulators) stay separate registers; merged into one long
# vector they need contiguous register blocks and spill.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-disable-promote-alloca-to-vector",
         "-I", os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature flag: drop that warning
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        sys.stderr.write("\n".join(noise) + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return out


def _link(lib: str, objs, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles libkda.so and libkda_calib.so; returns the path of libkda.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link(LIB, [objs[s] for s in SOURCES], verbose)
    _link(CALIB_LIB, [objs[s] for s in CALIB_SOURCES], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libbiasact.so (gfx950) in-tree with hipcc.

    python conv_bias_activation_amd/build.py        # always recompiles

(Run it as a script: importing the package would first load the library.)

Every HIP translation unit is compiled for gfx950 only, with packed-fp32
instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops), in
parallel, then linked into conv_bias_activation_amd/libbiasact.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbiasact.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

_TYPES = ("f32", "f16", "bf16")
HIP_SOURCES = ["api.hip", "act_cast.hip", "dispatch.hip"] + [
    f"{op}_{ti}_{to}.hip" for op in ("gemm", "conv") for ti in _TYPES for to in _TYPES] + [
    f"gemm_i8_{to}.hip" for to in ("f32", "f16", "bf16", "i32")]
CPP_SOURCES = ["plan.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall",
          "-Wno-unused-command-line-argument"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; that warning is expected
    noise = "'-packed-fp32-ops' is not a recognized feature"
    warn = "\n".join(l for l in r.stderr.splitlines() if noise not in l and l.strip())
    return time.time() - t0, warn


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    steps = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append((src, [HIPCC, *COMMON, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append((src, ["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC,
                            "-c", os.path.join(CSRC, src), "-o", obj], obj))
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_run, cmd): (name, obj) for name, cmd, obj in steps}
        for f in cf.as_completed(futs):
            name, obj = futs[f]
            dt, warn = f.result()
            if verbose:
                print(f"  compiled {name} in {dt:.1f}s", flush=True)
            if warn and verbose:
                print(warn, flush=True)
            objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *sorted(objs)])
    os.replace(tmp, LIB)
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    t = time.time()
    out = build(verbose=True)
    print(f"built {out} in {time.time() - t:.1f}s")
    sys.exit(0)

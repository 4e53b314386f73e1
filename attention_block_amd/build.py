"""Build libdab.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m attention_block_amd.build

Compiles every time it is called.  The library lands next to this file as
attention_block_amd/libdab.so, where the Python binding looks for it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdab.so")

SOURCES = ["dab_api.hip", "dab_phase_bf16.hip", "dab_phase_f32.hip", "dab_ffn.hip", "dab_layer.hip", "dab_mla.hip",
           "dab_plan.cpp"]

# Packed fp32 instructions are kept out of the device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdab.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; drop that line
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 (in parallel), link libdab.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", *DEVICE_FLAGS,
              "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append(common + ["-c", os.path.join(CSRC, src), "-o", obj])
    workers = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(workers) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

"""Compile libmk.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m tile_synchronized_decoder_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
OBJDIR = os.path.join(HERE, "_build")
# (source, extra defines, object name); inst.hip is compiled once per element type x batch bucket
UNITS = [("queue.cpp", [], "queue.o"), ("api.hip", [], "api.o"), ("prefill.hip", [], "prefill.o")] + [
    ("inst.hip", [f"-DMK_WT={wt}", f"-DMK_WT_NAME={name}", f"-DMK_NB={nb}"], f"inst_{name}_{nb}.o")
    for wt, name in (("uint16_t", "bf16"), ("float", "f32")) for nb in (1, 2, 4, 8, 16, 32)]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out:
        print(out, flush=True)


def build(verbose: bool = True, jobs: int = 0) -> str:
    """Compile every unit (in parallel) and link libmk.so; always rebuilds."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cmds = [[hipcc, *HIPCC_FLAGS, *inc, *defs, "-c", os.path.join(CSRC, src), "-o", os.path.join(OBJDIR, obj)]
            for src, defs, obj in UNITS]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp,
          *[os.path.join(OBJDIR, obj) for _, _, obj in UNITS]], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

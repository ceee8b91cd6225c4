"""Build libqlora.so (gfx950) in-tree with hipcc.

python -m parameter_efficient_fine_amd.build   (or call build())
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqlora.so")
OBJDIR = os.path.join(HERE, "_build")
# (source, object, extra flags): the fused GEMMs are built once per weight
# format (QL_WFMT 0 NF4, 1 INT8, 2 FP8), each into its own namespace
SOURCES = [("quant.hip", "quant.o", []), ("skinny.hip", "skinny.o", []), ("normrope.hip", "normrope.o", []),
           ("small.hip", "small.o", []),
           ("lmhead.hip", "lmhead.o", []),
           ("api.cpp", "api.o", [])] + [
    (f"{g}.hip", f"{g}_f{fmt}.o", [f"-DQL_WFMT={fmt}"]) for g in ("gemm_bwd", "gemm_fwd") for fmt in (0, 1, 2)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# No fast-math: the quantizer needs IEEE division and fp32 denormals. Packed
# fp32 VALU ops are disabled (the compiler would otherwise emit them by itself).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-result",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(entry) -> str:
    src, objname, extra = entry
    obj = os.path.join(OBJDIR, objname)
    cmd = [HIPCC, *FLAGS, *extra, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    warn = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln and "(ignoring feature)" not in ln)
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()

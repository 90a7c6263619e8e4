"""Build libts_mha.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m sinks_ts_mha_amd.build          # or: python sinks_ts_mha_amd/build.py

Every HIP source is compiled with packed-FP32 instruction selection turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.  -fno-honor-nans lets the
backend drop the NaN-quieting of max operands (the kernels never produce NaN;
infinities, which they do use, are still honoured).  The per-kernel register and
LDS report of the device compiler is kept in _build/resource_usage.txt.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libts_mha.so")
SOURCES = ["prefill_fwd.hip", "prefill_fwd_narrow.hip", "decode_fwd.hip", "ts_mha_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    report = "\n".join(line for line in r.stderr.splitlines()
                       if "remark" in line or "kernel-resource-usage" in line)
    return obj, report


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for (_, rep), src in zip(results, SOURCES):
            f.write(f"== {src}\n{rep}\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

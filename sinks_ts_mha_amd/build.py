"""Build libts_mha.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m sinks_ts_mha_amd.build          # or: python sinks_ts_mha_amd/build.py

Every HIP source is compiled with packed-FP32 instruction selection turned off
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.  -ffp-contract=off keeps the
arithmetic the source writes: every fused multiply-add is an explicit fmaf, so the
two prefill kernels, which spell the same per-row arithmetic in differently shaped
code, cannot be fused differently by the compiler and give bitwise-equal results
(HIP's default would let it fuse a product into a later sum wherever it finds one).
-fno-honor-nans lets the
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
# the benchmark's microbenchmarks (vector-ALU and MFMA issue rates, device info):
# a library of their own, which only bench.py loads
UBENCH_LIB = os.path.join(PKG, "libts_ubench.so")
UBENCH_SOURCES = ["ubench.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-honor-nans", "-ffp-contract=off",
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


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    every = SOURCES + UBENCH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(every)) as ex:
        results = dict(zip(every, ex.map(_compile, every)))
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        for src in every:
            f.write(f"== {src}\n{results[src][1]}\n")
    _link([results[src][0] for src in SOURCES], LIB)
    _link([results[src][0] for src in UBENCH_SOURCES], UBENCH_LIB)
    if verbose:
        print(f"built {LIB} and {UBENCH_LIB}")
    return LIB


# Address and undefined-behaviour sanitizers for the host code only (hipcc applies
# each flag after -Xarch_host to the host compilation; device code is unchanged).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build_host_sanitized(out_dir: str) -> str:
    """libts_mha.so with the C ABI layer (ts_mha_api.hip: validation, error text, pair
    counts, launch set-up) compiled under the sanitizers; the kernels' objects are the
    regular ones.  The result needs clang's ASan runtime preloaded
    (asan_runtime()).  Returns the library's path."""
    os.makedirs(out_dir, exist_ok=True)
    kernels = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "ts_mha_api.hip"]
    if not all(os.path.exists(o) for o in kernels):
        build()
    api = os.path.join(out_dir, "ts_mha_api_san.o")
    cmd = [HIPCC, *FLAGS, *SANITIZE_HOST, "-c", os.path.join(CSRC, "ts_mha_api.hip"), "-o", api]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized ABI layer:\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(out_dir, "libts_mha_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *kernels, api, "-o", lib],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    return lib


def asan_runtime() -> str:
    """clang's shared ASan runtime (it carries the UBSan handlers too)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

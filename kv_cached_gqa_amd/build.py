"""Build libkvc.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m kv_cached_gqa_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled; the
objects go to kv_cached_gqa_amd/_build/ and the library to
kv_cached_gqa_amd/libkvc.so. KVC_BUILD_DEFINES (space-separated NAME=VALUE)
adds preprocessor definitions to every source (the timestamp probe of
kv_cached_gqa_amd.probe builds a copy of the package with one).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")
INCLUDE = os.path.join(ROOT, "include")

ARCH = "gfx950"
# the decode kernels compile per (head dimension, storage type), in parallel
DECODE_UNITS = [f"kvc_decode_d{d}_{t}.hip" for d in (128, 64, 32) for t in ("bf16", "f16", "f32")]
SOURCES = [*DECODE_UNITS, "kvc_prefill.hip", "kvc_append.hip", "kvc_decode.hip", "kvc_api.cpp", "kvc_latent.cpp"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
          *[f"-D{d}" for d in os.environ.get("KVC_BUILD_DEFINES", "").split()]]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvc)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *DEVICE, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

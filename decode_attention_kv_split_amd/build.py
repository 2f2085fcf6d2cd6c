"""Build libkvsplit.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Usage: python -m decode_attention_kv_split_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libkvsplit.so")
SOURCES = ["abi.cpp", "plan.cpp", "decode_mfma.hip", "rows_mfma.hip", "decode_valu.hip", "merge.hip", "append.hip",
           "probe.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # packed fp32 instructions stay off: ordinary fp32 math only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the softmax rescale and the
    # bf16 packing read them every tile, and AGPR placement cost ~130 extra
    # register moves per tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    hip_src = src.endswith(".hip")
    cmd = [_hipcc(), *FLAGS, "-c", src, "-o", obj]
    if not hip_src:
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    jobs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        for s in SOURCES:
            src = os.path.join(CSRC, s)
            obj = os.path.join(OUT_DIR, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            jobs.append(ex.submit(_compile, src, obj))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()

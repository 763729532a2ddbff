"""Build liblq.so (the HIP library behind include/lq.h) for gfx950, in-tree.

    python quantized_lora_fine_lq_amd/build.py

hipcc cross-compiles without a GPU. Flags: -O3, no floating-point contraction
(the codec kernels are bit-exact and spell out every fused multiply-add),
packed-FP32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(LIB_DIR, "liblq.so")
SOURCES = ["lq_tables.cpp", "lq_api.cpp", "lq_codec.hip", "lq_gemm.hip", "lq_lloyd.hip", "lq_lowrank.hip"]
ARCH = os.environ.get("LQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    objs = []
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    common = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function"]
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(obj_dir, src + ".o")
        if src.endswith(".hip"):
            cmd = [hipcc(), f"--offload-arch={ARCH}", "-x", "hip", *common,
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-c", path, "-o", obj]
        else:
            cmd = [hipcc(), *common, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in res.stderr.splitlines()
                         if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {src}\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed\n" + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

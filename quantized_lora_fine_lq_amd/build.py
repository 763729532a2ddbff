"""Build liblq.so (the HIP library behind include/lq.h) and its LQ_DEBUG
variant liblq_debug.so for gfx950, in-tree.

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
LIB_DEBUG = os.path.join(LIB_DIR, "liblq_debug.so")
SOURCES = ["lq_tables.cpp", "lq_api.cpp", "lq_codec.hip", "lq_gemm.hip", "lq_lloyd.hip", "lq_lowrank.hip",
           "lq_noalloc.hip"]
ARCH = os.environ.get("LQ_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str, defines: list, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    common = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function", *defines]
    if src.endswith(".hip"):
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-x", "hip", *common,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *common, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    return obj


def _link(objs: list, lib: str) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed\n" + res.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile the release library (liblq.so) and, unless debug=False, the
    LQ_DEBUG variant (liblq_debug.so: device flag word for precondition
    violations, host checks of codebook layouts, launch-shape asserts)."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(LIB_DIR, exist_ok=True)
    variants = [("release", [], LIB)]
    if debug:
        variants.append(("debug", ["-DLQ_DEBUG=1"], LIB_DEBUG))
    jobs = []
    for name, defs, _ in variants:
        obj_dir = os.path.join(HERE, "_build", name)
        os.makedirs(obj_dir, exist_ok=True)
        for src in SOURCES:
            jobs.append((name, src, os.path.join(obj_dir, src + ".o"), defs))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [(name, ex.submit(_compile, src, obj, defs, verbose)) for name, src, obj, defs in jobs]
        objs = {}
        for name, f in futs:
            objs.setdefault(name, []).append(f.result())
    for name, _, lib in variants:
        _link(objs[name], lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

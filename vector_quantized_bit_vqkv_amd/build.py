"""Build libvqkv.so (HIP, gfx950) in-tree.

Usage: python -m vector_quantized_bit_vqkv_amd.build
Each .hip/.cpp source under csrc/ is compiled to an object with hipcc for
gfx950, then linked into vector_quantized_bit_vqkv_amd/libvqkv.so.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libvqkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Keep the compiler from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]
# Files whose floating point decides integers (codes, K-Means assignments):
# no fused multiply-add anywhere.
PER_FILE = {"quantize.hip": ["-ffp-contract=off"]}
SOURCES = ["capi.cpp", "transform_query.hip", "quantize.hip", "decode.hip", "baseline.hip", "static_scratch.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name and says so; that is harmless.
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("command failed: " + " ".join(cmd))
    return out


def build(verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        return obj, _run([HIPCC, *COMMON, *PER_FILE.get(src, []), *lang, "-c", path, "-o", obj])
    # The sources compile independently (a few at a time: each hipcc is one process).
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), max(1, (os.cpu_count() or 1) // 2))) as pool:
        results = list(pool.map(compile_one, SOURCES))
    objs = []
    for obj, out in results:
        if verbose and out:
            print(out)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

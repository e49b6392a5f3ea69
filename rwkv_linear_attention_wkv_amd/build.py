"""Build libwkv.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m rwkv_linear_attention_wkv_amd.build [--jobs N]

Each source is compiled by hipcc to an object under ``lib/obj`` and the
objects are linked into ``lib/libwkv.so``.  Packed-FP32 instruction
selection is disabled for every device compile (the target feature
``-packed-fp32-ops``).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libwkv.so")
SOURCES = ["wkv_api.cpp", "wkv4_scan.hip", "wkv56_scan.hip", "wkv6_decode.hip", "wkv6_backward.hip", "wkv6_backward_chunked.hip", "wkv56_chunked.hip", "wkv6_chunked_save.hip",
           "wkv7_scan.hip", "wkv7_chunked.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libwkv.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def compile_one(src, objdir):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build(jobs=None, verbose=False):
    objdir = os.path.join(LIBDIR, "obj")
    os.makedirs(objdir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: compile_one(s, objdir), SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                sys.stderr.write(err)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()

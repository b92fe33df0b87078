"""Builds libfused_proj.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Each translation unit is compiled to an object of its own, in parallel, and the objects are
linked into the library. The fast kernel's file is compiled once per part (FP_FAST_PART),
each part holding a share of its instantiations.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfused_proj.so")
OBJDIR = os.path.join(PKG, "_build")
FAST_PARTS = 5
SOURCES = [os.path.join(CSRC, "fused_proj_api.cpp"), os.path.join(CSRC, "fused_proj_kernels.hip"),
           os.path.join(CSRC, "fused_proj_fast.hip"), os.path.join(CSRC, "split_rope.hip"),
           os.path.join(CSRC, "fused_proj_bwd.hip"), os.path.join(CSRC, "mfma_ceiling.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 arithmetic stays off (the host pass ignores this feature with a warning)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def units():
    """(source, extra flags, object) for every translation unit."""
    out = []
    for src in SOURCES:
        stem = os.path.splitext(os.path.basename(src))[0]
        if stem == "fused_proj_fast":
            for k in range(FAST_PARTS):
                out.append((src, [f"-DFP_FAST_PART={k}"], os.path.join(OBJDIR, f"{stem}.part{k}.o")))
        else:
            out.append((src, [], os.path.join(OBJDIR, stem + ".o")))
    return out


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    return r.returncode, msgs


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    cflags = [f for f in FLAGS if f != "-shared"]
    jobs = [[HIPCC, *cflags, *extra, "-x", "hip", "-c", src, "-o", obj] for src, extra, obj in units()]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1), 16))
    if verbose:
        for cmd in jobs:
            print(" ".join(cmd), flush=True)
    # the longest units first
    order = sorted(range(len(jobs)), key=lambda i: "fused_proj_fast" not in jobs[i][-3])
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = dict(zip(order, ex.map(lambda i: _run(jobs[i]), order)))
    failed = [(jobs[i], results[i][1]) for i in range(len(jobs)) if results[i][0] != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(" ".join(c) + "\n" + "\n".join(m) for c, m in failed))
    if verbose:
        for i in range(len(jobs)):
            if results[i][1]:
                print("\n".join(results[i][1]), file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, _, o in units()], "-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Builds librtopk.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m beam_search_top_amd._build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librtopk.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 in the device code.
# -fno-honor-nans: NaN logits are outside the contract, so
# min/max need no NaN-quieting canonicalisation (infinities stay honoured).
# Atomic optimizer off: it rewrites the few-lane LDS maxima of the threshold
# pool into a scalar loop over the active lanes, slower than the single
# ds_max the hardware serialises by itself.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
    "-fno-honor-nans", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
KERNELS = os.path.join(CSRC, "rtopk_kernels.hip")
HOST = os.path.join(CSRC, "rtopk_host.cpp")
REORDER = os.path.join(CSRC, "rtopk_reorder.hip")
SAMPLE = os.path.join(CSRC, "rtopk_sample.hip")
NOALLOC = os.path.join(CSRC, "rtopk_noalloc.hip")
DTYPES = (0, 1, 2)  # the kernel source is compiled once per logit type, in parallel


def _run(cmds, verbose):
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = False
    for p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed to build librtopk.so")


def build(verbose: bool = False, extra=()) -> str:
    tag = f".tmp{os.getpid()}"
    objs = [LIB + f".dt{d}{tag}.o" for d in DTYPES] + [LIB + f".noalloc{tag}.o", LIB + f".sample{tag}.o",
                                                       LIB + f".reorder{tag}.o", LIB + f".host{tag}.o"]
    cmds = [[HIPCC, *FLAGS, *extra, f"-DRTOPK_DTYPE={d}", "-c", KERNELS, "-o", o] for d, o in zip(DTYPES, objs)]
    cmds.append([HIPCC, *FLAGS, *extra, "-c", NOALLOC, "-o", objs[-4]])
    cmds.append([HIPCC, *FLAGS, *extra, "-c", SAMPLE, "-o", objs[-3]])
    cmds.append([HIPCC, *FLAGS, *extra, "-c", REORDER, "-o", objs[-2]])
    cmds.append([HIPCC, *FLAGS, *extra, "-c", HOST, "-o", objs[-1]])
    tmp = LIB + tag
    try:
        _run(cmds, verbose)
        _run([[HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs + [tmp]:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

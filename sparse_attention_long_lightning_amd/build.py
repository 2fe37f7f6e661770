"""Builds ``libdsa.so`` (the C-ABI DSA library, HIP kernels for gfx950) and ``libpeak.so`` (the
device peak probes the benchmark divides by) in-tree with hipcc.

Usage: ``python -m sparse_attention_long_lightning_amd.build`` (also run by the repository's
``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdsa.so")
PEAK_LIB = os.path.join(HERE, "libpeak.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "mqa.hip", "cache.hip", "kl.hip", "check.hip"]
ARCH = "gfx950"

# Packed fp32 arithmetic is disabled for every HIP translation unit (hipcc otherwise forms
# v_pk_* fp32 instructions from plain float code).
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass reports the device-only feature flag as unknown; drop that noise
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = ["hipcc", *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd += ["-save-temps=obj"]
        cmds.append(cmd)
    with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    # --no-undefined: a kernel whose host stub was not emitted fails here, not at load time
    _run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # the peak probes the benchmark divides by (not part of the attention path)
    tmp = PEAK_LIB + ".tmp"
    _run(["hipcc", *HIP_FLAGS, "-shared", "-o", tmp, os.path.join(CSRC, "peak.hip")])
    os.replace(tmp, PEAK_LIB)
    if verbose:
        print("built", LIB, "and", PEAK_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)

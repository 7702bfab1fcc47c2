"""Compile the HIP library libspecverify.so for gfx950 in-tree.

Each source is compiled to an object under ``_build/`` (in parallel), then
linked into ``verify_pass_rejection_amd/libspecverify.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["attention.hip", "accept_chain.hip", "accept_tree.hip", "accept_tree_sampled.hip",
           "commit.hip", "ngram.hip", "spec_verify.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # never emit packed fp32 arithmetic
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # MFMA accumulators in ordinary VGPRs (no AGPR copies around the
          # online-softmax rescale)
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


# Per-file additions.  The attention kernels never produce or consume NaN
# (masked scores are -inf and every guard compares before subtracting), so
# max/min need no NaN-quieting of lane-swapped operands.
FILE_FLAGS = {"attention.hip": ["-fno-honor-nans"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if warn:
        print(warn, file=sys.stderr)
    return obj


def build_library(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library()

"""Builds libssverify.so (HIP, gfx950) in-tree, next to this file.

    python -m long_context_speculative_amd.build

Every call recompiles. Objects go to _build/ at the repository root; the
shared library lands in the package directory, where the binding loads it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssverify.so")

SOURCES = ["ss_api.hip", "ss_valu.hip", "ss_mfma.hip", "ss_region.hip", "ss_mfma_wide.hip", "ss_valu_small.hip",
           "ss_sparse.hip", "ss_probe.hip"]

# Packed-fp32 instructions are switched off for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC]


# Per-file extra flags. The wide-row kernel's row maxima run over MFMA
# results that are never NaN; without NaN semantics every fmaxf drops the
# quieting max it otherwise needs per input (20 fewer VALU per key tile).
# The file holds no NaN-dependent host logic (only its launcher).
FILE_FLAGS = {"ss_mfma_wide.hip": ["-fno-honor-nans"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIP_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    outs.append(_run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

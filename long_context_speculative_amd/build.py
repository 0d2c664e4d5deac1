"""Builds libssverify.so (HIP, gfx950) in-tree, next to this file.

    python -m long_context_speculative_amd.build [--asan]

Every call recompiles. --asan builds the host-sanitizer variant into
_build/asan/ (for the CPU tests; see ASAN_FLAGS). Objects go to _build/ at the repository root; the
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

SOURCES = ["ss_api.hip", "ss_valu.hip", "ss_mfma.hip", "ss_mfma_f32.hip", "ss_region.hip", "ss_mfma_wide.hip",
           "ss_valu_small.hip", "ss_sparse.hip", "ss_probe.hip"]

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


# Host AddressSanitizer build: the host side of every file (argument
# validation, plans, tree masks, copy address arithmetic, the streaming
# bookkeeping) instrumented, device code built as usual. The flags apply to
# the host compilation only. Loaded through SS_VERIFY_LIB with the ASan
# runtime preloaded (see asan_runtime()).
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libssverify.so")


def asan_runtime() -> str:
    """Path of the compiler's ASan runtime (to LD_PRELOAD into Python)."""
    return _run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"]).strip()


def build(verbose: bool = False, asan: bool = False) -> str:
    out_dir = ASAN_DIR if asan else BUILD
    lib = ASAN_LIB if asan else LIB
    extra = ASAN_FLAGS if asan else []
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIP_FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        outs = list(ex.map(_run, cmds))
    tmp = lib + ".tmp"
    outs.append(_run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp]))
    os.replace(tmp, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv))

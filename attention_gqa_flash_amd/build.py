"""Build libsinkattn.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m attention_gqa_flash_amd.build

Compiles every source under csrc/ with hipcc and links the shared library
next to this file.  Always rebuilds.
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
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsinkattn.so")
SOURCES = ["prefill.hip", "decode.hip", "rope.hip", "oproj.hip", "checks.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the HIP library")
    return path


def common_flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fno-honor-nans", "-fPIC", "--offload-arch=" + ARCH,
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        # keep the compiler from forming packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), msgs))
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (" ".join(cmd), proc.stdout + proc.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()

"""Builds libpagedkv.so in-tree for gfx950 with hipcc.

    python -m paged_kv_cache_408_amd._build

Every HIP translation unit is compiled with packed-FP32 instruction selection switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass warns that it
does not know that feature, which is harmless.  The allocator and error units are plain
C++ compiled by the same driver.  Objects are cached by content hash under ``_build/``.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagedkv.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]
SOURCES = ["pagedkv.hip", "prefill.hip", "probe.hip", "allocator.cpp", "pa_error.cpp", "tensor_api.cpp"]
HEADERS = ["pa_error.h", "pa_device.h", "pa_layout.h"]


def _digest(src: str, flags) -> str:
    h = hashlib.sha256()
    for p in [os.path.join(CSRC, src)] + [os.path.join(CSRC, x) for x in HEADERS] + [os.path.join(INCLUDE, "pagedkv.h")]:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def _compile(src: str, verbose: bool) -> str:
    is_hip = src.endswith(".hip")
    flags = COMMON + (HIP_FLAGS if is_hip else ["-x", "c++"])
    obj = os.path.join(OBJDIR, f"{os.path.splitext(src)[0]}-{_digest(src, flags)}.o")
    if os.path.exists(obj):
        return obj
    cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(obj + ".tmp", obj)
    return obj


def build(verbose: bool = True, force: bool = False) -> str:
    """Compile (or reuse cached objects) and link libpagedkv.so; returns its path."""
    if force and os.path.isdir(OBJDIR):
        shutil.rmtree(OBJDIR)
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, force="--force" in sys.argv)

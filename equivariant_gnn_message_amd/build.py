"""Build libe3conv.so in-tree with hipcc for gfx950.

Usage: ``python -m equivariant_gnn_message_amd.build`` (or ``build()``).
Sources are compiled to objects under ``_build/`` in parallel, then linked
into ``equivariant_gnn_message_amd/libe3conv.so``.
"""

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
LIB = os.path.join(PKG, "libe3conv.so")

SOURCES = ["host_core.cpp", "e3conv.cpp", "kernels.hip", "validate.hip", "layout_tiny.hip",
           "layout_gate.hip", "layout_mace.hip", "layout_big.hip", "linear.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]
# Device code: gfx950 only; packed FP32 instructions are kept out of the code
# object; fp32 atomics map to the hardware instruction.
DEVICE = ["--offload-arch=gfx950", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, flush=True)
    return obj


def _stale(src):
    """True if the object of src is missing or older than any source or header."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".h", ".hip", ".cpp"))
            and (f == src or f.endswith(".h"))]
    deps.append(os.path.join(INCLUDE, "e3conv.h"))
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose=False, incremental=False):
    """Compile every source (or, with incremental=True, only those whose object is
    older than the source or any header) and link libe3conv.so."""
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if not incremental or _stale(s)]
    with ThreadPoolExecutor(max(1, len(todo))) as ex:
        list(ex.map(lambda s: _compile(s, verbose), todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))

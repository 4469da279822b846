"""Build and load the read-ceiling probes of bench_ceiling.hip (measurement code
for bench.py, not part of the q3 library).

    python bench_ceiling.py        # builds libbench_ceiling.so beside this file
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(ROOT, "bench_ceiling.hip")
LIB = os.path.join(ROOT, "libbench_ceiling.so")

_lib = None


def build() -> str:
    hipcc = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
                  if c and os.path.exists(c)), None)
    if hipcc is None:
        raise RuntimeError("hipcc not found: the read-ceiling probe needs ROCm's hipcc to build")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-O3", "-fPIC", "-shared", "-std=c++17", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(f"{LIB} is missing: build it with `python bench_ceiling.py` "
                              "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB)
        L.ceiling_read.restype = ctypes.c_int
        L.ceiling_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
        L.ceiling_empty.restype = ctypes.c_int
        L.ceiling_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
        _lib = L
    return _lib


def read(buf, blocks: int, unroll: int, sink, stream) -> None:
    """One streaming read of the whole uint8 device tensor `buf`."""
    e = lib().ceiling_read(buf.data_ptr(), buf.numel(), blocks, unroll, sink.data_ptr(), stream)
    if e != 0:
        raise RuntimeError(f"ceiling_read failed with hipError {e}")


def empty(blocks: int, stream) -> None:
    e = lib().ceiling_empty(blocks, stream)
    if e != 0:
        raise RuntimeError(f"ceiling_empty failed with hipError {e}")


if __name__ == "__main__":
    print(build())

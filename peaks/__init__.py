"""Measured-peak kernels (HBM streaming read, FP4 and bf16 MFMA loops, an
empty kernel for the launch floor, a VALU loop for the per-wave issue rate) -
MEASUREMENT INFRASTRUCTURE ONLY: bench.py loads it to report every roofline
fraction against this part's sustained rates as well as the datasheet's.
The product library (long_context_compressed_05_amd) does not use it."""
from __future__ import annotations

import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libpeaks.so")
_lib = None

FLOP_FP4_MFMA = 2 * 32 * 32 * 64
FLOP_BF16_BIG = 2 * 32 * 32 * 16
FLOP_BF16_SMALL = 2 * 16 * 16 * 32


def build(verbose: bool = False) -> str:
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(_HERE, "peaks.hip"), "-o", _SO + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for peaks.hip:\n{r.stderr}")
    os.replace(_SO + ".tmp", _SO)
    return _SO


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        raise RuntimeError(f"{_SO} not built (python -c 'import peaks; peaks.build()')")
    L = ctypes.CDLL(_SO)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.peak_read.argtypes = [vp, sz, ci, ci, vp, vp, vp, vp]
    L.peak_read_chunked.argtypes = [vp, sz, ci, ci, vp, vp, vp, vp]
    L.peak_mfma_fp4.argtypes = [ci, ci, vp, vp, vp, vp]
    L.peak_mfma_bf16.argtypes = [ci, ci, ci, vp, vp, vp, vp]
    L.peak_empty.argtypes = [ci, ci, vp, vp, vp, vp]
    L.peak_valu.argtypes = [ci, ci, ci, vp, vp, vp, vp]
    for f in (L.peak_read, L.peak_read_chunked, L.peak_mfma_fp4, L.peak_mfma_bf16, L.peak_empty, L.peak_valu):
        f.restype = ci
    _lib = L
    return L

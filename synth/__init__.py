"""Seeded synthetic inputs for the compressed-attention workloads.

This module draws and formats random inputs only; it contains none of the
method's arithmetic (no pooling, scoring, selection or attention).  Both the
HIP path and the CPU oracle are fed from the arrays it returns.

Workload shapes follow the five synthetic configurations of the hot path:
single-sequence fp32 decode at T=4096, batched bf16 decode at T=64K, a 4096-
token prefill chunk on a 64K cache, 1M-token decode, and a ragged tie-heavy
batch.  There is no dataset behind any of them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream ids, one per generated tensor
S_KV, S_Z, S_Q, S_QCODE, S_QSCALE, S_W, S_KCODE, S_KSCALE, S_LEN, S_POOL = range(1, 11)

E2M1_ALL_CODES = tuple(range(16))
E2M1_TIE_CODES = (0x0, 0x1, 0x9)  # values 0, +0.5, -0.5


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           os.path.join(_HERE, "synth.c"), "-o", _SO + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    u64, i64, vp, ci, cd = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.synth_raw_draw.restype = u64
    lib.synth_raw_draw.argtypes = [u64, u64, u64]
    lib.synth_normal_one.restype = cd
    lib.synth_normal_one.argtypes = [u64, u64, u64]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, u64, vp, ci]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, u64, vp, ci]
    lib.synth_codes4.argtypes = [u64, u64, u64, u64, vp, ci, vp, ci]
    lib.synth_exp_bytes.argtypes = [u64, u64, u64, u64, ci, ci, ci, vp, ci]
    lib.synth_pow2_f32.argtypes = [u64, u64, u64, u64, ci, ci, vp, ci]
    lib.synth_loguniform_lengths.argtypes = [u64, u64, i64, cd, cd, i64, vp]
    _lib = lib
    return lib


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed: int, stream: int, n: int, dtype: str, off: int = 0) -> np.ndarray:
    """n standard normals (fp32 array, or bf16 bit patterns as uint16)."""
    lib = _load()
    if dtype == "f32":
        out = np.empty(n, dtype=np.float32)
        lib.synth_normal_f32(seed, stream, off, n, out.ctypes.data, _threads())
    elif dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        lib.synth_normal_bf16(seed, stream, off, n, out.ctypes.data, _threads())
    else:
        raise ValueError(dtype)
    return out


def codes4(seed: int, stream: int, n_bytes: int, codeset: Sequence[int], off: int = 0) -> np.ndarray:
    lib = _load()
    cs = np.asarray(codeset, dtype=np.uint8)
    out = np.empty(n_bytes, dtype=np.uint8)
    lib.synth_codes4(seed, stream, off, n_bytes, cs.ctypes.data, len(cs), out.ctypes.data, _threads())
    return out


def exp_bytes(seed: int, stream: int, n: int, lo: int, hi: int, bias: int = 127, off: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.uint8)
    lib.synth_exp_bytes(seed, stream, off, n, lo, hi, bias, out.ctypes.data, _threads())
    return out


def pow2(seed: int, stream: int, n: int, lo: int, hi: int, off: int = 0) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.float32)
    lib.synth_pow2_f32(seed, stream, off, n, lo, hi, out.ctypes.data, _threads())
    return out


def loguniform_lengths(seed: int, n: int, lo: float, hi: float, forbid_mod: int) -> np.ndarray:
    lib = _load()
    out = np.empty(n, dtype=np.int64)
    lib.synth_loguniform_lengths(seed, S_LEN, n, lo, hi, forbid_mod, out.ctypes.data)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (format plumbing only)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    name: str
    lengths: List[int]            # raw tokens per sequence (cache + any new chunk)
    q_start: List[int]            # first query position per sequence
    H: int = 64
    d: int = 128
    dtype: str = "bf16"
    m: int = 4
    k: int = 512
    W: int = 128
    m_hca: int = 128
    W_hca: int = 0
    H_I: int = 4
    d_I: int = 64
    codeset: Sequence[int] = E2M1_ALL_CODES
    scale_exp: tuple = (-2, 2)
    w_exp: tuple = (-1, 1)
    seed: int = 1001

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def n_q_per_seq(self) -> List[int]:
        return [L - s for L, s in zip(self.lengths, self.q_start)]

    @property
    def n_q(self) -> int:
        return sum(self.n_q_per_seq)

    def pooled(self, m: int) -> List[int]:
        return [L // m for L in self.lengths]

    def describe(self) -> Dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "d": self.d, "dtype": self.dtype,
                "m": self.m, "top_k": self.k, "W": self.W, "m_hca": self.m_hca,
                "max_len": max(self.lengths), "n_q": self.n_q}


def decode_t4096_fp32(seed: int = 1001) -> Workload:
    return Workload("decode_t4096_fp32", [4096], [4095], H=8, dtype="f32", k=64, seed=seed)


def decode_b16_t64k(seed: int = 1002) -> Workload:
    return Workload("decode_b16_t64k", [65536] * 16, [65535] * 16, k=512, seed=seed)


def prefill_4k_on_64k(seed: int = 1003) -> Workload:
    return Workload("prefill_4k_on_64k", [65536 + 4096], [65536], k=512, seed=seed)


def decode_b4_t1m(seed: int = 1004) -> Workload:
    return Workload("decode_b4_t1m", [1 << 20] * 4, [(1 << 20) - 1] * 4, k=1024, seed=seed)


def decode_ragged_b32(seed: int = 1005, n: int = 32, lo: int = 4096, hi: int = 1 << 20) -> Workload:
    lens = [int(x) for x in loguniform_lengths(seed, n, lo, hi, 4)]
    return Workload("decode_ragged_b32", lens, [L - 1 for L in lens], k=512,
                    codeset=E2M1_TIE_CODES, seed=seed)


WORKLOADS = {
    "decode_t4096_fp32": decode_t4096_fp32,
    "decode_b16_t64k": decode_b16_t64k,
    "prefill_4k_on_64k": prefill_4k_on_64k,
    "decode_b4_t1m": decode_b4_t1m,
    "decode_ragged_b32": decode_ragged_b32,
}


def offsets(sizes: Sequence[int]) -> np.ndarray:
    o = np.zeros(len(sizes) + 1, dtype=np.int64)
    o[1:] = np.cumsum(np.asarray(sizes, dtype=np.int64))
    return o


def q_positions(wl: Workload) -> np.ndarray:
    return np.concatenate([np.arange(s, L, dtype=np.int64) for L, s in zip(wl.lengths, wl.q_start)])


def make_inputs(wl: Workload, raw: bool = True) -> Dict[str, np.ndarray]:
    """All host inputs of one workload.

    kv   [sum L][2][d]  raw K|V rows (fp32, or bf16 bits as uint16)
    z    [sum L][2][d]  pooling logits for the K and V channels, same dtype
    q    [n_q][H][d]    attention queries
    qc   [n_q][H_I][d_I/2]  packed e2m1 indexer query codes (low nibble = even element)
    qs   [n_q][H_I][d_I/32] E8M0 indexer query block scales
    w    [n_q][H_I]     power-of-two indexer head weights (fp32)
    kc   [sum P][d_I/2] packed e2m1 indexer key codes, one key per CSA pooled entry
    ks   [sum P][d_I/32] E8M0 indexer key block scales
    plus the offset arrays tok_off, q_off, q_pos, pool_off (m), hpool_off (m_hca).
    """
    s = wl.seed
    L = wl.lengths
    C = 2 * wl.d
    n_tok = int(sum(L))
    P = wl.pooled(wl.m)
    n_pool = int(sum(P))
    n_q = wl.n_q
    out: Dict[str, np.ndarray] = {}
    if raw:
        out["kv"] = normal(s, S_KV, n_tok * C, wl.dtype).reshape(n_tok, 2, wl.d)
        out["z"] = normal(s, S_Z, n_tok * C, wl.dtype).reshape(n_tok, 2, wl.d)
    out["q"] = normal(s, S_Q, n_q * wl.H * wl.d, wl.dtype).reshape(n_q, wl.H, wl.d)
    out["qc"] = codes4(s, S_QCODE, n_q * wl.H_I * wl.d_I // 2, wl.codeset).reshape(n_q, wl.H_I, wl.d_I // 2)
    out["qs"] = exp_bytes(s, S_QSCALE, n_q * wl.H_I * wl.d_I // 32, *wl.scale_exp).reshape(n_q, wl.H_I, wl.d_I // 32)
    out["w"] = pow2(s, S_W, n_q * wl.H_I, *wl.w_exp).reshape(n_q, wl.H_I)
    out["kc"] = codes4(s, S_KCODE, n_pool * wl.d_I // 2, wl.codeset).reshape(n_pool, wl.d_I // 2)
    out["ks"] = exp_bytes(s, S_KSCALE, n_pool * wl.d_I // 32, *wl.scale_exp).reshape(n_pool, wl.d_I // 32)
    out["tok_off"] = offsets(L)
    out["q_off"] = offsets(wl.n_q_per_seq)
    out["q_pos"] = q_positions(wl)
    out["pool_off"] = offsets(P)
    out["hpool_off"] = offsets(wl.pooled(wl.m_hca))
    return out


def pooled_like(wl: Workload, m: int, stream: int = S_POOL) -> np.ndarray:
    """A stand-alone pooled cache [sum P][2][d] of N(0,1) rows, for stage-wise
    attention checks that must not depend on any pooling implementation."""
    P = int(sum(wl.pooled(m)))
    return normal(wl.seed, stream + 100 * m, P * 2 * wl.d, wl.dtype).reshape(P, 2, wl.d)

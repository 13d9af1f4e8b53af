"""CPU oracle for CSA / HCA — TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps ``oracle.cpp`` (plain C++, fp64 plus an exact
indexer) through ctypes and shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", os.path.join(_HERE, "oracle.cpp"),
           "-o", _SO + ".tmp"]
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
    vp, ci, i64, cd = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_e2m1_value.restype = cd
    lib.orc_e2m1_value.argtypes = [ci]
    lib.orc_e8m0_value.restype = cd
    lib.orc_e8m0_value.argtypes = [ci]
    lib.orc_pool.argtypes = [ci, i64, ci, ci, vp, vp, vp]
    lib.orc_mxfp4_quantize.argtypes = [i64, ci, ci, vp, vp, vp]
    lib.orc_index_scores.argtypes = [i64, ci, ci, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_topk.argtypes = [i64, vp, ci, vp]
    lib.orc_index_scores_bf16.argtypes = [i64, ci, ci, vp, vp, vp, vp]
    lib.orc_attend.argtypes = [ci, ci, cd, vp, i64, vp, vp, vp, vp]
    lib.orc_csa_query.argtypes = [ci, ci, ci, ci, ci, ci, cd, i64, vp, vp, vp, vp,
                                  ci, ci, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.orc_hca_query.argtypes = [ci, ci, ci, ci, ci, cd, i64, vp, vp, vp, vp, vp, vp]
    lib.orc_csa_attend_given.argtypes = [ci, ci, ci, ci, cd, i64, vp, vp, vp, ci, vp, vp, vp]
    lib.orc_hca_attend_given.argtypes = [ci, ci, ci, ci, ci, cd, i64, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"KV dtype must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _check(rc: int, what: str):
    if rc == -2:
        raise AssertionError(f"oracle {what}: the two exact indexer routes disagree")
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(code)


def e8m0_value(byte: int) -> float:
    return _load().orc_e8m0_value(byte)


def mxfp4_quantize(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Rows of x ([..., dim] fp32, or bf16 bit patterns as uint16) -> MXFP4
    (codes [..., dim/2] uint8, E8M0 scales [..., dim/32] uint8)."""
    x = np.ascontiguousarray(x)
    dim = x.shape[-1]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    codes = np.zeros(x.shape[:-1] + (dim // 2,), dtype=np.uint8)
    scales = np.zeros(x.shape[:-1] + (dim // 32,), dtype=np.uint8)
    _check(_load().orc_mxfp4_quantize(rows, dim, _dt(x), _p(x), _p(codes), _p(scales)), "mxfp4_quantize")
    return codes, scales


def pool(x: np.ndarray, z: np.ndarray, m: int) -> np.ndarray:
    """x, z: [rows][C] (or [rows][2][d]) -> fp64 [rows//m][C]."""
    x2 = np.ascontiguousarray(x.reshape(x.shape[0], -1))
    z2 = np.ascontiguousarray(z.reshape(z.shape[0], -1))
    assert x2.shape == z2.shape and x2.dtype == z2.dtype
    n, C = x2.shape
    out = np.empty((n // m, C), dtype=np.float64)
    _check(_load().orc_pool(_dt(x2), n, C, m, _p(x2), _p(z2), _p(out)), "pool")
    return out


def index_scores(qc, qs, w, kc, ks) -> Tuple[np.ndarray, np.ndarray]:
    """Exact scores of keys kc/ks [n][d_I/2],[n][d_I/32] for one query
    qc [H_I][d_I/2], qs [H_I][d_I/32], w [H_I].  Returns (S fp64, fp32-exact flags)."""
    qc, qs = np.ascontiguousarray(qc, np.uint8), np.ascontiguousarray(qs, np.uint8)
    w = np.ascontiguousarray(w, np.float32)
    kc, ks = np.ascontiguousarray(kc, np.uint8), np.ascontiguousarray(ks, np.uint8)
    H_I, half = qc.shape
    n = kc.shape[0]
    S = np.empty(n, dtype=np.float64)
    ex = np.empty(n, dtype=np.int32)
    _check(_load().orc_index_scores(n, H_I, 2 * half, _p(qc), _p(qs), _p(w), _p(kc), _p(ks), _p(S), _p(ex)),
           "index_scores")
    return S, ex.astype(bool)


def index_scores_bf16(q, w, keys) -> np.ndarray:
    """Scores of keys [n][d_I] (bf16 bit patterns, uint16) for one query
    q [H_I][d_I] (bf16 bits) with head weights w [H_I]: fp64, exact products."""
    q = np.ascontiguousarray(q, np.uint16)
    keys = np.ascontiguousarray(keys, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    H_I, d_I = q.shape
    S = np.empty(keys.shape[0], dtype=np.float64)
    _check(_load().orc_index_scores_bf16(keys.shape[0], H_I, d_I, _p(q), _p(w), _p(keys), _p(S)), "index_scores_bf16")
    return S


def topk(S: np.ndarray, k: int) -> np.ndarray:
    S = np.ascontiguousarray(S, np.float64)
    idx = np.empty(k, dtype=np.int32)
    _check(_load().orc_topk(S.shape[0], _p(S), k, _p(idx)), "topk")
    return idx


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """q [H][d], keys/vals [n][d] (fp64) -> out [H][d], lse [H]."""
    q = np.ascontiguousarray(q, np.float64)
    keys = np.ascontiguousarray(keys, np.float64).reshape(-1, q.shape[1])
    vals = np.ascontiguousarray(vals, np.float64).reshape(-1, q.shape[1])
    H, d = q.shape
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    _check(_load().orc_attend(H, d, scale, _p(q), keys.shape[0], _p(keys), _p(vals), _p(out), _p(lse)), "attend")
    return out, lse


def csa_query(kv, z, q, t, m, W, k, scale, qc, qs, w, kc, ks, pooled=None):
    """End-to-end CSA for one query at position t of one sequence.
    kv, z: the sequence's raw rows [L][2][d]; q [H][d]; indexer inputs for the
    query (qc, qs, w) and the sequence's keys (kc, ks).  Returns (out, lse, idx)."""
    kv = np.ascontiguousarray(kv)
    z = np.ascontiguousarray(z)
    q = np.ascontiguousarray(q)
    H, d = q.shape
    qc, qs = np.ascontiguousarray(qc, np.uint8), np.ascontiguousarray(qs, np.uint8)
    w = np.ascontiguousarray(w, np.float32)
    kc, ks = np.ascontiguousarray(kc, np.uint8), np.ascontiguousarray(ks, np.uint8)
    if pooled is not None:
        pooled = np.ascontiguousarray(pooled, np.float64)
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    idx = np.empty(k, dtype=np.int32)
    H_I, half = qc.shape
    _check(_load().orc_csa_query(_dt(kv), d, H, m, W, k, scale, t, _p(kv), _p(z), _p(pooled), _p(q),
                                 H_I, 2 * half, _p(qc), _p(qs), _p(w), _p(kc), _p(ks),
                                 _p(out), _p(lse), _p(idx)), "csa_query")
    return out, lse, idx


def hca_query(kv, z, q, t, m_h, W_h, scale, hpooled=None):
    kv = np.ascontiguousarray(kv)
    z = np.ascontiguousarray(z)
    q = np.ascontiguousarray(q)
    H, d = q.shape
    if hpooled is not None:
        hpooled = np.ascontiguousarray(hpooled, np.float64)
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    _check(_load().orc_hca_query(_dt(kv), d, H, m_h, W_h, scale, t, _p(kv), _p(z), _p(hpooled), _p(q),
                                 _p(out), _p(lse)), "hca_query")
    return out, lse


def csa_attend_given(kv, pooled, idx, q, t, W, scale):
    """Stage-wise CSA attention: given pooled cache [P][2][d] (KV dtype) and idx [k]."""
    kv, pooled, q = np.ascontiguousarray(kv), np.ascontiguousarray(pooled), np.ascontiguousarray(q)
    assert kv.dtype == pooled.dtype == q.dtype
    idx = np.ascontiguousarray(idx, np.int32)
    H, d = q.shape
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    _check(_load().orc_csa_attend_given(_dt(kv), d, H, W, scale, t, _p(kv), _p(pooled), _p(idx), idx.shape[0],
                                        _p(q), _p(out), _p(lse)), "csa_attend_given")
    return out, lse


def hca_attend_given(kv, hpooled, q, t, m_h, W_h, scale):
    kv, hpooled, q = np.ascontiguousarray(kv), np.ascontiguousarray(hpooled), np.ascontiguousarray(q)
    assert kv.dtype == hpooled.dtype == q.dtype
    H, d = q.shape
    out = np.empty((H, d), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    _check(_load().orc_hca_attend_given(_dt(kv), d, H, m_h, W_h, scale, t, _p(kv), _p(hpooled), _p(q),
                                        _p(out), _p(lse)), "hca_attend_given")
    return out, lse

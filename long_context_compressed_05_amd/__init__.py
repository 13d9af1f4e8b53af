"""Python binding of libcsa.so — compressed sparse attention (CSA) and heavily
compressed attention (HCA) on MI355X.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
(include/csa.h).  PyTorch provides device memory and the stream.  There is no
fallback: if libcsa.so is missing or a call fails, an exception is raised.
The function names are those of the C ABI.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# CSA_LIBRARY=debug loads libcsa_debug.so (the same kernels with device-side
# index checks, see csa_debug_checks); anything else loads libcsa.so
LIB_PATH = os.path.join(_HERE, "libcsa_debug.so" if os.environ.get("CSA_LIBRARY") == "debug" else "libcsa.so")

CSA_OK, CSA_ERR_INVALID, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_DEVICE = 0, -1, -2, -3, -4
CSA_F32, CSA_BF16 = 0, 1

EXPORTS = ("csa_status_string", "csa_last_error", "csa_compress", "csa_cache_append", "csa_mxfp4_quantize", "csa_index_topk_workspace",
           "csa_index_topk", "csa_index_topk_bf16", "csa_sparse_attn_workspace", "csa_sparse_attn", "hca_attn_workspace",
           "hca_attn", "csa_hca_decode_workspace", "csa_hca_decode", "csa_hca_decode_noalloc", "csa_hca_decode_shared",
           "csa_hca_decode_paged",
           "csa_hca_decode_check",
           "csa_hca_decode_fallbacks", "csa_profile_events", "csa_debug_checks")
(CSA_K_IDX_SCORE, CSA_K_IDX_SELECT, CSA_K_IDX_FINAL, CSA_K_ATTN, CSA_K_ATTN_COMBINE, CSA_K_COMPRESS,
 CSA_K_FUSED, CSA_K_PF_THRESH, CSA_K_PF_SELECT, CSA_K_APPEND, CSA_K_QUANT) = range(11)


class CsaBatch(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_q", ctypes.c_int64), ("max_len", ctypes.c_int64),
                ("max_q_per_seq", ctypes.c_int64), ("tok_off", ctypes.c_void_p),
                ("q_off", ctypes.c_void_p), ("q_pos", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libcsa.so not found at {LIB_PATH}; build it with "
                           "`python -m long_context_compressed_05_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, ci, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    bp = ctypes.POINTER(CsaBatch)
    L.csa_status_string.restype = ctypes.c_char_p
    L.csa_status_string.argtypes = [ci]
    L.csa_last_error.restype = ctypes.c_char_p
    L.csa_last_error.argtypes = []
    L.csa_debug_checks.argtypes = [vp]
    L.csa_compress.argtypes = [ci, i32, vp, vp, i64, ci, ci, vp, vp, vp, vp]
    L.csa_mxfp4_quantize.argtypes = [ci, i64, ci, vp, vp, vp, vp]
    L.csa_cache_append.argtypes = [ci, i32, ci, vp, vp, vp, i64, vp, vp, vp, vp, ci, vp, ci, vp, vp, ci, vp, vp, vp,
                                   ci, vp, vp, vp]
    L.csa_index_topk_workspace.argtypes = [bp, i64, ci, ctypes.POINTER(sz)]
    L.csa_index_topk.argtypes = [bp, vp, i64, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.csa_index_topk_bf16.argtypes = [bp, vp, i64, ci, ci, ci, ci, vp, vp, vp, vp, vp, sz, vp]
    L.csa_sparse_attn_workspace.argtypes = [ci, bp, ci, ci, ci, ci, ctypes.POINTER(sz)]
    L.csa_sparse_attn.argtypes = [ci, bp, vp, ci, ci, ctypes.c_float, ci, ci, vp, vp, vp, vp, vp, vp,
                                  vp, sz, vp]
    L.hca_attn_workspace.argtypes = [ci, bp, i64, ci, ci, ci, ctypes.POINTER(sz)]
    L.hca_attn.argtypes = [ci, bp, vp, i64, ci, ci, ci, ctypes.c_float, ci, vp, vp, vp, vp, vp, vp,
                           sz, vp]
    L.csa_hca_decode_workspace.argtypes = [bp, i64, i64, ci, ci, ci, ci, ci, ctypes.POINTER(sz)]
    L.csa_hca_decode.argtypes = [bp, vp, i64, vp, i64, ci, ci, ci, ci, ctypes.c_float, ci, ci, ci, vp, vp, vp, vp,
                                 vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.csa_hca_decode_noalloc.argtypes = [bp, vp, i64, vp, i64, ci, ci, ci, ci, ctypes.c_float, ci, ci, ci, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.csa_hca_decode_shared.argtypes = [bp, vp, vp, vp, i64, vp, i64, ci, ci, ci, ci, ctypes.c_float, ci, ci, ci, vp,
                                        vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.csa_hca_decode_paged.argtypes = [bp, ci, vp, ci, vp, ci, vp, ci, vp, i64, i64, ci, ci, ci, ci, ctypes.c_float, ci,
                                       ci, ci, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.csa_hca_decode_check.argtypes = [bp, vp, vp]
    L.csa_hca_decode_fallbacks.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    L.csa_profile_events.argtypes = [ci, vp, vp]
    for name in EXPORTS:
        L[name].restype = L[name].restype if name in ("csa_status_string", "csa_last_error") else ci
    _lib = L
    return L


class CsaError(RuntimeError):
    def __init__(self, rc: int, what: str):
        L = lib()
        super().__init__(f"{what}: {L.csa_status_string(rc).decode()} ({L.csa_last_error().decode()})")
        self.rc = rc


def _check(rc: int, what: str):
    if rc != CSA_OK:
        raise CsaError(rc, what)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libcsa must be contiguous")
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return CSA_BF16
    raise TypeError(f"KV dtype must be float32 or bfloat16, got {t.dtype}")


@dataclass
class Batch:
    """Sequences and their query rows (device offset arrays + host bounds)."""
    tok_off: torch.Tensor   # int64 [B+1] on the device
    q_off: torch.Tensor     # int64 [B+1]
    q_pos: torch.Tensor     # int64 [n_q]
    n_q: int
    max_len: int
    max_q_per_seq: int

    @property
    def n_seq(self) -> int:
        return self.tok_off.numel() - 1

    def c(self) -> CsaBatch:
        return CsaBatch(self.n_seq, self.n_q, self.max_len, self.max_q_per_seq, _ptr(self.tok_off),
                        _ptr(self.q_off), _ptr(self.q_pos))

    @staticmethod
    def from_host(tok_off, q_off, q_pos, device="cuda") -> "Batch":
        import numpy as np
        tok_off = np.asarray(tok_off, dtype=np.int64)
        q_off = np.asarray(q_off, dtype=np.int64)
        q_pos = np.asarray(q_pos, dtype=np.int64)
        lens = np.diff(tok_off)
        qn = np.diff(q_off)
        return Batch(torch.from_numpy(tok_off).to(device), torch.from_numpy(q_off).to(device),
                     torch.from_numpy(q_pos).to(device), int(q_off[-1]),
                     int(lens.max()) if lens.size else 0, int(qn.max()) if qn.size else 0)


class Workspace:
    """Reusable zero-initialised device workspace (the index workspace must be
    zero-filled before first use; the library leaves it zero-filled)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf: Optional[torch.Tensor] = None

    def get(self, nbytes: int) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


def csa_compress(x: torch.Tensor, z: torch.Tensor, tok_off: torch.Tensor, pool_off: torch.Tensor,
                 max_len: int, m: int, out: torch.Tensor, stream=None) -> torch.Tensor:
    """Pool whole blocks of m rows: x, z [rows][...] -> out [pooled rows][...] (same dtype)."""
    width = x[0].numel() if x.shape[0] > 0 else out[0].numel()
    _check(lib().csa_compress(_dtype_code(x), tok_off.numel() - 1, _ptr(tok_off), _ptr(pool_off),
                              max_len, m, width, _ptr(x), _ptr(z), _ptr(out), _stream(stream)),
           "csa_compress")
    return out


def csa_cache_append(x_new: torch.Tensor, z_new: torch.Tensor, new_off: torch.Tensor, max_new: int,
                     tok_off: torch.Tensor, length: torch.Tensor, kv_raw: torch.Tensor, z_tail: torch.Tensor,
                     pool_off: torch.Tensor, m: int, pooled: torch.Tensor,
                     hpool_off: Optional[torch.Tensor] = None, m_hca: int = 0,
                     hpooled: Optional[torch.Tensor] = None, kvec_off: Optional[torch.Tensor] = None,
                     kvec: Optional[torch.Tensor] = None, k_codes: Optional[torch.Tensor] = None,
                     k_scales: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append each sequence's new rows (x_new, z_new [sum n][...], new_off [B+1]) to
    the raw cache, pool the blocks they complete into `pooled` (and `hpooled`),
    encode the completed CSA blocks' indexer vectors (kvec [sum blocks][kdim],
    kvec_off [B+1]) into the MXFP4 key cache (k_codes, k_scales), keep the
    latest tokens' logits in `z_tail` [B][ring][...] and advance `length` [B]
    (int64, device) in place."""
    width = kv_raw[0].numel()
    ring = z_tail.shape[1]
    kdim = kvec.shape[-1] if kvec is not None else 0
    _check(lib().csa_cache_append(_dtype_code(kv_raw), new_off.numel() - 1, width, _ptr(tok_off), _ptr(length),
                                  _ptr(new_off), max_new, _ptr(x_new), _ptr(z_new), _ptr(kv_raw), _ptr(z_tail),
                                  ring, _ptr(pool_off), m, _ptr(pooled), _ptr(hpool_off), m_hca, _ptr(hpooled),
                                  _ptr(kvec_off), _ptr(kvec), kdim, _ptr(k_codes), _ptr(k_scales), _stream(stream)),
           "csa_cache_append")


def csa_debug_checks() -> int:
    """Violations counted by a debug library's device-side index checks since
    the last call (then cleared); raises on a release library."""
    n = ctypes.c_uint64(0)
    _check(lib().csa_debug_checks(ctypes.byref(n)), "csa_debug_checks")
    return int(n.value)


def csa_mxfp4_quantize(x: torch.Tensor, codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rows of x ([..., dim], fp32 or bf16, dim a multiple of 32) -> MXFP4 codes
    [..., dim/2] and E8M0 scales [..., dim/32] (uint8)."""
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (dim // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (dim // 32,), dtype=torch.uint8, device=x.device)
    _check(lib().csa_mxfp4_quantize(_dtype_code(x), rows, dim, _ptr(x), _ptr(codes), _ptr(scales), _stream(stream)),
           "csa_mxfp4_quantize")
    return codes, scales


def csa_index_topk_workspace(batch: Batch, max_pool: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    b = batch.c()
    _check(lib().csa_index_topk_workspace(ctypes.byref(b), max_pool, k, ctypes.byref(n)),
           "csa_index_topk_workspace")
    return n.value


def csa_index_topk(batch: Batch, pool_off: torch.Tensor, max_pool: int, m: int, k: int,
                   q_codes: torch.Tensor, q_scales: torch.Tensor, w: torch.Tensor,
                   k_codes: torch.Tensor, k_scales: torch.Tensor, idx: Optional[torch.Tensor] = None,
                   ws: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    if idx is None:
        idx = torch.empty((batch.n_q, k), dtype=torch.int32, device=q_codes.device)
    ws = ws or Workspace(q_codes.device)
    nbytes = csa_index_topk_workspace(batch, max_pool, k)
    buf = ws.get(nbytes)
    b = batch.c()
    n_heads, dim = q_codes.shape[-2], 2 * q_codes.shape[-1]
    _check(lib().csa_index_topk(ctypes.byref(b), _ptr(pool_off), max_pool, m, n_heads, dim, k,
                                _ptr(q_codes), _ptr(q_scales), _ptr(w), _ptr(k_codes), _ptr(k_scales),
                                _ptr(idx), _ptr(buf), nbytes, _stream(stream)), "csa_index_topk")
    return idx


def csa_index_topk_bf16(batch: Batch, pool_off: torch.Tensor, max_pool: int, m: int, k: int, q: torch.Tensor,
                        w: torch.Tensor, keys: torch.Tensor, idx: Optional[torch.Tensor] = None,
                        ws: Optional[Workspace] = None, stream=None) -> torch.Tensor:
    """The indexer with bf16 operands: q [n_q][4][64], keys [sum P][64] (bf16), w [n_q][4]."""
    if idx is None:
        idx = torch.empty((batch.n_q, k), dtype=torch.int32, device=q.device)
    ws = ws or Workspace(q.device)
    nbytes = csa_index_topk_workspace(batch, max_pool, k)
    buf = ws.get(nbytes)
    b = batch.c()
    _check(lib().csa_index_topk_bf16(ctypes.byref(b), _ptr(pool_off), max_pool, m, q.shape[-2], q.shape[-1], k,
                                     _ptr(q), _ptr(w), _ptr(keys), _ptr(idx), _ptr(buf), nbytes, _stream(stream)),
           "csa_index_topk_bf16")
    return idx


def csa_sparse_attn_workspace(dtype_code: int, batch: Batch, H: int, d: int, W: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    b = batch.c()
    _check(lib().csa_sparse_attn_workspace(dtype_code, ctypes.byref(b), H, d, W, k, ctypes.byref(n)),
           "csa_sparse_attn_workspace")
    return n.value


def csa_sparse_attn(batch: Batch, pool_off: torch.Tensor, q: torch.Tensor, kv_pool: torch.Tensor,
                    kv_raw: torch.Tensor, idx: torch.Tensor, W: int, scale: float,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    ws: Optional[Workspace] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    dt = _dtype_code(q)
    H, d = q.shape[-2], q.shape[-1]
    k = idx.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=q.device)
    ws = ws or Workspace(q.device)
    nbytes = csa_sparse_attn_workspace(dt, batch, H, d, W, k)
    buf = ws.get(nbytes)
    b = batch.c()
    _check(lib().csa_sparse_attn(dt, ctypes.byref(b), _ptr(pool_off), H, d, scale, W, k, _ptr(q),
                                 _ptr(kv_pool), _ptr(kv_raw), _ptr(idx), _ptr(out), _ptr(lse),
                                 _ptr(buf), nbytes, _stream(stream)), "csa_sparse_attn")
    return out, lse


def hca_attn_workspace(dtype_code: int, batch: Batch, max_hpool: int, H: int, d: int, W_hca: int) -> int:
    n = ctypes.c_size_t(0)
    b = batch.c()
    _check(lib().hca_attn_workspace(dtype_code, ctypes.byref(b), max_hpool, H, d, W_hca, ctypes.byref(n)),
           "hca_attn_workspace")
    return n.value


def hca_attn(batch: Batch, hpool_off: torch.Tensor, max_hpool: int, m_hca: int, q: torch.Tensor,
             kv_pool_hca: torch.Tensor, kv_raw: Optional[torch.Tensor], W_hca: int, scale: float,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             ws: Optional[Workspace] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    dt = _dtype_code(q)
    H, d = q.shape[-2], q.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=q.device)
    ws = ws or Workspace(q.device)
    nbytes = hca_attn_workspace(dt, batch, max_hpool, H, d, W_hca)
    buf = ws.get(nbytes)
    b = batch.c()
    _check(lib().hca_attn(dt, ctypes.byref(b), _ptr(hpool_off), max_hpool, m_hca, H, d, scale, W_hca,
                          _ptr(q), _ptr(kv_pool_hca), _ptr(kv_raw), _ptr(out), _ptr(lse), _ptr(buf),
                          nbytes, _stream(stream)), "hca_attn")
    return out, lse


_hip = None


def _hiplib():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return _hip


class HipEvent:
    """A plain hipEvent_t (timing enabled) for the tracing hook."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = _hiplib().hipEventCreateWithFlags(ctypes.byref(h), 0)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.handle = h

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        _hiplib().hipEventSynchronize(end.handle)
        rc = _hiplib().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if _hip is not None and self.handle:
            _hip.hipEventDestroy(self.handle)


def csa_profile_events(kernel_id: int, start: Optional[HipEvent] = None, stop: Optional[HipEvent] = None) -> None:
    """Bracket every launch of one internal kernel (this thread) with the given
    HipEvent pair; csa_profile_events(id) clears."""
    sp = start.handle if start is not None else None
    ep = stop.handle if stop is not None else None
    _check(lib().csa_profile_events(kernel_id, sp, ep), "csa_profile_events")


def csa_hca_decode_workspace(batch: Batch, max_pool: int, max_hpool: int, H: int, d: int, k: int, W: int,
                             W_hca: int) -> int:
    n = ctypes.c_size_t(0)
    b = batch.c()
    _check(lib().csa_hca_decode_workspace(ctypes.byref(b), max_pool, max_hpool, H, d, k, W, W_hca, ctypes.byref(n)),
           "csa_hca_decode_workspace")
    return n.value


def csa_hca_decode(batch: Batch, pool_off, max_pool: int, hpool_off, max_hpool: int, m: int, m_hca: int,
                   k: int, W: int, W_hca: int, scale: float, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool,
                   kv_pool_hca, kv_raw, idx=None, csa_out=None, csa_lse=None, hca_out=None, hca_lse=None,
                   ws: Optional[Workspace] = None, stream=None):
    """One fused decode step (index + top-k + CSA + HCA) in a single launch."""
    H, d = q.shape[-2], q.shape[-1]
    dev = q.device
    if idx is None:
        idx = torch.empty((batch.n_q, k), dtype=torch.int32, device=dev)
    if csa_out is None:
        csa_out = torch.empty_like(q)
    if hca_out is None:
        hca_out = torch.empty_like(q)
    if csa_lse is None:
        csa_lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=dev)
    if hca_lse is None:
        hca_lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=dev)
    ws = ws or Workspace(dev)
    nbytes = csa_hca_decode_workspace(batch, max_pool, max_hpool, H, d, k, W, W_hca)
    buf = ws.get(nbytes)
    b = batch.c()
    _check(lib().csa_hca_decode(ctypes.byref(b), _ptr(pool_off), max_pool, _ptr(hpool_off), max_hpool, m, m_hca, H, d,
                                scale, k, W, W_hca, _ptr(q_codes), _ptr(q_scales), _ptr(w), _ptr(k_codes),
                                _ptr(k_scales), _ptr(q), _ptr(kv_pool), _ptr(kv_pool_hca), _ptr(kv_raw), _ptr(idx),
                                _ptr(csa_out), _ptr(csa_lse), _ptr(hca_out), _ptr(hca_lse), _ptr(buf), nbytes,
                                _stream(stream)), "csa_hca_decode")
    return idx, csa_out, csa_lse, hca_out, hca_lse


def csa_hca_decode_noalloc(batch: Batch, pool_off, max_pool: int, hpool_off, max_hpool: int, m: int, m_hca: int,
                           k: int, W: int, W_hca: int, scale: float, q_codes, q_scales, w, k_codes, k_scales, q,
                           kv_pool, kv_pool_hca, kv_raw, idx, csa_out, csa_lse, hca_out, hca_lse, stream=None):
    """csa_hca_decode on the library's static scratch: no workspace, and no
    allocation in the call (the outputs are the caller's)."""
    H, d = q.shape[-2], q.shape[-1]
    b = batch.c()
    _check(lib().csa_hca_decode_noalloc(ctypes.byref(b), _ptr(pool_off), max_pool, _ptr(hpool_off), max_hpool, m,
                                        m_hca, H, d, scale, k, W, W_hca, _ptr(q_codes), _ptr(q_scales), _ptr(w),
                                        _ptr(k_codes), _ptr(k_scales), _ptr(q), _ptr(kv_pool), _ptr(kv_pool_hca),
                                        _ptr(kv_raw), _ptr(idx), _ptr(csa_out), _ptr(csa_lse), _ptr(hca_out),
                                        _ptr(hca_lse), _stream(stream)), "csa_hca_decode_noalloc")
    return idx, csa_out, csa_lse, hca_out, hca_lse


def csa_hca_decode_shared(batch: Batch, prefix_seq, prefix_tokens, pool_off, max_pool: int, hpool_off,
                          max_hpool: int, m: int, m_hca: int, k: int, W: int, W_hca: int, scale: float, q_codes,
                          q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca, kv_raw, idx=None, csa_out=None,
                          csa_lse=None, hca_out=None, hca_lse=None, ws: Optional[Workspace] = None, stream=None):
    """csa_hca_decode where sequence b's first prefix_tokens[b] tokens live in sequence prefix_seq[b]'s cache."""
    H, d = q.shape[-2], q.shape[-1]
    dev = q.device
    if idx is None:
        idx = torch.empty((batch.n_q, k), dtype=torch.int32, device=dev)
    if csa_out is None:
        csa_out = torch.empty_like(q)
    if hca_out is None:
        hca_out = torch.empty_like(q)
    if csa_lse is None:
        csa_lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=dev)
    if hca_lse is None:
        hca_lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=dev)
    ws = ws or Workspace(dev)
    nbytes = csa_hca_decode_workspace(batch, max_pool, max_hpool, H, d, k, W, W_hca)
    buf = ws.get(nbytes)
    b = batch.c()
    _check(lib().csa_hca_decode_shared(ctypes.byref(b), _ptr(prefix_seq), _ptr(prefix_tokens), _ptr(pool_off),
                                       max_pool, _ptr(hpool_off), max_hpool, m, m_hca, H, d, scale, k, W, W_hca,
                                       _ptr(q_codes), _ptr(q_scales), _ptr(w), _ptr(k_codes), _ptr(k_scales),
                                       _ptr(q), _ptr(kv_pool), _ptr(kv_pool_hca), _ptr(kv_raw), _ptr(idx),
                                       _ptr(csa_out), _ptr(csa_lse), _ptr(hca_out), _ptr(hca_lse), _ptr(buf),
                                       nbytes, _stream(stream)), "csa_hca_decode_shared")
    return idx, csa_out, csa_lse, hca_out, hca_lse


def csa_hca_decode_paged(batch: Batch, page_rows: int, page_table, pooled_rows, hca_page_rows: int, hca_page_table,
                         hca_pooled_rows, max_pool: int, max_hpool: int, m: int, m_hca: int, k: int, W: int,
                         W_hca: int, scale: float, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca,
                         kv_raw, idx=None, csa_out=None, csa_lse=None, hca_out=None, hca_lse=None,
                         ws: Optional[Workspace] = None, stream=None):
    """csa_hca_decode over paged pooled caches (page tables [n_seq][pages] int32, row counts [n_seq] int64)."""
    H, d = q.shape[-2], q.shape[-1]
    dev = q.device
    if idx is None:
        idx = torch.empty((batch.n_q, k), dtype=torch.int32, device=dev)
    if csa_out is None:
        csa_out = torch.empty_like(q)
    if hca_out is None:
        hca_out = torch.empty_like(q)
    if csa_lse is None:
        csa_lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=dev)
    if hca_lse is None:
        hca_lse = torch.empty((batch.n_q, H), dtype=torch.float32, device=dev)
    ws = ws or Workspace(dev)
    nbytes = csa_hca_decode_workspace(batch, max_pool, max_hpool, H, d, k, W, W_hca)
    buf = ws.get(nbytes)
    b = batch.c()
    _check(lib().csa_hca_decode_paged(ctypes.byref(b), page_rows, _ptr(page_table), page_table.shape[-1],
                                      _ptr(pooled_rows), hca_page_rows, _ptr(hca_page_table),
                                      hca_page_table.shape[-1], _ptr(hca_pooled_rows), max_pool, max_hpool, m, m_hca,
                                      H, d, scale, k, W, W_hca, _ptr(q_codes), _ptr(q_scales), _ptr(w),
                                      _ptr(k_codes), _ptr(k_scales), _ptr(q), _ptr(kv_pool), _ptr(kv_pool_hca),
                                      _ptr(kv_raw), _ptr(idx), _ptr(csa_out), _ptr(csa_lse), _ptr(hca_out),
                                      _ptr(hca_lse), _ptr(buf), nbytes, _stream(stream)), "csa_hca_decode_paged")
    return idx, csa_out, csa_lse, hca_out, hca_lse


def csa_hca_decode_fallbacks(ws: Workspace, stream=None) -> int:
    """Synchronise and return how many row selections on `ws` took the exact fallback."""
    n = ctypes.c_uint32(0)
    _check(lib().csa_hca_decode_fallbacks(_ptr(ws.buf), _stream(stream), ctypes.byref(n)), "csa_hca_decode_fallbacks")
    return int(n.value)


def csa_hca_decode_check(batch: Batch, ws: Workspace, stream=None) -> None:
    """Synchronise and raise if a fused decode launch on `ws` hit its wait bound."""
    b = batch.c()
    _check(lib().csa_hca_decode_check(ctypes.byref(b), _ptr(ws.buf), _stream(stream)), "csa_hca_decode")

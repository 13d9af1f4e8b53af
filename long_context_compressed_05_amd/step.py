"""One CSA + HCA attention step on device-resident buffers.

Sequences the C-ABI calls only (no arithmetic here):
  build_caches : csa_compress for the CSA block size m and the HCA block m'
  attend       : csa_index_topk -> csa_sparse_attn, and hca_attn
Buffers are plain torch tensors on the GPU; bf16 data may be given as
torch.bfloat16 or as its uint16/int16 bit pattern.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np
import torch

from . import (Batch, Workspace, csa_compress, csa_hca_decode, csa_hca_decode_check, csa_index_topk,
               csa_sparse_attn, hca_attn)


@dataclass
class Params:
    H: int
    d: int
    m: int
    k: int
    W: int
    m_hca: int
    W_hca: int = 0
    scale: Optional[float] = None

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)


def to_device(host: Dict[str, np.ndarray], device="cuda") -> Dict[str, torch.Tensor]:
    """numpy inputs -> device tensors (uint16 arrays are bf16 bit patterns)."""
    out = {}
    for name, a in host.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if a.dtype == np.uint16:
            t = t.view(torch.bfloat16)
        out[name] = t.to(device, non_blocking=False)
    return out


@dataclass
class Layer:
    """Device buffers of one layer: raw KV and logits, pooled caches, indexer keys."""
    p: Params
    batch: Batch
    tok_off: torch.Tensor
    pool_off: torch.Tensor
    hpool_off: torch.Tensor
    max_pool: int
    max_hpool: int
    kv: torch.Tensor
    kc: torch.Tensor
    ks: torch.Tensor
    z: Optional[torch.Tensor] = None
    pooled: Optional[torch.Tensor] = None
    hpooled: Optional[torch.Tensor] = None
    ws_idx: Workspace = field(default_factory=Workspace)
    ws_csa: Workspace = field(default_factory=Workspace)
    ws_hca: Workspace = field(default_factory=Workspace)
    ws_fused: Workspace = field(default_factory=Workspace)

    @staticmethod
    def from_host(p: Params, host: Dict[str, np.ndarray], device="cuda") -> "Layer":
        dev = to_device({k: host[k] for k in ("kv", "z", "kc", "ks", "tok_off", "pool_off", "hpool_off")
                         if k in host}, device)
        batch = Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"], device)
        pool_off, hpool_off = host["pool_off"], host["hpool_off"]
        return Layer(p=p, batch=batch, tok_off=dev["tok_off"], pool_off=dev["pool_off"],
                     hpool_off=dev["hpool_off"], max_pool=int(np.diff(pool_off).max()),
                     max_hpool=int(np.diff(hpool_off).max()), kv=dev["kv"], kc=dev["kc"], ks=dev["ks"],
                     z=dev.get("z"), ws_idx=Workspace(device), ws_csa=Workspace(device),
                     ws_hca=Workspace(device), ws_fused=Workspace(device))

    def build_caches(self, stream=None):
        """Pool the raw rows into the CSA (m) and HCA (m') caches."""
        n_pool = int(self.pool_off[-1].item())
        n_hpool = int(self.hpool_off[-1].item())
        shape = (2, self.p.d)
        if self.pooled is None:
            self.pooled = torch.empty((n_pool, *shape), dtype=self.kv.dtype, device=self.kv.device)
        if self.hpooled is None:
            self.hpooled = torch.empty((n_hpool, *shape), dtype=self.kv.dtype, device=self.kv.device)
        csa_compress(self.kv, self.z, self.tok_off, self.pool_off, self.batch.max_len, self.p.m,
                     self.pooled, stream)
        csa_compress(self.kv, self.z, self.tok_off, self.hpool_off, self.batch.max_len, self.p.m_hca,
                     self.hpooled, stream)

    def attend(self, q, qc, qs, w, idx=None, csa_out=None, csa_lse=None, hca_out=None, hca_lse=None,
               stream=None, hca_stream=None):
        """Index + top-k + CSA sparse attention, and HCA dense attention, for the batch's queries."""
        p = self.p
        idx = csa_index_topk(self.batch, self.pool_off, self.max_pool, p.m, p.k, qc, qs, w, self.kc,
                             self.ks, idx=idx, ws=self.ws_idx, stream=stream)
        csa_out, csa_lse = csa_sparse_attn(self.batch, self.pool_off, q, self.pooled, self.kv, idx, p.W,
                                           p.sm_scale, out=csa_out, lse=csa_lse, ws=self.ws_csa,
                                           stream=stream)
        hca_out, hca_lse = hca_attn(self.batch, self.hpool_off, self.max_hpool, p.m_hca, q, self.hpooled,
                                    self.kv, p.W_hca, p.sm_scale, out=hca_out, lse=hca_lse,
                                    ws=self.ws_hca, stream=hca_stream if hca_stream is not None else stream)
        return idx, csa_out, csa_lse, hca_out, hca_lse

    def decode_fused(self, q, qc, qs, w, idx=None, csa_out=None, csa_lse=None, hca_out=None, hca_lse=None,
                     stream=None, kc=None, ks=None, hpooled=None):
        """The same step as attend() in one fused launch (decode batches: one query per sequence)."""
        p = self.p
        return csa_hca_decode(self.batch, self.pool_off, self.max_pool, self.hpool_off, self.max_hpool, p.m, p.m_hca,
                              p.k, p.W, p.W_hca, p.sm_scale, qc, qs, w, self.kc if kc is None else kc,
                              self.ks if ks is None else ks, q, self.pooled,
                              self.hpooled if hpooled is None else hpooled, self.kv, idx=idx, csa_out=csa_out,
                              csa_lse=csa_lse, hca_out=hca_out, hca_lse=hca_lse, ws=self.ws_fused, stream=stream)

    def check_fused(self, stream=None):
        csa_hca_decode_check(self.batch, self.ws_fused, stream)

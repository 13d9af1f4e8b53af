"""csa_hca_decode_noalloc (the decode step on the library's static scratch,
for callers that cannot allocate) against csa_hca_decode with a caller-owned
workspace, through the C ABI: bit-identical outputs on two calls in a row, the
second with a smaller input (a new workspace layout, so the scratch is
cleared first), then the same smaller input again (the same layout, reused
without clearing), and the larger one once more."""
import math

import numpy as np
import pytest
import torch

import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _lib():
    import long_context_compressed_05_amd as csa
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    csa.lib()  # raises if libcsa.so is missing: no fallback
    return csa


def _case(name, lengths, k, seed, **kw):
    wl = synth.Workload(name, list(lengths), [L - 1 for L in lengths], k=k, seed=seed, **kw)
    host = synth.make_inputs(wl)
    from long_context_compressed_05_amd.step import Layer, Params, to_device
    layer = Layer.from_host(Params(H=wl.H, d=wl.d, m=wl.m, k=wl.k, W=wl.W, m_hca=wl.m_hca, W_hca=wl.W_hca), host)
    layer.build_caches()
    dq = to_device({x: host[x] for x in ("q", "qc", "qs", "w")})
    return wl, layer, dq


def _noalloc(csa, wl, layer, dq):
    """The new entry point, with outputs allocated here (outside the call)."""
    p = layer.p
    dev = dq["q"].device
    idx = torch.full((wl.n_q, wl.k), -7, dtype=torch.int32, device=dev)
    co, ho = torch.zeros_like(dq["q"]), torch.zeros_like(dq["q"])
    cl = torch.zeros((wl.n_q, wl.H), dtype=torch.float32, device=dev)
    hl = torch.zeros_like(cl)
    out = csa.csa_hca_decode_noalloc(layer.batch, layer.pool_off, layer.max_pool, layer.hpool_off, layer.max_hpool,
                                     p.m, p.m_hca, p.k, p.W, p.W_hca, p.sm_scale, dq["qc"], dq["qs"], dq["w"],
                                     layer.kc, layer.ks, dq["q"], layer.pooled, layer.hpooled, layer.kv, idx, co, cl,
                                     ho, hl)
    torch.cuda.synchronize()
    return [P.torch_to_np(t) for t in out]


def _with_workspace(layer, dq):
    out = layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])
    layer.check_fused()
    torch.cuda.synchronize()
    return [P.torch_to_np(t) for t in out]


def _same(got, want, what):
    for name, x, y in zip(("idx", "csa_out", "csa_lse", "hca_out", "hca_lse"), got, want):
        assert np.array_equal(x, y), f"{what}: {name} differs from csa_hca_decode with a workspace"


def test_noalloc_decode_equals_the_workspace_entry_point():
    csa = _lib()
    big = _case("noalloc_big", [20003, 9001, 70001, 4099], k=256, seed=71)
    small = _case("noalloc_small", [3001, 517], k=64, seed=72, H=32)
    want_big = _with_workspace(big[1], big[2])
    want_small = _with_workspace(small[1], small[2])
    _same(_noalloc(csa, *big), want_big, "first call (4 sequences up to 70K tokens)")
    _same(_noalloc(csa, *small), want_small, "second call, smaller input")
    _same(_noalloc(csa, *small), want_small, "third call, same shapes")
    _same(_noalloc(csa, *big), want_big, "fourth call, the larger input again")


def test_noalloc_decode_rejects_steps_beyond_its_scratch():
    """64 sequences with max_pool = 262,144 need more than the 64 MiB scratch
    (the candidate keys alone take 64 MiB): the call is rejected before it
    enqueues anything.  The caches are real (64 sequences of 1030 tokens, so
    the host bounds are valid upper bounds of the true sizes)."""
    csa = _lib()
    wl, layer, dq = _case("noalloc_too_big", [1030] * 64, k=64, seed=73, H=16)
    p = layer.p
    max_pool, max_hpool = 262144, 8192
    need = csa.csa_hca_decode_workspace(layer.batch, max_pool, max_hpool, wl.H, wl.d, wl.k, wl.W, wl.W_hca)
    assert need > SCRATCH_BYTES
    idx = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device="cuda")
    co, ho = torch.empty_like(dq["q"]), torch.empty_like(dq["q"])
    cl = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device="cuda")
    hl = torch.empty_like(cl)
    with pytest.raises(csa.CsaError) as e:
        csa.csa_hca_decode_noalloc(layer.batch, layer.pool_off, max_pool, layer.hpool_off, max_hpool, p.m, p.m_hca,
                                   p.k, p.W, p.W_hca, p.sm_scale, dq["qc"], dq["qs"], dq["w"], layer.kc, layer.ks,
                                   dq["q"], layer.pooled, layer.hpooled, layer.kv, idx, co, cl, ho, hl)
    assert e.value.rc == csa.CSA_ERR_UNSUPPORTED
    assert "64 MiB" in str(e.value)
    # the scratch still serves a step that fits, bit for bit
    small = _case("noalloc_after_reject", [3001, 517, 9000], k=128, seed=74)
    _same(_noalloc(csa, *small), _with_workspace(small[1], small[2]), "a step after the rejected one")

"""GPU parity of the whole prefill step at full size: a 4096-token chunk on a
65,536-token cache (reading D16: append the chunk's rows, pool the blocks it
completes, then index and attend), through the C ABI, against the CPU oracle
on sampled queries.  Pages: discuss.pytorch.kr CSA/HCA section (top-k over the
compressed entries plus a sliding window for CSA, dense attention over the
heavily compressed entries for HCA); sigco.tistory.com KV-cache section (the
compressed entries, the window and the tail state are kept apart)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _lib():
    import long_context_compressed_05_amd as csa
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    csa.lib()  # raises if libcsa.so is missing: no fallback
    return csa


def run_prefill_chunk(csa, wl, host, T0):
    """Device pipeline of one prefill chunk: caches of the first T0 tokens
    (bulk pooling), csa_cache_append of the chunk, csa_index_topk,
    csa_sparse_attn and hca_attn for every query of the chunk.  Returns the
    device caches and outputs."""
    from long_context_compressed_05_amd.step import to_device
    dev = "cuda"
    L = wl.lengths[0]
    n = L - T0
    d = to_device({k: host[k] for k in ("kv", "z", "q", "qc", "qs", "w", "kc", "ks")})
    kv_raw = torch.zeros_like(d["kv"])
    kv_raw[:T0] = d["kv"][:T0]
    P_cap, Ph_cap = L // wl.m, L // wl.m_hca
    pooled = torch.zeros((P_cap, 2, wl.d), dtype=d["kv"].dtype, device=dev)
    hpooled = torch.zeros((Ph_cap, 2, wl.d), dtype=d["kv"].dtype, device=dev)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int64)).to(dev)
    tok0, pool_off, hpool_off = t([0, T0]), t([0, P_cap]), t([0, Ph_cap])
    csa.csa_compress(d["kv"], d["z"], tok0, pool_off, T0, wl.m, pooled)
    csa.csa_compress(d["kv"], d["z"], tok0, hpool_off, T0, wl.m_hca, hpooled)
    ring = wl.m_hca
    slots = np.array([T0 - ring + ((s - (T0 - ring)) % ring) for s in range(ring)])
    z_tail = d["z"][t(slots)].reshape(1, ring, 2, wl.d).contiguous()
    length = t([T0])
    tok_off = t([0, L])
    csa.csa_cache_append(d["kv"][T0:].contiguous(), d["z"][T0:].contiguous(), t([0, n]), n, tok_off, length, kv_raw,
                         z_tail, pool_off, wl.m, pooled, hpool_off, wl.m_hca, hpooled)
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    scale = 1 / math.sqrt(wl.d)
    idx = csa.csa_index_topk(batch, pool_off, P_cap, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"], d["ks"])
    co, cl = csa.csa_sparse_attn(batch, pool_off, d["q"], pooled, kv_raw, idx, wl.W, scale)
    ho, hl = csa.hca_attn(batch, hpool_off, Ph_cap, wl.m_hca, d["q"], hpooled, kv_raw, wl.W_hca, scale)
    torch.cuda.synchronize()
    return dict(d=d, kv_raw=kv_raw, pooled=pooled, hpooled=hpooled, length=length, z_tail=z_tail, idx=idx, co=co,
                cl=cl, ho=ho, hl=hl, tok_off=tok_off, pool_off=pool_off, hpool_off=hpool_off)


def check_prefill_rows(wl, host, res, rows):
    """Oracle parity of the sampled query rows: top-k bit for bit, CSA and HCA
    outputs and lse within the bf16 tolerances over the sampled rows."""
    scale = 1 / math.sqrt(wl.d)
    kv, z = host["kv"], host["z"]
    pooled64 = oracle.pool(kv, z, wl.m)
    hpooled64 = oracle.pool(kv, z, wl.m_hca)
    idx = P.torch_to_np(res["idx"])
    co, cl = P.torch_to_np(res["co"]), P.torch_to_np(res["cl"])
    ho, hl = P.torch_to_np(res["ho"]), P.torch_to_np(res["hl"])
    want = {name: [] for name in ("co", "cl", "ho", "hl")}
    for r in rows:
        tq = int(host["q_pos"][r])
        o, l, i = oracle.csa_query(kv, z, host["q"][r], tq, wl.m, wl.W, wl.k, scale, host["qc"][r], host["qs"][r],
                                   host["w"][r], host["kc"], host["ks"], pooled=pooled64)
        assert np.array_equal(idx[r], i), f"top-k of query {r} (t={tq})"
        want["co"].append(o)
        want["cl"].append(l)
        o, l = oracle.hca_query(kv, z, host["q"][r], tq, wl.m_hca, wl.W_hca, scale, hpooled=hpooled64)
        want["ho"].append(o)
        want["hl"].append(l)
    rows = list(rows)
    P.check_close(co[rows], np.stack(want["co"]), wl.dtype, "csa output of the sampled queries")
    P.check_close(cl[rows], np.stack(want["cl"]), "bf16", "csa lse of the sampled queries")
    P.check_close(ho[rows], np.stack(want["ho"]), wl.dtype, "hca output of the sampled queries")
    P.check_close(hl[rows], np.stack(want["hl"]), "bf16", "hca lse of the sampled queries")


def test_prefill_chunk_full_size_end_to_end():
    """4096 queries at positions 65,536..69,631 of one sequence, H = 64 bf16,
    m = 4 (17,408 pooled entries, top-512), W = 128, m' = 128 (544 HCA rows), in
    the launch configuration the benchmark times.  The appended caches equal
    the bulk pooling of the whole sequence bit for bit; 72 sampled queries
    (first, last and spread over the chunk) match the oracle."""
    csa = _lib()
    wl = synth.prefill_4k_on_64k()
    host = synth.make_inputs(wl)
    T0 = wl.q_start[0]
    res = run_prefill_chunk(csa, wl, host, T0)
    assert int(res["length"].item()) == wl.lengths[0]
    # the appended raw rows and pooled caches against the whole sequence's bulk pooling
    assert torch.equal(res["kv_raw"], res["d"]["kv"])
    bulk = torch.empty_like(res["pooled"])
    hbulk = torch.empty_like(res["hpooled"])
    tok = torch.from_numpy(host["tok_off"]).cuda()
    csa.csa_compress(res["d"]["kv"], res["d"]["z"], tok, res["pool_off"], wl.lengths[0], wl.m, bulk)
    csa.csa_compress(res["d"]["kv"], res["d"]["z"], tok, res["hpool_off"], wl.lengths[0], wl.m_hca, hbulk)
    torch.cuda.synchronize()
    assert torch.equal(res["pooled"], bulk), "CSA pooled rows after the append differ from the bulk pooling"
    assert torch.equal(res["hpooled"], hbulk), "HCA pooled rows after the append differ from the bulk pooling"
    n_q = wl.n_q
    rng = np.random.default_rng(3)
    rows = sorted(set([0, 1, 2, 127, 128, n_q - 2, n_q - 1] + [int(x) for x in rng.choice(n_q, 65, replace=False)]))
    assert len(rows) >= 64
    check_prefill_rows(wl, host, res, rows)


def test_prefill_chunk_ragged_small_end_to_end():
    """The same pipeline on a chunk that spans a few tiles with ragged ends:
    a 1,030-token cache and a 301-token chunk (its first query at a position
    that is not on a block boundary, its last block incomplete), every query
    against the oracle."""
    csa = _lib()
    T0, n = 1030, 301
    wl = synth.Workload("prefill_ragged_small", [T0 + n], [T0], k=64, seed=61)
    host = synth.make_inputs(wl)
    res = run_prefill_chunk(csa, wl, host, T0)
    check_prefill_rows(wl, host, res, range(wl.n_q))


def test_prefill_step_replays_from_a_hip_graph():
    """The prefill step (append, index, CSA and HCA attention) captured once in
    a HIP graph and replayed three times, with the caches' lengths and tail
    rings reset and unrelated eager work between the replays: every replay's
    top-k is bit-identical and its outputs and LSEs equal to the eager step's
    (nothing in the step records a memset or allocates)."""
    csa = _lib()
    from long_context_compressed_05_amd.step import to_device
    T0, n = 1030, 301
    wl = synth.Workload("prefill_graph", [T0 + n], [T0], k=64, seed=62)
    host = synth.make_inputs(wl)
    dev = "cuda"
    L = wl.lengths[0]
    d = to_device({k: host[k] for k in ("kv", "z", "q", "qc", "qs", "w", "kc", "ks")})
    kv_raw = torch.zeros_like(d["kv"])
    kv_raw[:T0] = d["kv"][:T0]
    P_cap, Ph_cap = L // wl.m, L // wl.m_hca
    pooled = torch.zeros((P_cap, 2, wl.d), dtype=d["kv"].dtype, device=dev)
    hpooled = torch.zeros((Ph_cap, 2, wl.d), dtype=d["kv"].dtype, device=dev)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int64)).to(dev)
    tok0, pool_off, hpool_off, tok_off = t([0, T0]), t([0, P_cap]), t([0, Ph_cap]), t([0, L])
    csa.csa_compress(d["kv"], d["z"], tok0, pool_off, T0, wl.m, pooled)
    csa.csa_compress(d["kv"], d["z"], tok0, hpool_off, T0, wl.m_hca, hpooled)
    ring = wl.m_hca
    slots = np.array([T0 - ring + ((s - (T0 - ring)) % ring) for s in range(ring)])
    tail0 = d["z"][t(slots)].reshape(1, ring, 2, wl.d).contiguous()
    z_tail, len0 = tail0.clone(), t([T0])
    length = len0.clone()
    x_new, z_new, new_off = d["kv"][T0:].contiguous(), d["z"][T0:].contiguous(), t([0, n])
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    scale = 1 / math.sqrt(wl.d)
    idx = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device=dev)
    co, ho = torch.empty_like(d["q"]), torch.empty_like(d["q"])
    cl = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=dev)
    hl = torch.empty_like(cl)
    ws_i, ws_c, ws_h = csa.Workspace(), csa.Workspace(), csa.Workspace()

    def step():
        csa.csa_cache_append(x_new, z_new, new_off, n, tok_off, length, kv_raw, z_tail, pool_off, wl.m, pooled,
                             hpool_off, wl.m_hca, hpooled)
        csa.csa_index_topk(batch, pool_off, P_cap, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"], d["ks"], idx=idx,
                           ws=ws_i)
        csa.csa_sparse_attn(batch, pool_off, d["q"], pooled, kv_raw, idx, wl.W, scale, out=co, lse=cl, ws=ws_c)
        csa.hca_attn(batch, hpool_off, Ph_cap, wl.m_hca, d["q"], hpooled, kv_raw, wl.W_hca, scale, out=ho, lse=hl,
                     ws=ws_h)

    def reset():
        length.copy_(len0)
        z_tail.copy_(tail0)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (idx, co, cl, ho, hl, length, z_tail)]
    reset()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(3):
        reset()
        for x in (idx, co, cl, ho, hl):
            x.fill_(0)
        junk = junk * 1.0001 + 1.0  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("idx", "csa out", "csa lse", "hca out", "hca lse", "length", "tail ring"),
                                   (idx, co, cl, ho, hl, length, z_tail), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager step"

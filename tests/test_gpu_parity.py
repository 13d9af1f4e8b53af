"""GPU parity of the HIP path (through the C ABI) against the CPU oracle on
the same seeded inputs, at sizes the oracle finishes in seconds that still
span several tiles, ragged batches and tails, and the degenerate cases
(no visible block, k above the visible count, k = 1, window clipped at the
sequence start, empty HCA list)."""
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


def small_wl(name, lengths, q_counts, H=64, dtype="bf16", k=64, W=128, m=4, m_hca=128, W_hca=0,
             codeset=synth.E2M1_ALL_CODES, seed=77):
    return synth.Workload(name, list(lengths), [L - c for L, c in zip(lengths, q_counts)], H=H,
                          dtype=dtype, k=k, W=W, m=m, m_hca=m_hca, W_hca=W_hca, codeset=codeset, seed=seed)


WORKLOADS = {
    "decode_fp32_t4096_h8": lambda: synth.decode_t4096_fp32(),
    "decode_bf16_ragged": lambda: small_wl("decode_bf16_ragged", [1, 3, 130, 517, 1030, 2049, 4099],
                                           [1] * 7, k=64, seed=11),
    "prefill_bf16_chunks": lambda: small_wl("prefill_bf16_chunks", [700, 1500], [37, 100], k=32,
                                            W=64, seed=12),
    "decode_bf16_ties": lambda: small_wl("decode_bf16_ties", [3001, 2998, 4097, 5003], [1] * 4, k=50,
                                         codeset=synth.E2M1_TIE_CODES, seed=13),
    "decode_fp32_k1_h24": lambda: small_wl("decode_fp32_k1_h24", [333, 1024], [2, 3], H=24,
                                           dtype="f32", k=1, W=5, m=3, m_hca=16, seed=14),
    # fp32 head counts that fill a thread's outputs unevenly (5 heads: 640
    # outputs over 256 threads) and beyond the staged-query limit (100 > 64)
    "decode_fp32_h5": lambda: small_wl("decode_fp32_h5", [70, 517, 1030], [1, 2, 1], H=5, dtype="f32", k=40,
                                       W=96, m=4, m_hca=32, W_hca=16, seed=16),
    "decode_fp32_h100": lambda: small_wl("decode_fp32_h100", [900, 260], [1, 3], H=100, dtype="f32", k=48,
                                         W=64, m=4, m_hca=16, seed=17),
    "decode_bf16_kbig_whca": lambda: small_wl("decode_bf16_kbig_whca", [200, 900], [1, 4], H=32, k=4000,
                                              W=200, m=4, m_hca=64, W_hca=64, seed=15),
    "prefill_bf16_ties": lambda: small_wl("prefill_bf16_ties", [5000, 9001], [64, 200], k=128,
                                          codeset=synth.E2M1_TIE_CODES, seed=18),
    # 635 prefill queries over three sequences: HCA serves two rows per workgroup,
    # with pairs across sequence boundaries, rows whose visible counts differ by
    # one, and an unpaired last row
    "prefill_bf16_pairs": lambda: small_wl("prefill_bf16_pairs", [2000, 1500, 900], [301, 256, 78], k=64, W=64,
                                           m_hca=32, seed=19),
}


def _params(wl):
    from long_context_compressed_05_amd.step import Params
    return Params(H=wl.H, d=wl.d, m=wl.m, k=wl.k, W=wl.W, m_hca=wl.m_hca, W_hca=wl.W_hca)


def _run_path(wl, host):
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    idx, co, cl, ho, hl = layer.attend(dq["q"], dq["qc"], dq["qs"], dq["w"])
    torch.cuda.synchronize()
    return layer, (P.torch_to_np(idx), P.torch_to_np(co), P.torch_to_np(cl), P.torch_to_np(ho),
                   P.torch_to_np(hl))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("m", [1, 3, 4, 16, 48, 64, 128])
def test_compress_parity(dtype, m):
    csa = _lib()
    wl = small_wl("compress", [5, 130, 517, 1030, 2049], [1] * 5, dtype=dtype, m=m, seed=21)
    host = synth.make_inputs(wl)
    from long_context_compressed_05_amd.step import to_device
    d = to_device({k: host[k] for k in ("kv", "z", "tok_off")})
    P_b = [L // m for L in wl.lengths]
    pool_off = synth.offsets(P_b)
    out = torch.empty((int(pool_off[-1]), 2, wl.d), dtype=d["kv"].dtype, device="cuda")
    csa.csa_compress(d["kv"], d["z"], d["tok_off"], torch.from_numpy(pool_off).cuda(), max(wl.lengths), m, out)
    torch.cuda.synchronize()
    got = P.torch_to_np(out)
    for b in range(wl.B):
        t0, t1 = int(host["tok_off"][b]), int(host["tok_off"][b + 1])
        want = oracle.pool(host["kv"][t0:t1], host["z"][t0:t1], m).reshape(-1, 2, wl.d)
        P.check_close(got[pool_off[b]:pool_off[b + 1]], want, dtype, f"pooled rows of sequence {b}")
        # one rounding of an fp32 result: within 2^-8 relative (+ tiny) of the exact value
        g = P.as_f64(got[pool_off[b]:pool_off[b + 1]])
        bound = (2.0 ** -8 if dtype == "bf16" else 2.0 ** -20) * np.abs(want) + 1e-6
        assert np.all(np.abs(g - want) <= bound)


@pytest.mark.parametrize("dtype,m,m_hca", [("f32", 4, 128), ("bf16", 4, 128), ("bf16", 32, 64), ("bf16", 4, 40)])
def test_cache_append_builds_the_bulk_caches(dtype, m, m_hca):
    """Caches grown by ragged appends (prefill chunks, single decode tokens,
    sequences with nothing new; decode-sized steps take the one-launch path
    that issues all loads first, steps of at most 64 tokens the one-launch
    workgroup-per-sequence path, longer ones two kernels) equal the raw rows and the bulk
    pooling of the whole sequences: raw rows and pooled rows bit for bit (the
    same pooling arithmetic), pooled rows within one rounding of the oracle's
    exact pooling, the completed blocks' indexer keys bit for bit equal to the
    oracle's MXFP4 encoding of their vectors, the tail ring holding the latest
    tokens' logits, and the lengths advanced.  m = 32 makes the CSA blocks
    long too (pooled by channel-slice workgroups in the multi-kernel path);
    m' = 40 ends every HCA block with a segment of 8 rows."""
    csa = _lib()
    ring = m_hca
    wl = small_wl("append", [1, 131, 517, 1030, 2050], [1] * 5, dtype=dtype, m=m, m_hca=m_hca, seed=23)
    host = synth.make_inputs(wl)
    B, L = wl.B, np.array(wl.lengths)
    es = torch.float32 if dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(5)
    # the append schedule: two single-token steps for every sequence, then chunks per
    # sequence, ragged, with zero-length and single-token steps
    steps = []
    done = np.zeros(B, dtype=np.int64)
    for _ in range(2):
        n = np.minimum(L - done, 1)
        steps.append(n)
        done += n
    while (done < L).any():
        n = np.minimum(L - done, rng.choice([0, 1, 1, 3, 64, 200, 777], size=B))
        if n.sum() == 0:
            n = np.minimum(L - done, 1)
        steps.append(n)
        done += n
    cap = L + 5
    tok_off = synth.offsets(list(cap))
    pool_off, hpool_off = synth.offsets(list(cap // m)), synth.offsets(list(cap // m_hca))
    dev = "cuda"
    # the indexer vector of every CSA block of each sequence (64 elements, the KV dtype)
    kdim = 64
    kf = [rng.standard_normal((int(l) // m, kdim)).astype(np.float32) for l in L]
    if dtype == "bf16":
        kf = [((v.view(np.uint32).astype(np.uint64) + 0x7FFF + ((v.view(np.uint32) >> 16) & 1)) >> 16)
              .astype(np.uint16) for v in kf]
    k_codes = torch.zeros((int(pool_off[-1]), kdim // 2), dtype=torch.uint8, device=dev)
    k_scales = torch.zeros((int(pool_off[-1]), kdim // 32), dtype=torch.uint8, device=dev)
    kv_raw = torch.zeros((int(tok_off[-1]), 2, wl.d), dtype=es, device=dev)
    pooled = torch.zeros((int(pool_off[-1]), 2, wl.d), dtype=es, device=dev)
    hpooled = torch.zeros((int(hpool_off[-1]), 2, wl.d), dtype=es, device=dev)
    z_tail = torch.zeros((B, ring, 2, wl.d), dtype=es, device=dev)
    length = torch.zeros(B, dtype=torch.int64, device=dev)
    from long_context_compressed_05_amd.step import to_device
    dd = to_device({"kv": host["kv"], "z": host["z"]})
    kv, z = dd["kv"], dd["z"]
    t_tok, t_pool, t_hpool = (torch.from_numpy(a).to(dev) for a in (tok_off, pool_off, hpool_off))
    done[:] = 0
    saw_step = saw_short = saw_long = False
    for n in steps:
        rows = np.concatenate([np.arange(host["tok_off"][b] + done[b], host["tok_off"][b] + done[b] + n[b])
                               for b in range(B)]).astype(np.int64)
        r = torch.from_numpy(rows).to(dev)
        new_off = torch.from_numpy(synth.offsets(list(n))).to(dev)
        c0, c1 = done // m, (done + n) // m
        kv_np = np.concatenate([kf[b][c0[b]:c1[b]] for b in range(B)]) if (c1 > c0).any() else kf[0][:0]
        kvec = to_device({"k": np.ascontiguousarray(kv_np.reshape(-1, kdim) if kv_np.size else
                                                    np.zeros((1, kdim), kf[0].dtype))})["k"]
        kvec_off = torch.from_numpy(synth.offsets(list(c1 - c0))).to(dev)
        csa.csa_cache_append(kv[r].contiguous(), z[r].contiguous(), new_off, int(n.max()), t_tok, length, kv_raw,
                             z_tail, t_pool, m, pooled, t_hpool, m_hca, hpooled, kvec_off=kvec_off, kvec=kvec,
                             k_codes=k_codes, k_scales=k_scales)
        saw_step |= 0 < int(n.max()) <= (8 if dtype == "bf16" else 4)
        saw_short |= (8 if dtype == "bf16" else 4) < int(n.max()) <= 64
        saw_long |= int(n.max()) > 64
        done += n
    assert (saw_step or m > 8) and saw_short and saw_long, "the schedule should take every append path"
    torch.cuda.synchronize()
    assert P.torch_to_np(length).tolist() == L.tolist()
    # the bulk path over the whole sequences, for comparison
    bulk = torch.empty((int(synth.offsets([l // m for l in L])[-1]), 2, wl.d), dtype=es, device=dev)
    hbulk = torch.empty((int(synth.offsets([l // m_hca for l in L])[-1]), 2, wl.d), dtype=es, device=dev)
    bp, hbp = synth.offsets([l // m for l in L]), synth.offsets([l // m_hca for l in L])
    csa.csa_compress(kv, z, torch.from_numpy(host["tok_off"]).to(dev), torch.from_numpy(bp).to(dev), int(L.max()),
                     m, bulk)
    csa.csa_compress(kv, z, torch.from_numpy(host["tok_off"]).to(dev), torch.from_numpy(hbp).to(dev), int(L.max()),
                     m_hca, hbulk)
    torch.cuda.synchronize()
    raw_np, pooled_np, hpooled_np = P.torch_to_np(kv_raw), P.torch_to_np(pooled), P.torch_to_np(hpooled)
    kv_np, z_np, bulk_np, hbulk_np = P.torch_to_np(kv), P.torch_to_np(z), P.torch_to_np(bulk), P.torch_to_np(hbulk)
    tail_np = P.torch_to_np(z_tail)
    for b in range(B):
        t0 = int(host["tok_off"][b])
        np.testing.assert_array_equal(raw_np[tok_off[b]:tok_off[b] + L[b]], kv_np[t0:t0 + L[b]])
        for mm, got, off, ref, roff in ((m, pooled_np, pool_off, bulk_np, bp), (m_hca, hpooled_np, hpool_off,
                                                                                 hbulk_np, hbp)):
            nb = L[b] // mm
            g = got[off[b]:off[b] + nb]
            np.testing.assert_array_equal(g, ref[roff[b]:roff[b] + nb], err_msg=f"seq {b} m={mm}")
            want = oracle.pool(host["kv"][t0:t0 + L[b]], host["z"][t0:t0 + L[b]], mm).reshape(-1, 2, wl.d)
            bound = (2.0 ** -8 if dtype == "bf16" else 2.0 ** -20) * np.abs(want) + 1e-6
            assert np.all(np.abs(P.as_f64(g) - want) <= bound), f"seq {b} m={mm} vs the oracle"
        for p in range(max(0, L[b] - ring), L[b]):
            np.testing.assert_array_equal(tail_np[b, p % ring], z_np[t0 + p], err_msg=f"tail slot of token {p}")
        # the completed blocks' keys against the oracle's encoding of their vectors
        nb = L[b] // m
        if nb:
            want_c, want_s = oracle.mxfp4_quantize(kf[b])
            np.testing.assert_array_equal(P.torch_to_np(k_codes)[pool_off[b]:pool_off[b] + nb], want_c,
                                          err_msg=f"key codes of sequence {b}")
            np.testing.assert_array_equal(P.torch_to_np(k_scales)[pool_off[b]:pool_off[b] + nb], want_s,
                                          err_msg=f"key scales of sequence {b}")


def _quant_inputs(dtype, rows, dim, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, dim)) * np.exp(rng.uniform(-8, 8, size=(rows, 1)))).astype(np.float32)
    # special blocks: zeros, exact midpoints and saturation, tiny (subnormal) and huge magnitudes
    x[0] = 0.0
    mids = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5, 7.9],
                    np.float32)
    x[1, :32] = np.resize(mids, 32) * np.float32(2.0 ** -40)
    x[2, :32] = np.float32(1e-42)
    x[3, :32] = np.resize(mids, 32) * np.float32(2.0 ** 100)
    x[4, :] = -x[4, :]
    if dtype == "bf16":  # the same values rounded to bf16 (nearest even), as bit patterns
        u = x.view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,dim", [(1, 32), (37, 64), (300, 256), (4096, 64)])
def test_mxfp4_quantize_bit_exact(dtype, rows, dim):
    csa = _lib()
    x = np.ascontiguousarray(_quant_inputs(dtype, max(rows, 5), dim, seed=rows + dim)[:rows])
    from long_context_compressed_05_amd.step import to_device
    xd = to_device({"x": x})["x"]
    codes, scales = csa.csa_mxfp4_quantize(xd)
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp4_quantize(x)
    np.testing.assert_array_equal(P.torch_to_np(scales), want_s)
    np.testing.assert_array_equal(P.torch_to_np(codes), want_c)


def test_mxfp4_quantize_then_index_matches_the_oracle_pipeline():
    """fp32 indexer queries and keys quantised on the GPU and selected with
    csa_index_topk give the same indices as the oracle's quantiser followed by
    its exact scores and full sort."""
    csa = _lib()
    rng = np.random.default_rng(9)
    lengths, k, m = [4096 + 3, 1031, 9000], 64, 4
    B = len(lengths)
    P_b = [L // m for L in lengths]
    pool_off = synth.offsets(P_b)
    q = rng.standard_normal((B, 4, 64)).astype(np.float32)
    kf = rng.standard_normal((int(pool_off[-1]), 64)).astype(np.float32)
    w = np.array([[0.5, 1.0, 2.0, 1.0]] * B, np.float32)
    qc, qs = oracle.mxfp4_quantize(q)
    kc, ks = oracle.mxfp4_quantize(kf)
    from long_context_compressed_05_amd.step import to_device
    d = to_device({"q": q, "k": kf, "w": w, "pool_off": pool_off})
    gqc, gqs = csa.csa_mxfp4_quantize(d["q"])
    gkc, gks = csa.csa_mxfp4_quantize(d["k"])
    batch = csa.Batch.from_host(synth.offsets(lengths), np.arange(B + 1), np.array(lengths) - 1)
    idx = csa.csa_index_topk(batch, d["pool_off"], max(P_b), m, k, gqc, gqs, d["w"], gkc, gks)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(P.torch_to_np(gqc), qc)
    np.testing.assert_array_equal(P.torch_to_np(gkc), kc)
    got = P.torch_to_np(idx)
    for b in range(B):
        p0, p1 = int(pool_off[b]), int(pool_off[b + 1])
        S, exact = oracle.index_scores(qc[b], qs[b], w[b], kc[p0:p1], ks[p0:p1])
        assert exact.all()
        want = oracle.topk(S, k)
        np.testing.assert_array_equal(got[b], want)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_index_topk_bit_exact(name):
    csa = _lib()
    wl = WORKLOADS[name]()
    host = synth.make_inputs(wl, raw=False)
    from long_context_compressed_05_amd.step import to_device
    d = to_device({k: host[k] for k in ("qc", "qs", "w", "kc", "ks", "pool_off")})
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    max_pool = int(np.diff(host["pool_off"]).max())
    ws = csa.Workspace()
    idx = csa.csa_index_topk(batch, d["pool_off"], max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"],
                             d["ks"], ws=ws)
    got = P.torch_to_np(idx)
    seqs = P.row_seq(host)
    for row in range(wl.n_q):
        want = P.oracle_topk_row(host, wl, row, seqs[row], wl.k, wl.m)
        assert np.array_equal(got[row], want), f"row {row} (seq {seqs[row]}, t={host['q_pos'][row]})"
    # the library leaves its workspace zero-filled; a second call is bit-identical
    assert int(torch.count_nonzero(ws.buf[:4096 * 4 * wl.n_q])) == 0
    idx2 = csa.csa_index_topk(batch, d["pool_off"], max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"],
                              d["ks"], ws=ws)
    assert torch.equal(idx, idx2)


@pytest.mark.parametrize("name", ["decode_fp32_t4096_h8", "decode_bf16_ragged", "prefill_bf16_chunks",
                                  "decode_fp32_k1_h24", "decode_bf16_kbig_whca"])
def test_sparse_attn_stagewise(name):
    """Attention on given inputs: a generated pooled cache and the oracle's indices."""
    csa = _lib()
    wl = WORKLOADS[name]()
    host = synth.make_inputs(wl)
    pooled = synth.pooled_like(wl, wl.m)
    seqs = P.row_seq(host)
    idx = np.stack([P.oracle_topk_row(host, wl, r, seqs[r], wl.k, wl.m) for r in range(wl.n_q)])
    from long_context_compressed_05_amd.step import to_device
    d = to_device({"kv": host["kv"], "q": host["q"], "pooled": pooled, "idx": idx,
                   "pool_off": host["pool_off"]})
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    scale = 1 / math.sqrt(wl.d)
    out, lse = csa.csa_sparse_attn(batch, d["pool_off"], d["q"], d["pooled"], d["kv"], d["idx"], wl.W, scale)
    got, gl = P.torch_to_np(out), P.torch_to_np(lse)
    want = np.zeros(got.shape)
    wl_ = np.zeros(gl.shape)
    for r in range(wl.n_q):
        b = seqs[r]
        (t0, t1), (p0, p1), _ = P.seq_slices(host, b)
        want[r], wl_[r] = oracle.csa_attend_given(host["kv"][t0:t1], pooled[p0:p1], idx[r], host["q"][r],
                                                 int(host["q_pos"][r]), wl.W, scale)
    P.check_close(got, want, wl.dtype, "csa output")
    P.check_close(gl, wl_, "f32" if wl.dtype == "f32" else "bf16", "csa lse")


@pytest.mark.parametrize("name", ["decode_fp32_t4096_h8", "decode_bf16_ragged", "prefill_bf16_chunks",
                                  "decode_fp32_k1_h24", "decode_bf16_kbig_whca", "prefill_bf16_pairs"])
def test_hca_attn_stagewise(name):
    csa = _lib()
    wl = WORKLOADS[name]()
    host = synth.make_inputs(wl)
    hpooled = synth.pooled_like(wl, wl.m_hca)
    seqs = P.row_seq(host)
    from long_context_compressed_05_amd.step import to_device
    d = to_device({"kv": host["kv"], "q": host["q"], "hpooled": hpooled, "hpool_off": host["hpool_off"]})
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    scale = 1 / math.sqrt(wl.d)
    max_hpool = int(np.diff(host["hpool_off"]).max())
    out, lse = csa.hca_attn(batch, d["hpool_off"], max_hpool, wl.m_hca, d["q"], d["hpooled"], d["kv"], wl.W_hca,
                            scale)
    got, gl = P.torch_to_np(out), P.torch_to_np(lse)
    want = np.zeros(got.shape)
    wl_ = np.zeros(gl.shape)
    for r in range(wl.n_q):
        b = seqs[r]
        t0, t1 = int(host["tok_off"][b]), int(host["tok_off"][b + 1])
        h0, h1 = int(host["hpool_off"][b]), int(host["hpool_off"][b + 1])
        want[r], wl_[r] = oracle.hca_attend_given(host["kv"][t0:t1], hpooled[h0:h1], host["q"][r],
                                                 int(host["q_pos"][r]), wl.m_hca, wl.W_hca, scale)
    P.check_close(got, want, wl.dtype, "hca output")
    P.check_close(gl, wl_, "f32" if wl.dtype == "f32" else "bf16", "hca lse")


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_end_to_end(name):
    """Raw rows -> compress -> index/top-k -> CSA and HCA, against the oracle
    pooling in fp64 from the same raw rows."""
    _lib()
    wl = WORKLOADS[name]()
    host = synth.make_inputs(wl)
    _, (idx, co, cl, ho, hl) = _run_path(wl, host)
    seqs = P.row_seq(host)
    scale = 1 / math.sqrt(wl.d)
    want_co, want_cl = np.zeros(co.shape), np.zeros(cl.shape)
    want_ho, want_hl = np.zeros(ho.shape), np.zeros(hl.shape)
    for r in range(wl.n_q):
        b = seqs[r]
        (t0, t1), (p0, p1), _ = P.seq_slices(host, b)
        t = int(host["q_pos"][r])
        o, l, i = oracle.csa_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m, wl.W, wl.k, scale,
                                   host["qc"][r], host["qs"][r], host["w"][r], host["kc"][p0:p1],
                                   host["ks"][p0:p1])
        assert np.array_equal(idx[r], i), f"top-k of row {r}"
        want_co[r], want_cl[r] = o, l
        want_ho[r], want_hl[r] = oracle.hca_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m_hca,
                                                  wl.W_hca, scale)
    P.check_close(co, want_co, wl.dtype, "csa output")
    P.check_close(cl, want_cl, "f32" if wl.dtype == "f32" else "bf16", "csa lse")
    P.check_close(ho, want_ho, wl.dtype, "hca output")
    P.check_close(hl, want_hl, "f32" if wl.dtype == "f32" else "bf16", "hca lse")


def test_deterministic_repeat():
    _lib()
    wl = WORKLOADS["decode_bf16_ties"]()
    host = synth.make_inputs(wl)
    _, a = _run_path(wl, host)
    _, b = _run_path(wl, host)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("lengths,k,codeset", [
    ([160001, 200003, 150002], 1000, synth.E2M1_ALL_CODES),   # 8 histogram replicas, bitmap ordering
    ([160001, 200003], 777, synth.E2M1_TIE_CODES),             # the same with heavy ties
    ([3200003], 4096, synth.E2M1_ALL_CODES),                   # visible range beyond the LDS bitmap: bitonic
])
def test_index_topk_large_ranges(lengths, k, codeset):
    csa = _lib()
    wl = small_wl("index_large", lengths, [1] * len(lengths), k=k, codeset=codeset, seed=31)
    host = synth.make_inputs(wl, raw=False)
    from long_context_compressed_05_amd.step import to_device
    d = to_device({kk: host[kk] for kk in ("qc", "qs", "w", "kc", "ks", "pool_off")})
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    max_pool = int(np.diff(host["pool_off"]).max())
    idx = csa.csa_index_topk(batch, d["pool_off"], max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"], d["ks"])
    got = P.torch_to_np(idx)
    seqs = P.row_seq(host)
    for row in range(wl.n_q):
        want = P.oracle_topk_row(host, wl, row, seqs[row], wl.k, wl.m)
        assert np.array_equal(got[row], want), f"row {row}"


def _index_rows(wl, host, rows):
    csa = _lib()
    from long_context_compressed_05_amd.step import to_device
    d = to_device({kk: host[kk] for kk in ("qc", "qs", "w", "kc", "ks", "pool_off")})
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    max_pool = int(np.diff(host["pool_off"]).max())
    ws = csa.Workspace()
    idx = csa.csa_index_topk(batch, d["pool_off"], max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"],
                             d["ks"], ws=ws)
    got = P.torch_to_np(idx)
    seqs = P.row_seq(host)
    for row in rows:
        want = P.oracle_topk_row(host, wl, row, seqs[row], wl.k, wl.m)
        assert np.array_equal(got[row], want), f"row {row} (seq {seqs[row]}, t={host['q_pos'][row]})"
    if batch.max_q_per_seq >= 16:  # the prefill path's workspace is all candidate bitmaps, left zero
        assert int(torch.count_nonzero(ws.buf)) == 0, "the workspace is not left zero-filled"
    # reused without clearing, the workspace gives the same selection
    idx2 = csa.csa_index_topk(batch, d["pool_off"], max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"],
                              d["ks"], ws=ws)
    assert np.array_equal(P.torch_to_np(idx2), got), "a second call on the same workspace differs"
    return got


def test_prefill_topk_equal_keys():
    """Every indexer key equal: every visible score of a query ties, the
    sampled threshold passes all of them, the candidates overflow the per-query
    buffer and the exact path over all keys runs; the top-k is the first k
    visible indices."""
    wl = small_wl("prefill_equal_keys", [12001, 3000], [40, 17], k=256, seed=19)
    host = synth.make_inputs(wl, raw=False)
    host["kc"][:] = 0x22
    host["ks"][:] = 127
    got = _index_rows(wl, host, range(wl.n_q))
    assert np.array_equal(got[0], np.arange(wl.k))


def test_prefill_topk_full_size_sampled():
    """The 4096-query chunk on a 65,536-token cache (17,408 pooled keys, top-512)
    in the launch configuration the benchmark times; 96 sampled rows (first,
    last and spread) against the oracle, bit for bit."""
    wl = synth.prefill_4k_on_64k()
    host = synth.make_inputs(wl, raw=False)
    rows = sorted(set([0, 1, wl.n_q - 1] + list(np.random.default_rng(7).choice(wl.n_q, 93, replace=False))))
    _index_rows(wl, host, rows)



def test_prefill_topk_two_sequences_mixed_batches():
    """4096 queries over two sequences (16,384 and 12,000 cached tokens, the
    second sequence's queries starting at a position off a block boundary):
    up to 4,608 pooled keys per sequence, so the scoring workgroups hold 1,152
    keys (9 tiles per wave): a first batch of 8 tiles that every query of a
    block sees whole (the straight-line path), a last batch of 1 (the
    per-tile path), and blocks at each query's visible edge.  The first and
    last rows of each sequence and 250 spread rows against the oracle, bit for
    bit."""
    wl = small_wl("prefill_mixed_batches", [16384 + 2048, 12001 + 2048], [2048, 2048], k=256, seed=63)
    host = synth.make_inputs(wl, raw=False)
    q_off = host["q_off"]
    ends = [0, int(q_off[1]) - 1, int(q_off[1]), wl.n_q - 1]
    rows = sorted(set(ends + list(np.random.default_rng(9).choice(wl.n_q, 250, replace=False))))
    _index_rows(wl, host, rows)


@pytest.mark.parametrize("codeset", [synth.E2M1_ALL_CODES, synth.E2M1_TIE_CODES])
def test_prefill_topk_long_caches(codeset):
    """Prefill batches on long caches: up to 50,000 pooled keys per query, so a
    query's bitmap has more than 16 groups of 64 words (the selection reads its
    words in several batches), the threshold sample stride exceeds 16 and the
    sample fills its 2048 slots.  With tie-heavy codes the candidates
    overflow and the exact path over all visible keys runs at that length.
    The first and last row of each sequence and every fourth row against the
    oracle, bit for bit."""
    wl = small_wl("prefill_long", [200003, 140001], [32, 20], k=512, codeset=codeset, seed=71)
    host = synth.make_inputs(wl, raw=False)
    q_off = host["q_off"]
    rows = sorted(set([0, int(q_off[1]) - 1, int(q_off[1]), wl.n_q - 1] + list(range(0, wl.n_q, 4))))
    _index_rows(wl, host, rows)

_MANY_ROWS = [1, 2, 3, 5, 17, 64, 100, 127, 128, 129, 200, 255, 256, 257, 300, 511, 512, 513, 700, 1000,
              30001, 1030, 1500, 2049, 2500, 3001, 3500, 4099, 4500, 5003, 32000, 5555, 6000, 6100, 640, 90, 7,
              2222, 999, 32771]

_SHARED_TAILS = [1, 5, 77, 130, 300, 517, 1000, 2049, 3001, 4099, 5003, 6000, 7, 90, 640, 999, 2222, 1500, 2500,
                 3500, 4500, 5555, 6100, 700, 200, 255, 256, 257, 511, 512, 513, 1030, 33, 64, 100, 127, 128, 129,
                 17]

FUSED_CASES = {
    "decode_bf16_ragged": lambda: small_wl("decode_bf16_ragged", [1, 3, 130, 517, 1030, 2049, 4099], [1] * 7,
                                           k=64, seed=11),
    "decode_bf16_ties": lambda: small_wl("decode_bf16_ties", [3001, 2998, 4097, 5003], [1] * 4, k=50,
                                         codeset=synth.E2M1_TIE_CODES, seed=13),
    "decode_bf16_h32_whca": lambda: small_wl("decode_bf16_h32_whca", [200, 900, 70001], [1] * 3, H=32, k=700,
                                             W=200, m=4, m_hca=64, W_hca=64, seed=15),
    "decode_bf16_long": lambda: small_wl("decode_bf16_long", [160001, 200003, 150002, 99999], [1] * 4, k=1024,
                                         seed=16),
    # one long row: 74 chunks of 1024, 4440 list positions (the 24-slot selection)
    "decode_bf16_single_300k": lambda: small_wl("decode_bf16_single_300k", [300001], [1], k=1024, seed=18),
    # 40 rows, two of them long: the plan has 7 chunks of 1280 per row (280 >
    # 256 first-round units), so rows 30 and 39 have their last chunk handed
    # out by ticket, and the ticket units are numbered over the row table
    # (rows without HCA rows get no split and merge zero partials)
    "decode_bf16_many_rows": lambda: small_wl("decode_bf16_many_rows", _MANY_ROWS, [1] * 40, k=200, seed=19),
    # the same rows with an HCA window: every row keeps all of its HCA splits
    "decode_bf16_many_rows_whca": lambda: small_wl("decode_bf16_many_rows_whca", _MANY_ROWS, [1] * 40, k=200,
                                                   m_hca=64, W_hca=64, seed=20),
}


def _concentrate(host, n_top=2600):
    """Gives the first n_top pooled entries of every sequence one and the same
    indexer key aligned with that sequence's query (code +-6 with the sign of
    the w-weighted head sum of q, scale 2^2), so that they are equal and hold
    the whole top-k: single score chunks then hold more selected entries than
    their candidate lists can, and the equal keys are ranked by index."""
    kc, ks = host["kc"].copy(), host["ks"].copy()
    for b in range(len(host["pool_off"]) - 1):
        row = int(host["q_off"][b])
        qv = np.zeros(64)
        for h in range(4):
            for c in range(64):
                byte = int(host["qc"][row, h, c // 2])
                code = byte & 15 if c % 2 == 0 else byte >> 4
                qv[c] += (float(host["w"][row, h]) * oracle.e2m1_value(code)
                          * oracle.e8m0_value(int(host["qs"][row, h, c // 32])))
        nib = np.where(qv >= 0, 0x7, 0xF).astype(np.uint8)
        packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
        p0, p1 = int(host["pool_off"][b]), int(host["pool_off"][b + 1])
        e = min(p0 + n_top, p1)
        kc[p0:e] = packed
        ks[p0:e] = 127 + 2
    host["kc"], host["ks"] = kc, ks
    return host


# name -> (workload, host post-processing or None, whether the exact fallback must be taken)
FUSED_EXTRA = {
    "decode_bf16_concentrated": (lambda: small_wl("decode_bf16_concentrated", [40001, 30002], [1, 1], k=1024,
                                                  seed=17), _concentrate, True),
}


@pytest.mark.parametrize("name", list(FUSED_CASES) + list(FUSED_EXTRA))
def test_fused_decode_matches_oracle_and_separate_calls(name):
    """The one-launch decode step gives the oracle's top-k bit for bit, outputs
    within tolerance, and the separate calls' top-k; repeated launches on the
    same workspace are bit-identical.  The concentrated case drives the
    selection into its exact fallback and checks that it was taken."""
    csa = _lib()
    post, want_fallback = None, False
    if name in FUSED_EXTRA:
        make, post, want_fallback = FUSED_EXTRA[name]
        wl = make()
    else:
        wl = FUSED_CASES[name]()
    host = synth.make_inputs(wl)
    if post is not None:
        host = post(host)
    layer, (idx_s, co_s, cl_s, ho_s, hl_s) = _run_path(wl, host)
    from long_context_compressed_05_amd.step import to_device
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    outs = [layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"]) for _ in range(3)]
    layer.check_fused()
    torch.cuda.synchronize()
    n_fallback = csa.csa_hca_decode_fallbacks(layer.ws_fused)
    if want_fallback:
        assert n_fallback == 3 * wl.n_q, f"expected every row of every launch to take the fallback, got {n_fallback}"
    res = [[P.torch_to_np(t) for t in o] for o in outs]
    idx, co, cl, ho, hl = res[0]
    for other in res[1:]:
        for x, y in zip(res[0], other):
            assert np.array_equal(x, y), "fused decode is not deterministic"
    assert np.array_equal(idx, idx_s), "fused top-k differs from csa_index_topk"
    seqs = P.row_seq(host)
    scale = 1 / math.sqrt(wl.d)
    want_co, want_cl = np.zeros(co.shape), np.zeros(cl.shape)
    want_ho, want_hl = np.zeros(ho.shape), np.zeros(hl.shape)
    for r in range(wl.n_q):
        b = seqs[r]
        (t0, t1), (p0, p1), _ = P.seq_slices(host, b)
        t = int(host["q_pos"][r])
        o, l, i = oracle.csa_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m, wl.W, wl.k, scale,
                                   host["qc"][r], host["qs"][r], host["w"][r], host["kc"][p0:p1], host["ks"][p0:p1])
        assert np.array_equal(idx[r], i), f"top-k of row {r}"
        want_co[r], want_cl[r] = o, l
        want_ho[r], want_hl[r] = oracle.hca_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m_hca,
                                                  wl.W_hca, scale)
    P.check_close(co, want_co, wl.dtype, "fused csa output")
    P.check_close(cl, want_cl, "bf16", "fused csa lse")
    P.check_close(ho, want_ho, wl.dtype, "fused hca output")
    P.check_close(hl, want_hl, "bf16", "fused hca lse")


def _full_size_decode(wl, rows, hca_rows):
    """Runs the benchmark's one-launch decode step on a full-size workload and
    the separate calls on the same inputs; checks the top-k of `rows` and the
    CSA outputs of `rows` against the oracle, the HCA outputs of `hca_rows`,
    and that both paths agree on every row."""
    csa = _lib()
    host = synth.make_inputs(wl)
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    idx, co, cl, ho, hl = [P.torch_to_np(t) for t in layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])]
    layer.check_fused()
    idx_s, co_s, cl_s, ho_s, hl_s = [P.torch_to_np(t) for t in layer.attend(dq["q"], dq["qc"], dq["qs"], dq["w"])]
    torch.cuda.synchronize()
    assert np.array_equal(idx, idx_s), "fused and separate top-k differ"
    P.check_close(co, P.as_f64(co_s), wl.dtype, "fused vs separate csa output")
    P.check_close(ho, P.as_f64(ho_s), wl.dtype, "fused vs separate hca output")
    seqs = P.row_seq(host)
    scale = 1 / math.sqrt(wl.d)
    for r in rows:
        b = seqs[r]
        (t0, t1), (p0, p1), _ = P.seq_slices(host, b)
        t = int(host["q_pos"][r])
        o, l, i = oracle.csa_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m, wl.W, wl.k, scale,
                                   host["qc"][r], host["qs"][r], host["w"][r], host["kc"][p0:p1], host["ks"][p0:p1])
        assert np.array_equal(idx[r], i), f"top-k of row {r}"
        P.check_close(co[r], o, wl.dtype, f"csa output of row {r}")
        P.check_close(cl[r], l, "bf16", f"csa lse of row {r}")
    for r in hca_rows:
        b = seqs[r]
        (t0, t1), _, _ = P.seq_slices(host, b)
        t = int(host["q_pos"][r])
        o, l = oracle.hca_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m_hca, wl.W_hca, scale)
        P.check_close(ho[r], o, wl.dtype, f"hca output of row {r}")
        P.check_close(hl[r], l, "bf16", f"hca lse of row {r}")


def test_decode_full_size_b4_t1m():
    """The benchmark workload: 4 sequences of 2^20 tokens, top-1024 of 262,144
    pooled entries, 8192 HCA entries, in the launch configuration bench.py
    times; every row against the oracle."""
    wl = synth.decode_b4_t1m()
    _full_size_decode(wl, range(wl.n_q), range(wl.n_q))


def test_decode_full_size_b16_t64k():
    """16 sequences of 65,536 tokens, top-512 of 16,384; every row's top-k and
    CSA output, HCA outputs of four rows."""
    wl = synth.decode_b16_t64k()
    _full_size_decode(wl, range(wl.n_q), [0, 5, 10, 15])


def test_decode_full_size_ragged_b32_sampled():
    """32 ragged sequences (log-uniform lengths up to 2^20, tails not a
    multiple of m) with tie-heavy indexer codes; sampled rows against the
    oracle, and the fused and separate paths agree on every row."""
    wl = synth.decode_ragged_b32()
    lens = np.array(wl.lengths)
    rows = sorted(set([int(np.argmin(lens)), int(np.argmax(lens)), 0, 7, 19, 31]))
    _full_size_decode(wl, rows, rows[:3])


# name -> (workload, prefix tokens T): sequence 0 holds the prefix; the others
# share its first T tokens (a long own suffix, a window across the prefix's
# end, the prefix alone)
SHARED_CASES = {
    "shared_t4096": (lambda: small_wl("decode_shared", [20003, 4096 + 9001, 4096 + 50, 4096], [1] * 4, k=256,
                                      seed=31), 4096),
    "shared_whca": (lambda: small_wl("decode_shared_whca", [9000, 2048 + 3000, 2048 + 20], [1] * 3, H=32, k=300,
                                     W=200, m_hca=64, W_hca=64, seed=32), 2048),
    "shared_long": (lambda: small_wl("decode_shared_long", [262147, 131072 + 4099, 131072 + 77, 131072 + 1030],
                                     [1] * 4, k=1024, seed=33), 131072),
    # a prefix of 4226 tokens: the CSA block 1056 (tokens 4224..4227) and the HCA block 33
    # (tokens 4224..4351) straddle its end, so each sharer's own caches pool them from
    # the prefix's tokens and its own
    "shared_straddle": (lambda: small_wl("decode_shared_straddle", [20003, 4226 + 5001, 4226 + 77, 4226 + 2],
                                         [1] * 4, k=256, seed=35), 4226),
    # 40 rows over one 8192-token prefix; the longest row's 16,384 pooled entries
    # give 7 chunks per row (280 > 256 first-round units): the compact form
    "shared_many_rows": (lambda: small_wl("decode_shared_many", [65539] + [8192 + v for v in _SHARED_TAILS],
                                          [1] * 40, k=200, seed=36), 8192),
}


def _share_prefix(host, wl, T):
    """Makes every sequence's first T tokens (and their indexer keys) equal to
    sequence 0's, so the logical sequences really share a prefix."""
    to, po = host["tok_off"], host["pool_off"]
    pT = T // wl.m
    for b in range(1, len(to) - 1):
        for name in ("kv", "z"):
            host[name][to[b]:to[b] + T] = host[name][to[0]:to[0] + T]
        for name in ("kc", "ks"):
            host[name][po[b]:po[b] + pT] = host[name][po[0]:po[0] + pT]
    return host


@pytest.mark.parametrize("name", list(SHARED_CASES))
def test_shared_prefix_decode_is_bit_identical_to_contiguous_caches(name):
    """csa_hca_decode_shared over caches where sequences 1.. store only their
    rows after a prefix held by sequence 0 gives exactly the outputs of
    csa_hca_decode over the same logical sequences stored contiguously, and
    the oracle's top-k and outputs on sampled rows."""
    csa = _lib()
    make, T = SHARED_CASES[name]
    wl = make()
    host = _share_prefix(synth.make_inputs(wl), wl, T)
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    want = [P.torch_to_np(t) for t in layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])]
    layer.check_fused()
    # the shared layout: sequence 0 whole, the others from the prefix's end on
    to, po, ho = host["tok_off"], host["pool_off"], host["hpool_off"]
    B = len(to) - 1
    cut = [(0, 0, 0)] + [(T, T // wl.m, T // wl.m_hca)] * (B - 1)
    segs = [((int(to[b]) + c[0], int(to[b + 1])), (int(po[b]) + c[1], int(po[b + 1])),
             (int(ho[b]) + c[2], int(ho[b + 1]))) for b, c in enumerate(cut)]
    for s in segs:
        assert all(a <= e for a, e in s), "a sequence shorter than the prefix"

    def cat(t, which):
        return torch.cat([t[s[which][0]:s[which][1]] for s in segs]).contiguous()

    def offs(which):
        return np.concatenate([[0], np.cumsum([s[which][1] - s[which][0] for s in segs])]).astype(np.int64)
    kv2, pooled2, hpooled2 = cat(layer.kv, 0), cat(layer.pooled, 1), cat(layer.hpooled, 2)
    kc2, ks2 = cat(layer.kc, 1), cat(layer.ks, 1)
    tok2, pool2, hpool2 = offs(0), offs(1), offs(2)
    batch2 = csa.Batch.from_host(tok2, host["q_off"], host["q_pos"])
    pre_seq = torch.tensor([-1] + [0] * (B - 1), dtype=torch.int32, device="cuda")
    pre_tok = torch.tensor([0] + [T] * (B - 1), dtype=torch.int64, device="cuda")
    p = layer.p
    ws = csa.Workspace()
    got = [P.torch_to_np(t) for t in csa.csa_hca_decode_shared(
        batch2, pre_seq, pre_tok, torch.from_numpy(pool2).cuda(), layer.max_pool, torch.from_numpy(hpool2).cuda(),
        layer.max_hpool, p.m, p.m_hca, p.k, p.W, p.W_hca, p.sm_scale, dq["qc"], dq["qs"], dq["w"], kc2, ks2, dq["q"],
        pooled2, hpooled2, kv2, ws=ws)]
    csa.csa_hca_decode_check(batch2, ws)
    torch.cuda.synchronize()
    for what, x, y in zip(("idx", "csa_out", "csa_lse", "hca_out", "hca_lse"), got, want):
        assert np.array_equal(x, y), f"{what} differs from the contiguous layout"
    # the oracle on the logical sequences, sharer rows first
    idx, co, cl, hop, hl = got
    seqs = P.row_seq(host)
    scale = 1 / math.sqrt(wl.d)
    for r in [1, B - 1]:
        b = seqs[r]
        (t0, t1), (p0, p1), _ = P.seq_slices(host, b)
        t = int(host["q_pos"][r])
        o, l, i = oracle.csa_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m, wl.W, wl.k, scale,
                                   host["qc"][r], host["qs"][r], host["w"][r], host["kc"][p0:p1], host["ks"][p0:p1])
        assert np.array_equal(idx[r], i), f"top-k of row {r}"
        P.check_close(co[r:r + 1], o[None], wl.dtype, f"csa output of row {r}")
        ho_r, hl_r = oracle.hca_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m_hca, wl.W_hca, scale)
        P.check_close(hop[r:r + 1], ho_r[None], wl.dtype, f"hca output of row {r}")


def test_shared_prefix_entry_without_prefixes_equals_plain_decode():
    """csa_hca_decode_shared with no prefix (-1, or a holder out of range, or
    the sequence itself, or T = 0) reads each sequence's own rows only and
    gives csa_hca_decode's outputs bit for bit."""
    csa = _lib()
    wl = small_wl("decode_shared_none", [3001, 2998, 4097, 5003], [1] * 4, k=128, seed=34)
    host = synth.make_inputs(wl)
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    want = [P.torch_to_np(t) for t in layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])]
    layer.check_fused()
    p = layer.p
    pre_seq = torch.tensor([-1, 7, 2, 0], dtype=torch.int32, device="cuda")  # none, out of range, itself, T = 0
    pre_tok = torch.tensor([4096, 1024, 1024, 0], dtype=torch.int64, device="cuda")
    ws = csa.Workspace()
    got = [P.torch_to_np(t) for t in csa.csa_hca_decode_shared(
        layer.batch, pre_seq, pre_tok, layer.pool_off, layer.max_pool, layer.hpool_off, layer.max_hpool, p.m,
        p.m_hca, p.k, p.W, p.W_hca, p.sm_scale, dq["qc"], dq["qs"], dq["w"], layer.kc, layer.ks, dq["q"],
        layer.pooled, layer.hpooled, layer.kv, ws=ws)]
    csa.csa_hca_decode_check(layer.batch, ws)
    torch.cuda.synchronize()
    for what, x, y in zip(("idx", "csa_out", "csa_lse", "hca_out", "hca_lse"), got, want):
        assert np.array_equal(x, y), f"{what} differs from csa_hca_decode"


# name -> (workload, CSA page rows, HCA page rows, prefix tokens shared by sequence 1 with sequence 0 or 0)
PAGED_CASES = {
    "paged_p64_h32": (lambda: small_wl("decode_paged", [20003, 9001, 4099, 70001], [1] * 4, k=256, seed=41),
                      64, 32, 0),
    "paged_p256_h64_shared": (lambda: small_wl("decode_paged_sh", [30000, 8192 + 6001, 2050], [1] * 3, H=32, k=300,
                                               W=200, m_hca=64, W_hca=64, seed=42), 256, 64, 8192),
    "paged_long": (lambda: small_wl("decode_paged_long", [262147, 131075], [1] * 2, k=1024, seed=43), 128, 32, 0),
    # 40 rows whose plan leaves chunks past the first round: the compact form
    # (ticket units over the row table) through page tables
    "paged_many_rows": (lambda: small_wl("decode_paged_many", _MANY_ROWS, [1] * 40, k=200, seed=44), 64, 32, 0),
    # every row takes the exact fallback (its entries come from the stored keys)
    "paged_concentrated": (lambda: small_wl("decode_paged_conc", [40001, 30002], [1, 1], k=1024, seed=17), 64, 32, 0,
                           "concentrate"),
}


def _pages(rows_per_seq, page_rows, rng, shared=None):
    """A page table for sequences of the given row counts over one shuffled
    pool of pages (plus spare pages); shared = (seq, n_pages): that sequence's
    first pages are sequence 0's.  Returns (table [n_seq][max_pages], n_pool_pages)."""
    need = [(n + page_rows - 1) // page_rows for n in rows_per_seq]
    total = sum(need) + 3
    perm = rng.permutation(total)
    table = np.zeros((len(need), max(1, max(need))), dtype=np.int32)
    nxt = 0
    for b, n in enumerate(need):
        for i in range(n):
            if shared is not None and b == shared[0] and i < shared[1]:
                table[b, i] = table[0, i]
            else:
                table[b, i] = perm[nxt]
                nxt += 1
    return table, total


def _scatter(src, off, table, page_rows, n_pages):
    """Rows [off[b], off[b+1]) of a contiguous cache -> their pages."""
    dst = torch.zeros((n_pages * page_rows, *src.shape[1:]), dtype=src.dtype, device=src.device)
    for b in range(len(off) - 1):
        n = int(off[b + 1] - off[b])
        for i in range((n + page_rows - 1) // page_rows):
            r0, r1 = i * page_rows, min(n, (i + 1) * page_rows)
            p = int(table[b, i])
            dst[p * page_rows:p * page_rows + (r1 - r0)] = src[int(off[b]) + r0:int(off[b]) + r1]
    return dst


@pytest.mark.parametrize("name", list(PAGED_CASES))
def test_paged_decode_is_bit_identical_to_contiguous_caches(name):
    """csa_hca_decode_paged over pooled caches scattered into shuffled pages
    (one case with a sequence whose first pages are another's, over equal
    data) gives exactly csa_hca_decode's outputs on the contiguous caches, and
    the oracle's top-k and outputs on the first and last rows."""
    csa = _lib()
    make, pr, hpr, T = PAGED_CASES[name][:4]
    wl = make()
    host = synth.make_inputs(wl)
    if PAGED_CASES[name][4:] == ("concentrate",):
        host = _concentrate(host)
    if T:
        to, po = host["tok_off"], host["pool_off"]
        for nm in ("kv", "z"):
            host[nm][to[1]:to[1] + T] = host[nm][to[0]:to[0] + T]
        for nm in ("kc", "ks"):
            host[nm][po[1]:po[1] + T // wl.m] = host[nm][po[0]:po[0] + T // wl.m]
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    want = [P.torch_to_np(t) for t in layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])]
    layer.check_fused()
    rng = np.random.default_rng(7)
    po, ho = host["pool_off"], host["hpool_off"]
    P_b, Ph_b = np.diff(po), np.diff(ho)
    tab, npg = _pages(P_b, pr, rng, (1, T // wl.m // pr) if T else None)
    htab, nhpg = _pages(Ph_b, hpr, rng, (1, T // wl.m_hca // hpr) if T else None)
    pooled2 = _scatter(layer.pooled, po, tab, pr, npg)
    kc2, ks2 = _scatter(layer.kc, po, tab, pr, npg), _scatter(layer.ks, po, tab, pr, npg)
    hpooled2 = _scatter(layer.hpooled, ho, htab, hpr, nhpg)
    p = layer.p
    ws = csa.Workspace()
    dev = lambda a, t: torch.from_numpy(np.ascontiguousarray(a, dtype=t)).cuda()
    got = [P.torch_to_np(t) for t in csa.csa_hca_decode_paged(
        layer.batch, pr, dev(tab, np.int32), dev(P_b, np.int64), hpr, dev(htab, np.int32), dev(Ph_b, np.int64),
        layer.max_pool, layer.max_hpool, p.m, p.m_hca, p.k, p.W, p.W_hca, p.sm_scale, dq["qc"], dq["qs"], dq["w"],
        kc2, ks2, dq["q"], pooled2, hpooled2, layer.kv, ws=ws)]
    csa.csa_hca_decode_check(layer.batch, ws)
    torch.cuda.synchronize()
    for what, x, y in zip(("idx", "csa_out", "csa_lse", "hca_out", "hca_lse"), got, want):
        assert np.array_equal(x, y), f"{what} differs from the contiguous layout"
    # the oracle on the logical sequences: the first and the last row
    idx, co, cl, hop, hl = got
    seqs = P.row_seq(host)
    scale = 1 / math.sqrt(wl.d)
    for r in sorted({0, wl.n_q - 1}):
        b = seqs[r]
        (t0, t1), (p0, p1), _ = P.seq_slices(host, b)
        t = int(host["q_pos"][r])
        o, l, i = oracle.csa_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m, wl.W, wl.k, scale,
                                   host["qc"][r], host["qs"][r], host["w"][r], host["kc"][p0:p1], host["ks"][p0:p1])
        assert np.array_equal(idx[r], i), f"top-k of row {r}"
        P.check_close(co[r:r + 1], o[None], wl.dtype, f"csa output of row {r}")
        P.check_close(cl[r:r + 1], l[None], "bf16", f"csa lse of row {r}")
        ho_r, hl_r = oracle.hca_query(host["kv"][t0:t1], host["z"][t0:t1], host["q"][r], t, wl.m_hca, wl.W_hca, scale)
        P.check_close(hop[r:r + 1], ho_r[None], wl.dtype, f"hca output of row {r}")
        P.check_close(hl[r:r + 1], hl_r[None], "bf16", f"hca lse of row {r}")


def _zero_weight_blocks(host):
    """Indexer query blocks the fold of a head weight must survive: for every
    query, head 0's first 32-element block all zero (codes 0 and -0) with
    scale byte 0, head 1's second block all zero with byte 0, head 2's first
    block all zero with byte 254, all with weights 0.5 on heads 0 and 1 (a
    folded byte of -1 would be E8M0's NaN) and 2 on head 2 (255)."""
    qc, qs, w = host["qc"].copy(), host["qs"].copy(), host["w"].copy()
    qc[:, 0, :16] = np.where(np.arange(16) % 2 == 0, 0x00, 0x88).astype(np.uint8)
    qs[:, 0, 0] = 0
    qc[:, 1, 16:] = 0x08
    qs[:, 1, 1] = 0
    qc[:, 2, :16] = 0x80
    qs[:, 2, 0] = 254
    w[:, 0] = 0.5
    w[:, 1] = 0.5
    w[:, 2] = 2.0
    host["qc"], host["qs"], host["w"] = qc, qs, w
    return host


@pytest.mark.parametrize("lengths,q_counts", [([3001, 70001, 517], [1, 1, 1]), ([5000, 9001], [40, 100])])
def test_index_topk_with_zero_query_blocks_and_folded_weights(lengths, q_counts):
    """csa_index_topk (decode and prefill paths) on queries with all-zero blocks
    whose scale byte sits at the edge of E8M0's range, under head weights whose
    fold would leave that range: the same top-k as the oracle's exact scores."""
    csa = _lib()
    wl = small_wl("index_zero_blocks", lengths, q_counts, k=128, seed=51)
    host = _zero_weight_blocks(synth.make_inputs(wl, raw=False))
    got = _index_rows(wl, host, range(wl.n_q))
    assert got.shape == (wl.n_q, wl.k)


def test_fused_decode_with_zero_query_blocks_and_folded_weights():
    """The one-launch decode step on the same edge-case queries: top-k equal to
    the oracle's and to csa_index_topk's."""
    csa = _lib()
    wl = small_wl("decode_zero_blocks", [3001, 70001, 517, 40003], [1] * 4, k=256, seed=52)
    host = _zero_weight_blocks(synth.make_inputs(wl))
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    idx = P.torch_to_np(layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])[0])
    layer.check_fused()
    seqs = P.row_seq(host)
    for r in range(wl.n_q):
        want = P.oracle_topk_row(host, wl, r, seqs[r], wl.k, wl.m)
        assert np.array_equal(idx[r], want), f"top-k of row {r}"


@pytest.mark.parametrize("name", ["decode_bf16_long", "decode_bf16_ragged"])
def test_fused_decode_groups_compute_late_chunks_themselves(name, monkeypatch):
    """With the steal threshold at one poll, a CSA group that finds any list of
    its row not yet written computes that score chunk itself (the path that
    keeps the step going when a first-round workgroup has not started) and a
    chunk may run twice: the outputs are bit-identical to a normal launch and
    the top-k equals the oracle's."""
    csa = _lib()
    wl = FUSED_CASES[name]()
    host = synth.make_inputs(wl)
    from long_context_compressed_05_amd.step import Layer, to_device
    layer = Layer.from_host(_params(wl), host)
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    want = [P.torch_to_np(t) for t in layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])]
    layer.check_fused()
    monkeypatch.setenv("CSA_FUSED_STEAL_POLLS", "1")
    for _ in range(3):
        got = [P.torch_to_np(t) for t in layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])]
        layer.check_fused()
        for what, x, y in zip(("idx", "csa_out", "csa_lse", "hca_out", "hca_lse"), got, want):
            assert np.array_equal(x, y), f"{what} differs when groups compute late chunks"
    seqs = P.row_seq(host)
    for r in range(wl.n_q):
        assert np.array_equal(got[0][r], P.oracle_topk_row(host, wl, r, seqs[r], wl.k, wl.m)), f"top-k of row {r}"


def _bf16_exact_inputs(rng, lengths, m):
    """Decode indexer inputs on which fp32 accumulation is exact: bf16 queries
    in {-4..4}/4, keys in {-3..3}/2, head weights powers of two (every partial
    sum a multiple of 1/8 below 2^10).  Small ranges give many tied scores."""
    B = len(lengths)
    P_b = [L // m for L in lengths]
    pool_off = synth.offsets(P_b)
    q = (rng.integers(-4, 5, size=(B, 4, 64)) * 0.25).astype(np.float32)
    keys = (rng.integers(-3, 4, size=(int(pool_off[-1]), 64)) * 0.5).astype(np.float32)
    w = np.exp2(rng.integers(-1, 2, size=(B, 4))).astype(np.float32)
    bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    return P_b, pool_off, bits(q), bits(keys), w


@pytest.mark.parametrize("lengths,k", [
    ([1, 3, 130, 517, 1030, 2049, 4099], 64),    # ragged, k above the visible count, empty sequences
    ([160001, 200003], 1000),                    # large ranges, heavy ties
    ([3200003], 2048),                           # visible range beyond the LDS bitmap
])
def test_index_topk_bf16_matches_the_oracle(lengths, k):
    """csa_index_topk_bf16 against the oracle's fp64 bf16 scores and full sort,
    bit for bit, on inputs where the kernel's fp32 arithmetic is exact."""
    csa = _lib()
    m = 4
    P_b, pool_off, qb, kb, w = _bf16_exact_inputs(np.random.default_rng(41), lengths, m)
    B = len(lengths)
    as_bf16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q_pos = np.array(lengths) - 1
    batch = csa.Batch.from_host(synth.offsets(lengths), np.arange(B + 1), q_pos)
    ws = csa.Workspace()
    args = (batch, torch.from_numpy(pool_off).cuda(), max(P_b), m, k, as_bf16(qb),
            torch.from_numpy(w).cuda(), as_bf16(kb))
    got = P.torch_to_np(csa.csa_index_topk_bf16(*args, ws=ws))
    for b in range(B):
        p0 = int(pool_off[b])
        n_vis = min((int(q_pos[b]) + 1) // m, P_b[b])
        S = oracle.index_scores_bf16(qb[b], w[b], kb[p0:p0 + n_vis])
        np.testing.assert_array_equal(got[b], oracle.topk(S, k), err_msg=f"sequence {b}")
    again = P.torch_to_np(csa.csa_index_topk_bf16(*args, ws=ws))
    assert np.array_equal(again, got), "a second call on the same workspace differs"

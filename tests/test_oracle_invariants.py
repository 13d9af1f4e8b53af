"""Method-level invariants of the CPU oracle (CPU only).

  * with k >= the number of visible pooled entries, CSA equals dense attention
    over all visible pooled entries plus the window;
  * m = 1 with one-hot pooling reduces CSA / HCA to plain causal MQA;
  * causality: nothing after position t, and no block ending after t, matters.
The dense / MQA references are computed here with scipy on rows assembled by
the test, so a slip in the oracle's list assembly, window bounds or block
visibility fails them.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import synth

SCALE = 1 / math.sqrt(32)


def _f64(a):
    return a.astype(np.float64) if a.dtype == np.float32 else synth.bf16_bits_to_f32(a).astype(np.float64)


def _mqa(q, keys, vals, bias=None):
    lg = SCALE * (_f64(q) @ keys.T)
    if bias is not None:
        lg = lg + bias[None, :]
    return softmax(lg, axis=1) @ vals, logsumexp(lg, axis=1)


def _seq(L, d=32, H=4, dt="f32", seed=0, n_idx_keys=None, m=4):
    kv = synth.normal(seed, synth.S_KV, L * 2 * d, dt).reshape(L, 2, d)
    z = synth.normal(seed, synth.S_Z, L * 2 * d, dt).reshape(L, 2, d)
    q = synth.normal(seed, synth.S_Q, H * d, dt).reshape(H, d)
    P = (n_idx_keys if n_idx_keys is not None else L // m)
    qc = synth.codes4(seed, synth.S_QCODE, 4 * 32, synth.E2M1_ALL_CODES).reshape(4, 32)
    qs = synth.exp_bytes(seed, synth.S_QSCALE, 8, -2, 2).reshape(4, 2)
    w = synth.pow2(seed, synth.S_W, 4, -1, 1)
    kc = synth.codes4(seed, synth.S_KCODE, P * 32, synth.E2M1_ALL_CODES).reshape(P, 32)
    ks = synth.exp_bytes(seed, synth.S_KSCALE, P * 2, -2, 2).reshape(P, 2)
    return kv, z, q, qc, qs, w, kc, ks


@pytest.mark.parametrize("t", [3, 50, 199, 202])
@pytest.mark.parametrize("W", [0, 1, 16, 300])
def test_csa_with_k_covering_all_equals_dense_over_pooled_plus_window(t, W):
    L, m, d = 203, 4, 32
    kv, z, q, qc, qs, w, kc, ks = _seq(L, d=d, seed=t)
    n_vis = (t + 1) // m
    out, lse, idx = oracle.csa_query(kv, z, q, t, m, W, n_vis + 5, SCALE, qc, qs, w, kc, ks)
    assert list(idx[:n_vis]) == list(range(n_vis)) and np.all(idx[n_vis:] == -1)
    pooled = oracle.pool(kv.reshape(L, -1), z.reshape(L, -1), m).reshape(-1, 2, d)[:n_vis]
    w0 = max(0, t - W + 1)
    win = _f64(kv[w0:t + 1]) if W > 0 else np.zeros((0, 2, d))
    keys = np.concatenate([pooled[:, 0], win[:, 0]])
    vals = np.concatenate([pooled[:, 1], win[:, 1]])
    o2, l2 = _mqa(q, keys, vals)
    assert np.allclose(out, o2, atol=1e-12) and np.allclose(lse, l2, atol=1e-12)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_m1_reduces_to_causal_mqa(dt):
    L, d, t = 150, 32, 120
    kv, z, q, qc, qs, w, kc, ks = _seq(L, d=d, dt=dt, seed=3, m=1)
    ref_o, ref_l = _mqa(q, _f64(kv[:t + 1, 0]), _f64(kv[:t + 1, 1]))
    # HCA with m' = 1 and no window: plain causal MQA over tokens 0..t
    o, l = oracle.hca_query(kv, z, q, t, 1, 0, SCALE)
    assert np.allclose(o, ref_o, atol=1e-12) and np.allclose(l, ref_l, atol=1e-12)
    # CSA with m = 1, k >= t+1, W = 0: the same
    o, l, idx = oracle.csa_query(kv, z, q, t, 1, 0, t + 1, SCALE, qc, qs, w, kc, ks)
    assert np.allclose(o, ref_o, atol=1e-12) and np.allclose(l, ref_l, atol=1e-12)
    # CSA with m = 1, k >= t+1, W > 0: window tokens appear twice (pooled and raw,
    # no dedup), which equals adding ln 2 to those tokens' logits
    W = 17
    bias = np.zeros(t + 1)
    bias[t - W + 1:] = math.log(2.0)
    ref_o2, ref_l2 = _mqa(q, _f64(kv[:t + 1, 0]), _f64(kv[:t + 1, 1]), bias)
    o, l, idx = oracle.csa_query(kv, z, q, t, 1, W, t + 1, SCALE, qc, qs, w, kc, ks)
    assert np.allclose(o, ref_o2, atol=1e-12) and np.allclose(l, ref_l2, atol=1e-12)


def test_onehot_pooling_reduces_to_mqa_over_chosen_tokens():
    L, m, d, t = 256, 8, 32, 250
    kv, z, q, qc, qs, w, kc, ks = _seq(L, d=d, seed=4, m=m)
    pick = 5  # every block keeps its 6th token
    z = np.full_like(z, -1.0e4)
    z[pick::m] = 0.0
    n_vis = (t + 1) // m
    chosen = np.arange(n_vis) * m + pick
    ref_o, ref_l = _mqa(q, _f64(kv[chosen, 0]), _f64(kv[chosen, 1]))
    o, l = oracle.hca_query(kv, z, q, t, m, 0, SCALE)
    assert np.allclose(o, ref_o, atol=1e-12) and np.allclose(l, ref_l, atol=1e-12)
    o, l, idx = oracle.csa_query(kv, z, q, t, m, 0, n_vis, SCALE, qc, qs, w, kc, ks)
    assert np.allclose(o, ref_o, atol=1e-12) and np.allclose(l, ref_l, atol=1e-12)


def test_causality():
    L, m, d, t = 200, 4, 32, 137  # (t+1) % m == 2: block 34 (tokens 136..139) is not complete
    kv, z, q, qc, qs, w, kc, ks = _seq(L, d=d, seed=5)
    n_vis = (t + 1) // m
    assert n_vis == 34
    o1, l1, i1 = oracle.csa_query(kv, z, q, t, m, 8, 10, SCALE, qc, qs, w, kc, ks)
    h1, hl1 = oracle.hca_query(kv, z, q, t, 16, 0, SCALE)
    kv2, z2, kc2 = kv.copy(), z.copy(), kc.copy()
    kv2[t + 1:] = kv2[t + 1:] * 3  # the future
    z2[t + 1:] = -z2[t + 1:]
    kc2[n_vis:] = 0x77  # keys of blocks that are not yet complete get huge scores
    o2, l2, i2 = oracle.csa_query(kv2, z2, q, t, m, 8, 10, SCALE, qc, qs, w, kc2, ks)
    h2, hl2 = oracle.hca_query(kv2, z2, q, t, 16, 0, SCALE)
    assert np.array_equal(i1, i2) and np.all(i1 < n_vis)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    # the window ends at t and includes it: changing token t changes the output
    kv3 = kv.copy()
    kv3[t, 1] += 1
    o3, _, _ = oracle.csa_query(kv3, z, q, t, m, 8, 10, SCALE, qc, qs, w, kc, ks)
    assert not np.array_equal(o1, o3)
    # ... and starts at t-W+1: token t-W does not matter (it is in no selected block here)
    blk = (t - 8) // m
    if blk not in set(i1.tolist()):
        kv4 = kv.copy()
        kv4[t - 8] += 1
        o4, _, _ = oracle.csa_query(kv4, z, q, t, m, 8, 10, SCALE, qc, qs, w, kc, ks)
        assert np.array_equal(o1, o4)


def test_hca_empty_visible_set():
    kv, z, q, *_ = _seq(64, seed=6)
    o, l = oracle.hca_query(kv, z, q, 10, 16, 0, SCALE)  # (10+1)//16 == 0 entries
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_selected_set_is_the_exact_topk_of_scores():
    L, m, d, t = 400, 4, 32, 399
    kv, z, q, qc, qs, w, kc, ks = _seq(L, d=d, seed=7)
    _, _, idx = oracle.csa_query(kv, z, q, t, m, 16, 20, SCALE, qc, qs, w, kc, ks)
    S, _ = oracle.index_scores(qc, qs, w, kc, ks)
    order = sorted(range(100), key=lambda j: (-S[j], j))
    assert list(idx) == sorted(order[:20])


def test_stagewise_given_matches_end_to_end():
    L, m, d, t, W, k = 300, 4, 32, 299, 24, 12
    kv, z, q, qc, qs, w, kc, ks = _seq(L, d=d, seed=8)
    pooled64 = oracle.pool(kv.reshape(L, -1), z.reshape(L, -1), m)
    o1, l1, idx = oracle.csa_query(kv, z, q, t, m, W, k, SCALE, qc, qs, w, kc, ks, pooled=pooled64)
    o0, l0, idx0 = oracle.csa_query(kv, z, q, t, m, W, k, SCALE, qc, qs, w, kc, ks)
    assert np.array_equal(idx, idx0) and np.allclose(o0, o1, atol=1e-14)
    pooled32 = pooled64.astype(np.float32).reshape(-1, 2, d)
    o2, l2 = oracle.csa_attend_given(kv, pooled32, idx, q, t, W, SCALE)
    assert np.allclose(o1, o2, atol=1e-6) and np.allclose(l1, l2, atol=1e-6)
    hp64 = oracle.pool(kv.reshape(L, -1), z.reshape(L, -1), 32)
    h1, hl1 = oracle.hca_query(kv, z, q, t, 32, 0, SCALE, hpooled=hp64)
    h2, hl2 = oracle.hca_attend_given(kv, hp64.astype(np.float32).reshape(-1, 2, d), q, t, 32, 0, SCALE)
    assert np.allclose(h1, h2, atol=1e-6) and np.allclose(hl1, hl2, atol=1e-6)

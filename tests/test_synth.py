"""Input generator checks (CPU): determinism, counter addressing, formats."""
import numpy as np
import pytest
import torch

import synth


def test_deterministic_and_counter_addressed():
    a = synth.normal(7, synth.S_KV, 10000, "f32")
    b = synth.normal(7, synth.S_KV, 10000, "f32")
    assert np.array_equal(a, b)
    # element i can be regenerated on its own (counter-based)
    part = synth.normal(7, synth.S_KV, 100, "f32", off=5000)
    assert np.array_equal(part, a[5000:5100])
    # streams and seeds are independent
    c = synth.normal(7, synth.S_Z, 10000, "f32")
    d = synth.normal(8, synth.S_KV, 10000, "f32")
    assert not np.array_equal(a, c) and not np.array_equal(a, d)
    # threaded and single-threaded generation agree (large n uses threads)
    big = synth.normal(3, synth.S_Q, 300000, "f32")
    assert np.array_equal(big[123456:123466], synth.normal(3, synth.S_Q, 10, "f32", off=123456))


def test_normal_moments():
    x = synth.normal(11, synth.S_KV, 1 << 20, "f32").astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1.0) < 0.01
    assert abs((x ** 3).mean()) < 0.02 and abs((x ** 4).mean() - 3.0) < 0.05


def test_bf16_rounding_matches_torch():
    f = synth.normal(5, synth.S_Q, 100000, "f32")
    b = synth.normal(5, synth.S_Q, 100000, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_code_and_exponent_ranges():
    c = synth.codes4(1, synth.S_KCODE, 50000, synth.E2M1_TIE_CODES)
    lo, hi = c & 15, c >> 4
    allowed = set(synth.E2M1_TIE_CODES)
    assert set(np.unique(lo)) == allowed and set(np.unique(hi)) == allowed
    c16 = synth.codes4(1, synth.S_KCODE, 50000, synth.E2M1_ALL_CODES)
    assert len(np.unique(c16 & 15)) == 16 and len(np.unique(c16 >> 4)) == 16
    e = synth.exp_bytes(1, synth.S_KSCALE, 50000, -2, 2)
    assert set(np.unique(e)) == {125, 126, 127, 128, 129}
    w = synth.pow2(1, synth.S_W, 50000, -1, 1)
    assert set(np.unique(w)) == {0.5, 1.0, 2.0}


def test_ragged_lengths():
    L = synth.loguniform_lengths(1005, 32, 4096, 1 << 20, 4)
    assert L.min() >= 4096 and L.max() <= (1 << 20)
    assert np.all(L % 4 != 0)
    assert np.array_equal(L, synth.loguniform_lengths(1005, 32, 4096, 1 << 20, 4))


def test_workload_shapes():
    wl = synth.decode_t4096_fp32()
    inp = synth.make_inputs(wl)
    assert inp["kv"].shape == (4096, 2, 128) and inp["kv"].dtype == np.float32
    assert inp["qc"].shape == (1, 4, 32) and inp["qs"].shape == (1, 4, 2)
    assert inp["kc"].shape == (1024, 32) and inp["ks"].shape == (1024, 2)
    assert list(inp["pool_off"]) == [0, 1024] and list(inp["hpool_off"]) == [0, 32]
    assert list(inp["q_pos"]) == [4095]
    wl2 = synth.prefill_4k_on_64k()
    assert wl2.n_q == 4096 and wl2.pooled(4) == [17408] and wl2.pooled(128) == [544]

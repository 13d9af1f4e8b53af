"""Pins of the CPU oracle to facts fixed outside itself (CPU only).

Every pin here comes from a hand-worked golden value, a closed form, an
invariant of the method, or a library routine (numpy / scipy) for a special
case — never from the oracle's own arithmetic retyped.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def golden_e2m1():
    table = {}
    with open(os.path.join(GOLD, "e2m1_codes.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            table[int(c)] = float(v)
    return table


E2M1 = golden_e2m1()


def pack_hex(s):
    """one hex e2m1 code per element, element 0 first -> packed bytes (even element low)"""
    codes = [int(ch, 16) for ch in s]
    return np.array([codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(len(codes) // 2)], np.uint8)


def decode_vec(packed, scales):
    """MXFP4 vector -> float64 values via the golden code table (test-side decoding)."""
    codes = np.empty(2 * packed.shape[-1], np.int64)
    codes[0::2] = packed & 15
    codes[1::2] = packed >> 4
    vals = np.array([E2M1[int(c)] for c in codes])
    sc = np.repeat(np.array([2.0 ** (int(e) - 127) for e in scales]), 32)
    return vals * sc


# ----------------------------------------------------------------------------
# MXFP4 quantiser (the step before the indexer)
# ----------------------------------------------------------------------------
def _nibbles(codes_row):
    out = []
    for b in codes_row:
        out += [int(b) & 15, int(b) >> 4]
    return out


def test_mxfp4_quantize_golden_hand_cases():
    g = json.load(open(os.path.join(GOLD, "mxfp4_quant_hand.json")))
    for c in g["cases"]:
        x = np.zeros((1, 32), np.float32)
        x[0, :len(c["x"])] = c["x"]
        codes, scales = oracle.mxfp4_quantize(x)
        nib = _nibbles(codes[0])
        assert int(scales[0, 0]) == c["scale_byte"], c["what"]
        assert nib[:len(c["codes"])] == c["codes"], c["what"]
        assert all(v == 0 for v in nib[len(c["codes"]):]), c["what"]


def test_mxfp4_quantize_round_trips_representable_blocks():
    """A block built from e2m1 values times one power of two, with its largest
    magnitude in [4, 6], comes back exactly: same codes (zero canonical), same scale."""
    rng = np.random.default_rng(3)
    for e in (-20, -3, 0, 5, 30):
        codes = rng.integers(0, 16, size=(64, 32))
        codes[:, 0] = rng.choice([6, 7, 14, 15], size=64)  # magnitude 4 or 6 sets the scale
        vals = np.array([[E2M1[int(c)] for c in row] for row in codes]) * 2.0 ** e
        q, sc = oracle.mxfp4_quantize(vals.astype(np.float32))
        assert (sc == e + 127).all()
        got = np.array([_nibbles(r) for r in q])
        want = np.where(codes == 8, 0, codes)  # -0 quantises to +0
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(np.stack([decode_vec(q[i], sc[i]) for i in range(64)]), vals)


def test_mxfp4_quantize_sign_scale_and_error_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((200, 64)).astype(np.float32) * np.float32(3.0)
    q, sc = oracle.mxfp4_quantize(x)
    # sign symmetry: -x flips the sign bit of every non-zero code
    qn, scn = oracle.mxfp4_quantize(-x)
    np.testing.assert_array_equal(scn, sc)
    a, b = np.array([_nibbles(r) for r in q]), np.array([_nibbles(r) for r in qn])
    np.testing.assert_array_equal(b, np.where(a == 0, 0, a ^ 8))
    # a power-of-two rescale moves only the scale byte
    q2, sc2 = oracle.mxfp4_quantize(x * np.float32(2.0 ** 9))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(sc2.astype(int), sc.astype(int) + 9)
    # error bound: within half the gap between the neighbouring e2m1 values
    # (the largest gap, between 4 and 6, is 2), in units of the block scale;
    # the block maximum lies in [4, 8) units and may saturate (error < 2)
    deq = np.stack([decode_vec(q[i], sc[i]) for i in range(len(x))])
    unit = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=1)
    v = np.abs(x.astype(np.float64)) / unit
    mags = np.array(sorted(set(abs(E2M1[c]) for c in range(16))))
    gap = np.array([[np.diff(mags)[min(np.searchsorted(mags, t, side="right") - 1, len(mags) - 2)] for t in row]
                    for row in v])
    err = np.abs(deq - x.astype(np.float64)) / unit
    assert np.all(err <= np.where(v <= 6.0, gap / 2, 2.0) + 1e-12)
    assert np.all(np.where(v > 6.0, err < 2.0, True))


# ----------------------------------------------------------------------------
# codec
# ----------------------------------------------------------------------------
def test_e2m1_matches_golden_table():
    for code, val in E2M1.items():
        got = oracle.e2m1_value(code)
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code


def fp8_e4m3_values():
    """All finite FP8 E4M3 (OCP 8-bit float) values, from the format definition."""
    vals = set()
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            continue  # NaN
        mag = (m / 8.0) * 2.0 ** (1 - 7) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals.add(-mag if s else mag)
    return vals


def test_fp4_to_fp8_dequant_is_lossless():
    """The pages state FP4->FP8 dequantisation is lossless: every e2m1 value is an E4M3 value."""
    e4m3 = fp8_e4m3_values()
    for code in range(16):
        assert oracle.e2m1_value(code) in e4m3


def test_e8m0():
    for e in (0, 1, 120, 125, 127, 129, 200, 254):
        assert oracle.e8m0_value(e) == 2.0 ** (e - 127)
    assert math.isnan(oracle.e8m0_value(255))


# ----------------------------------------------------------------------------
# pooling (compression)
# ----------------------------------------------------------------------------
def test_pool_golden_hand_cases():
    cases = json.load(open(os.path.join(GOLD, "pool_hand.json")))["cases"]
    for c in cases:
        x = np.array(c["x"], np.float32).reshape(-1, 1)
        z = np.array(c["z"], np.float32).reshape(-1, 1)
        out = oracle.pool(x, z, c["m"])
        assert out.shape == (1, 1)
        assert abs(out[0, 0] - c["expected"]) < 1e-6, c["derivation"]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_pool_m1_is_identity(dt):
    x = synth.normal(1, 1, 64 * 16, dt).reshape(64, 16)
    z = synth.normal(1, 2, 64 * 16, dt).reshape(64, 16)
    out = oracle.pool(x, z, 1)
    xf = x if dt == "f32" else synth.bf16_bits_to_f32(x)
    assert np.array_equal(out, xf.astype(np.float64))


def test_pool_equal_logits_is_mean_and_onehot_is_token():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((40, 8)).astype(np.float32)
    z = np.full((40, 8), 0.25, np.float32)
    out = oracle.pool(x, z, 4)
    assert np.allclose(out, x.astype(np.float64).reshape(10, 4, 8).mean(1), rtol=0, atol=1e-12)
    # one logit 0, the rest -1e4: exp underflows to exactly 0, so the token itself comes out
    pick = rng.integers(0, 4, size=(10, 8))
    zz = np.full((40, 8), -1.0e4, np.float32)
    for j in range(10):
        for c in range(8):
            zz[4 * j + pick[j, c], c] = 0.0
    out = oracle.pool(x, zz, 4)
    want = np.take_along_axis(x.reshape(10, 4, 8), pick[:, None, :], axis=1)[:, 0, :]
    assert np.array_equal(out, want.astype(np.float64))


def test_pool_shift_invariance_hull_and_locality():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((96, 6)).astype(np.float32)
    z = (rng.integers(-16, 16, size=(96, 6)) / 8.0).astype(np.float32)  # dyadic: z+1 is exact
    a = oracle.pool(x, z, 8)
    b = oracle.pool(x, z + np.float32(1.0), 8)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-14)
    xb = x.astype(np.float64).reshape(12, 8, 6)
    assert np.all(a >= xb.min(1) - 1e-12) and np.all(a <= xb.max(1) + 1e-12)
    # block locality: changing rows of block 5 only changes pooled row 5
    x2 = x.copy()
    x2[40:48] += 1.0
    c = oracle.pool(x2, z, 8)
    diff = np.any(c != a, axis=1)
    assert diff[5] and diff.sum() == 1
    # channel locality: changing logits of channel 2 only changes channel 2
    z2 = z.copy()
    z2[:, 2] = -z2[:, 2]
    e = oracle.pool(x, z2, 8)
    assert np.array_equal(np.delete(e, 2, axis=1), np.delete(a, 2, axis=1))
    # tail rows that do not fill a block are not pooled
    assert oracle.pool(x[:95], z[:95], 8).shape == (11, 6)


def test_pool_matches_scipy_softmax():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((12, 5)).astype(np.float32)
    z = rng.standard_normal((12, 5)).astype(np.float32)
    out = oracle.pool(x, z, 3)
    xb = x.astype(np.float64).reshape(4, 3, 5)
    wb = softmax(z.astype(np.float64).reshape(4, 3, 5), axis=1)
    assert np.allclose(out, (wb * xb).sum(1), rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# indexer score
# ----------------------------------------------------------------------------
def _case_arrays(c):
    qc = np.stack([pack_hex(s) for s in c["q"]])
    qs = np.array(c["qs"], np.uint8)
    w = np.array(c["w"], np.float32)
    kc = pack_hex(c["k"])[None, :]
    ks = np.array(c["ks"], np.uint8)[None, :]
    return qc, qs, w, kc, ks


def test_index_golden_hand_cases():
    cases = json.load(open(os.path.join(GOLD, "index_hand.json")))["cases"]
    for c in cases:
        S, ex = oracle.index_scores(*_case_arrays(c))
        assert S[0] == c["expected"], c["derivation"]
        assert ex[0]


def _random_index(seed, n, codeset=synth.E2M1_ALL_CODES):
    qc = synth.codes4(seed, synth.S_QCODE, 4 * 32, codeset).reshape(4, 32)
    qs = synth.exp_bytes(seed, synth.S_QSCALE, 8, -2, 2).reshape(4, 2)
    w = synth.pow2(seed, synth.S_W, 4, -1, 1)
    kc = synth.codes4(seed, synth.S_KCODE, n * 32, codeset).reshape(n, 32)
    ks = synth.exp_bytes(seed, synth.S_KSCALE, n * 2, -2, 2).reshape(n, 2)
    return qc, qs, w, kc, ks


def test_index_relu_identities_against_matmul():
    """S(k) - S(-k) = sum_h w_h D_h and S(k) + S(-k) = sum_h w_h |D_h|, where
    D = Q K^T is taken from a numpy matmul of test-decoded values."""
    qc, qs, w, kc, ks = _random_index(3, 500)
    S_pos, _ = oracle.index_scores(qc, qs, w, kc, ks)
    S_neg, _ = oracle.index_scores(qc, qs, w, kc ^ np.uint8(0x88), ks)  # flip both sign bits
    Q = np.stack([decode_vec(qc[h], qs[h]) for h in range(4)])
    K = np.stack([decode_vec(kc[j], ks[j]) for j in range(kc.shape[0])])
    D = K @ Q.T  # [n][4]
    assert np.array_equal(S_pos - S_neg, D @ w.astype(np.float64))
    assert np.array_equal(S_pos + S_neg, np.abs(D) @ w.astype(np.float64))
    assert np.array_equal(S_pos, np.maximum(D, 0) @ w.astype(np.float64))


def test_index_scale_doubling_and_head_weights():
    qc, qs, w, kc, ks = _random_index(4, 200)
    S, _ = oracle.index_scores(qc, qs, w, kc, ks)
    # doubling every key scale doubles every head dot and hence S (ReLU is positively homogeneous)
    S2, _ = oracle.index_scores(qc, qs, w, kc, ks + np.uint8(1))
    assert np.array_equal(S2, 2 * S)
    # doubling one head weight adds exactly that head's term again
    w2 = w.copy()
    w2[1] *= 2
    S3, _ = oracle.index_scores(qc, qs, w2, kc, ks)
    Q = decode_vec(qc[1], qs[1])
    K = np.stack([decode_vec(kc[j], ks[j]) for j in range(kc.shape[0])])
    assert np.array_equal(S3 - S, w[1] * np.maximum(K @ Q, 0))


@pytest.mark.parametrize("codeset", [synth.E2M1_ALL_CODES, synth.E2M1_TIE_CODES])
def test_index_fp32_exactness_precondition_holds_for_workload_distributions(codeset):
    qc, qs, w, kc, ks = _random_index(5, 20000, codeset)
    S, ex = oracle.index_scores(qc, qs, w, kc, ks)
    assert ex.all()
    assert S.max() < 2.0 ** 17 and np.all(S * 128 == np.round(S * 128))


def test_index_exactness_flag_detects_wide_scale_spread():
    qc = np.full((4, 32), 0x77, np.uint8)  # all 6.0
    qs = np.array([[127 + 12, 127 - 12]] * 4, np.uint8)  # exact in fp64, not in fp32
    w = np.ones(4, np.float32)
    kc = np.full((1, 32), 0x77, np.uint8)
    ks = np.array([[127, 127]], np.uint8)
    S, ex = oracle.index_scores(qc, qs, w, kc, ks)
    assert not ex[0]
    assert S[0] == 4 * 32 * 36.0 * (2.0 ** 12 + 2.0 ** -12)


def test_index_zero_block_scale_does_not_matter():
    """A query block whose codes are all zero (+0 and -0) adds nothing to the
    head's dot whatever its scale byte, from 0 (2^-127) to 254: the scores
    equal those with the block's scale at 2^0, they equal the matmul of the
    decoded values, and the fp32-exactness flag is not lost to the unused
    scale."""
    qc, qs, w, kc, ks = _random_index(8, 300)
    qc[0, :16] = np.where(np.arange(16) % 2 == 0, 0x80, 0x08).astype(np.uint8)
    qc[2, 16:] = 0x00
    base = qs.copy()
    base[0, 0] = 127
    base[2, 1] = 127
    S_ref, ex_ref = oracle.index_scores(qc, base, w, kc, ks)
    Q = np.stack([decode_vec(qc[h], base[h]) for h in range(4)])
    K = np.stack([decode_vec(kc[j], ks[j]) for j in range(kc.shape[0])])
    assert np.array_equal(S_ref, np.maximum(K @ Q.T, 0) @ w.astype(np.float64))
    assert ex_ref.all()
    for b0, b2 in ((0, 0), (254, 254), (0, 254)):
        q2 = qs.copy()
        q2[0, 0] = b0
        q2[2, 1] = b2
        S, ex = oracle.index_scores(qc, q2, w, kc, ks)
        assert np.array_equal(S, S_ref)
        assert ex.all()


def _to_bf16_bits(v):
    """fp64 values exactly representable in bf16 -> bf16 bit patterns (checked)."""
    f = np.asarray(v, np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(v, np.float64))
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((b.astype(np.uint32) << 16).view(np.float32), f), "not a bf16 value"
    return b


def test_index_bf16_scores_equal_the_mxfp4_scores_of_the_same_values():
    """Every MXFP4 value (an e2m1 value times 2^e) is a bf16 value: the bf16
    score of the decoded vectors equals the exact MXFP4 score, for the whole
    set, ties and zeros included."""
    for seed, codeset in ((10, synth.E2M1_ALL_CODES), (11, synth.E2M1_TIE_CODES)):
        qc, qs, w, kc, ks = _random_index(seed, 400, codeset)
        S, _ = oracle.index_scores(qc, qs, w, kc, ks)
        qb = _to_bf16_bits(np.stack([decode_vec(qc[h], qs[h]) for h in range(4)]))
        kb = _to_bf16_bits(np.stack([decode_vec(kc[j], ks[j]) for j in range(kc.shape[0])]))
        assert np.array_equal(oracle.index_scores_bf16(qb, w, kb), S)


def test_index_bf16_relu_identities_and_hand_case():
    """S(k) - S(-k) = sum_h w_h D_h, S(k) + S(-k) = sum_h w_h |D_h| with D from
    a numpy matmul; and one worked case: q_0 = e_0, q_1 = -e_1, k = (3, 2, 0..),
    w = (0.5, 2, 1, 1): S = 0.5 * 3 + 2 * max(0, -2) = 1.5."""
    rng = np.random.default_rng(12)
    Q = rng.integers(-5, 6, size=(4, 64)) * 0.25
    K = rng.integers(-5, 6, size=(300, 64)) * 0.5
    w = np.array([0.5, 1.0, 2.0, 1.0], np.float32)
    qb, kb, knb = _to_bf16_bits(Q), _to_bf16_bits(K), _to_bf16_bits(-K)
    D = K @ Q.T
    Sp, Sn = oracle.index_scores_bf16(qb, w, kb), oracle.index_scores_bf16(qb, w, knb)
    assert np.array_equal(Sp - Sn, D @ w.astype(np.float64))
    assert np.array_equal(Sp + Sn, np.abs(D) @ w.astype(np.float64))
    q = np.zeros((4, 64))
    q[0, 0], q[1, 1] = 1.0, -1.0
    k = np.zeros((1, 64))
    k[0, 0], k[0, 1] = 3.0, 2.0
    assert oracle.index_scores_bf16(_to_bf16_bits(q), np.array([0.5, 2, 1, 1], np.float32), _to_bf16_bits(k))[0] == 1.5


# ----------------------------------------------------------------------------
# top-k
# ----------------------------------------------------------------------------
def test_topk_matches_full_sort_exhaustively_on_tiny_inputs():
    rng = np.random.default_rng(6)
    for n in range(0, 11):
        for trial in range(20):
            S = rng.integers(0, 4, size=n).astype(np.float64) / 2.0  # many ties
            for k in range(1, n + 3):
                idx = oracle.topk(S, k)
                order = sorted(range(n), key=lambda j: (-S[j], j))
                want = sorted(order[:min(k, n)]) + [-1] * (k - min(k, n))
                assert list(idx) == want, (S, k)


def test_topk_properties_at_size():
    rng = np.random.default_rng(7)
    S = rng.integers(0, 50, size=20000).astype(np.float64)
    k = 777
    idx = oracle.topk(S, k)
    assert np.all(np.diff(idx) > 0) and len(idx) == k
    sel = np.zeros(S.shape[0], bool)
    sel[idx] = True
    # every selected entry beats every unselected one under (S desc, j asc)
    worst_sel = min((S[j], -j) for j in idx)
    best_rest = max((S[j], -j) for j in np.nonzero(~sel)[0])
    assert worst_sel > best_rest


# ----------------------------------------------------------------------------
# attention with one softmax
# ----------------------------------------------------------------------------
def _scipy_attend(q, keys, vals, scale, bias=None):
    lg = scale * (q @ keys.T)
    if bias is not None:
        lg = lg + bias[None, :]
    p = softmax(lg, axis=1)
    return p @ vals, logsumexp(lg, axis=1)


def test_attend_matches_scipy_and_closed_forms():
    rng = np.random.default_rng(8)
    q, keys, vals = rng.standard_normal((8, 128)), rng.standard_normal((300, 128)), rng.standard_normal((300, 128))
    s = 1 / math.sqrt(128)
    out, lse = oracle.attend(q, keys, vals, s)
    o2, l2 = _scipy_attend(q, keys, vals, s)
    assert np.allclose(out, o2, atol=1e-12) and np.allclose(lse, l2, atol=1e-12)
    # q = 0: uniform weights, the mean of the values, lse = log n
    out, lse = oracle.attend(np.zeros((2, 128)), keys, vals, s)
    assert np.allclose(out, vals.mean(0)[None], atol=1e-13) and np.allclose(lse, math.log(300), atol=1e-13)
    # one key: its value, lse = its logit
    out, lse = oracle.attend(q, keys[:1], vals[:1], s)
    assert np.allclose(out, np.repeat(vals[:1], 8, 0), atol=1e-14)
    assert np.allclose(lse, s * q @ keys[0], atol=1e-12)
    # empty list: zero output, lse = -inf
    out, lse = oracle.attend(q, keys[:0], vals[:0], s)
    assert np.all(out == 0) and np.all(np.isneginf(lse))
    # key order does not matter; a split merged by log-sum-exp equals the whole
    perm = rng.permutation(300)
    o3, l3 = oracle.attend(q, keys[perm], vals[perm], s)
    o1, l1 = oracle.attend(q, keys, vals, s)
    assert np.allclose(o3, o1, atol=1e-13) and np.allclose(l3, l1, atol=1e-13)
    oa, la = oracle.attend(q, keys[:120], vals[:120], s)
    ob, lb = oracle.attend(q, keys[120:], vals[120:], s)
    L = np.logaddexp(la, lb)
    merged = np.exp(la - L)[:, None] * oa + np.exp(lb - L)[:, None] * ob
    assert np.allclose(merged, o1, atol=1e-13) and np.allclose(L, l1, atol=1e-13)

"""The candidate test of the prefill scoring kernel (k_prefill.hip,
pf_relu_sum_bits and pf_tau_signed) on the CPU, in float32 and int32 as the
kernel computes it: for four head products x0..x3 the test v >= tau must
agree with key >= tau, key = (relu(x0) + relu(x1)) + (relu(x2) + relu(x3))
as the sort key's bit pattern, for every threshold, including tau = 0.  The
inputs cover signs, zeros of both signs, subnormals, ties, and sums that
round."""
import numpy as np

F = np.float32


def relu_bits(x):
    b = x.view(np.int32)
    return np.maximum(b, 0).view(np.float32)


def key_bits(x0, x1, x2, x3):
    s = (relu_bits(x0) + relu_bits(x1)) + (relu_bits(x2) + relu_bits(x3))
    return s.view(np.uint32)


def kernel_bits(x0, x1, x2, x3):
    i = lambda v: v.view(np.int32)
    p01 = np.maximum(np.maximum(i(x0 + x1), i(x0)), i(x1))
    p23 = np.maximum(np.maximum(i(x2 + x3), i(x2)), i(x3))
    s = p01.view(np.float32) + p23.view(np.float32)
    return np.maximum(np.maximum(i(s), p01), p23)


def tau_signed(tau):
    tau = np.asarray(tau, dtype=np.uint32)
    return np.where(tau == 0, np.int32(-2**31), np.minimum(tau, 0x7fffffff).astype(np.int64)).astype(np.int32)


def _values(rng, n):
    specials = np.array([0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 3.0, -3.0, 1e-40, -1e-40, 1.5e-45, -1.5e-45, 6.0, -6.0,
                         2.0**-20, -(2.0**-20), 2.0**24, -(2.0**24), 1.0 + 2.0**-23, -(1.0 + 2.0**-23)], dtype=F)
    dyad = (rng.integers(-12, 13, n) * np.exp2(rng.integers(-30, 10, n))).astype(F)
    wide = (rng.standard_normal(n) * np.exp2(rng.integers(-40, 40, n))).astype(F)
    pick = rng.integers(0, 3, n)
    out = np.where(pick == 0, dyad, wide)
    sp = rng.integers(0, len(specials), n)
    return np.where(pick == 2, specials[sp], out).astype(F)


def test_kernel_test_equals_the_key_comparison():
    rng = np.random.default_rng(5)
    n = 400_000
    xs = [_values(rng, n) for _ in range(4)]
    key = key_bits(*xs)
    v = kernel_bits(*xs)
    # positive keys: the same value; zero keys: a non-positive value
    pos = key.view(np.int32) > 0
    assert np.array_equal(v[pos], key.view(np.int32)[pos])
    assert np.all(v[~pos].view(np.float32) <= 0)
    # thresholds: zero, the keys themselves and their neighbours, random ones
    taus = np.concatenate([[0, 1, 0x7f7fffff], key[:2000], key[:2000] + 1, key[:2000] - 1,
                           rng.integers(0, 0x7f800000, 2000)]).astype(np.uint32)
    taus = taus[taus.view(np.int32) >= 0]
    for tau in taus[:3000]:
        want = key >= tau
        got = v >= tau_signed(tau)
        assert np.array_equal(want, got), hex(int(tau))


def test_hand_cases():
    c = lambda *a: [np.array([x], dtype=F) for x in a]
    # all negative: key 0, passes only tau = 0
    x = c(-1.0, -2.0, -0.0, -3.0)
    assert key_bits(*x)[0] == 0 and kernel_bits(*x)[0] <= 0
    assert kernel_bits(*x)[0] >= tau_signed(0) and not kernel_bits(*x)[0] >= tau_signed(1)
    # one positive term: exactly that term
    x = c(-1.0, 2.5, -0.0, -3.0)
    assert kernel_bits(*x)[0] == np.float32(2.5).view(np.int32)
    # rounding: 1 + 2^-24 + 2^-24 + 2^-24 summed in the key's order
    x = c(1.0, 2.0**-24, 2.0**-24, 2.0**-24)
    assert kernel_bits(*x)[0] == key_bits(*x).view(np.int32)[0]

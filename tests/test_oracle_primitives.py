"""Pins of the oracle's primitives against closed forms, special cases and
brute force (not against a retyped copy of the same formula)."""
import itertools
import math

import numpy as np
import pytest

import oracle


def test_round_bf16_nearest_even():
    r = oracle.round_bf16
    assert r(1.0) == 1.0
    assert r(1 + 2 ** -8) == 1.0                     # halfway -> even (down)
    assert r(1 + 3 * 2 ** -8) == 1 + 2 ** -6         # halfway -> even (up)
    assert r(1 + 2 ** -8 + 2 ** -20) == 1 + 2 ** -7  # above halfway -> up
    # the value goes to fp32 first (as on the GPU), so a sub-fp32 excess is lost
    assert r(1 + 2 ** -8 + 2 ** -30) == 1.0
    assert r(-3.0) == -3.0


def test_rmsnorm_closed_forms():
    n, eps = 64, 1e-6
    for c in (0.5, -3.0, 1e-2):
        y = oracle.rmsnorm(np.full(n, c), None, eps)
        assert np.allclose(y, c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    x = np.random.default_rng(1).normal(size=n)
    y = oracle.rmsnorm(x, None, 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-14          # unit mean square
    assert np.allclose(oracle.rmsnorm(7.5 * x, None, 0.0), y, rtol=1e-14, atol=0)
    g = np.linspace(0.5, 2.0, n)
    assert np.allclose(oracle.rmsnorm(x, g, 0.0), y * g, rtol=1e-14, atol=0)


def test_rope_rotate_half_pairs_and_frequencies():
    hd, theta = 64, 1e6
    h = hd // 2
    for p in (0, 1, 7, 1000):
        e0 = np.zeros(hd); e0[0] = 1.0
        v = oracle.rope(e0, p, theta)
        # frequency 1 on the first pair, which is (0, hd/2) -- not (0, 1)
        assert np.allclose(v[[0, h]], [math.cos(p), math.sin(p)], atol=1e-15)
        assert np.count_nonzero(np.abs(v) > 1e-15) <= 2
        el = np.zeros(hd); el[h - 1] = 1.0
        w = oracle.rope(el, p, theta)
        f = theta ** (-2.0 * (h - 1) / hd)
        assert np.allclose(w[[h - 1, hd - 1]], [math.cos(p * f), math.sin(p * f)], atol=1e-15)


def test_rope_norm_identity_and_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=128), rng.normal(size=128)
    assert np.allclose(oracle.rope(q, 0), q, atol=0)
    for p in (3, 555):
        assert abs(np.linalg.norm(oracle.rope(q, p)) - np.linalg.norm(q)) < 1e-12
    d1 = oracle.rope(q, 10) @ oracle.rope(k, 4)
    d2 = oracle.rope(q, 106) @ oracle.rope(k, 100)
    d3 = oracle.rope(q, 11) @ oracle.rope(k, 4)
    assert abs(d1 - d2) < 1e-10 and abs(d1 - d3) > 1e-6


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    hd = 16
    q = rng.normal(size=hd)
    K = rng.normal(size=(5, hd))
    V = rng.normal(size=(5, hd))
    # one key: output is its value
    assert np.allclose(oracle.attention(q, K[:1], V[:1]), V[0], atol=1e-15)
    # identical keys or a zero query: plain mean of the values
    assert np.allclose(oracle.attention(q, np.repeat(K[:1], 5, 0), V), V.mean(0), atol=1e-14)
    assert np.allclose(oracle.attention(np.zeros(hd), K, V), V.mean(0), atol=1e-14)
    # key order does not matter
    perm = [3, 0, 4, 1, 2]
    assert np.allclose(oracle.attention(q, K[perm], V[perm]), oracle.attention(q, K, V),
                       atol=1e-14)
    # two keys, closed form with the 1/sqrt(hd) scale: weight = sigmoid(a/sqrt(hd))
    a = 3.0
    qq = np.zeros(hd); qq[0] = a
    KK = np.zeros((2, hd)); KK[0, 0] = 1.0
    VV = np.zeros((2, hd)); VV[0, 1] = 1.0; VV[1, 2] = 1.0
    w = 1.0 / (1.0 + math.exp(-a / math.sqrt(hd)))
    out = oracle.attention(qq, KK, VV)
    assert abs(out[1] - w) < 1e-15 and abs(out[2] - (1 - w)) < 1e-15
    # a dominant key selects its value
    qd = 200.0 * K[2] / np.linalg.norm(K[2])
    Kn = K / np.linalg.norm(K, axis=1, keepdims=True)
    assert np.allclose(oracle.attention(qd, Kn, V), V[2], atol=1e-6)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    for x in (0.3, 2.0, 7.5):
        assert abs(oracle.silu(x) - oracle.silu(-x) - x) < 1e-14   # x*s(x) + x*s(-x) = x
    assert abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu(-40.0)) < 1e-12


def test_argmax_lowest_index_on_ties():
    assert oracle.argmax([1.0, 3.0, 3.0, 2.0]) == 1
    assert oracle.argmax([5.0, 5.0]) == 0
    assert oracle.argmax([-1.0, -0.5, -0.5, -2.0]) == 1
    assert oracle.argmax([0.0, float("nan")]) == -1
    rng = np.random.default_rng(4)
    for _ in range(200):
        x = rng.integers(0, 4, size=9).astype(np.float64)
        assert oracle.argmax(x) == min(i for i in range(9) if x[i] == x.max())


@pytest.mark.parametrize("V,K", [(2, 1), (2, 2), (2, 3), (2, 4), (3, 1), (3, 2), (3, 3)])
def test_accept_brute_force(V, K):
    """m = the first i (0-based) with d_{i+1} != a_i, or K if none -- for
    every (d, a) in V^K x V^(K+1)."""
    for d in itertools.product(range(V), repeat=K):
        for a in itertools.product(range(V), repeat=K + 1):
            bad = [i for i in range(K) if d[i] != a[i]]
            want = bad[0] if bad else K
            assert oracle.accept(d, a) == want

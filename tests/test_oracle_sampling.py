"""Pins of the oracle's sampling at T > 0 (rejection sampling; HN item page
and atlas.scime.ai page, "Limitations"): the counter-based generator
against its published known answers, the categorical draw against its
closed form, and the acceptance rule against the property that makes it
lossless -- the first emitted token is distributed exactly as the AR
distribution p_0, whatever the draft distribution q (exact integration over
the uniforms on a fine grid)."""
import json
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_philox_known_answers():
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "philox4x32_10_kat.json")))["cases"]
    for c in cases:
        got = oracle.philox4x32_10([int(x, 16) for x in c["ctr"]], [int(x, 16) for x in c["key"]])
        assert [f"{v:08x}" for v in got] == c["out"]


def test_uniform_is_24_bits_of_the_first_word():
    seed, step, purpose, index, seq = 0x1234567890ABCDEF, 7, 2, 5, 3
    x0 = oracle.philox4x32_10([index, seq, step, purpose], [seed & 0xFFFFFFFF, seed >> 32])[0]
    assert oracle.uniform(seed, step, purpose, index, seq) == (int(x0) >> 8) / 2.0 ** 24


def test_draw_matches_cdf_intervals():
    w = np.array([0.0, 2.0, 0.5, 0.0, 1.5, 4.0])
    cdf = np.cumsum(w) / w.sum()
    n = 4000
    us = (np.arange(n) + 0.5) / n
    got = np.array([oracle.draw(w, u) for u in us])
    for j in range(w.size):
        lo = cdf[j - 1] if j else 0.0
        assert np.all(got[(us > lo) & (us < cdf[j])] == j)
    assert not np.isin(got, [0, 3]).any()            # zero weights are never drawn
    assert oracle.draw(np.zeros(3), 0.5) == -1


def test_sample_logits_temperature():
    z = np.array([0.3, 2.0, -1.0, 1.9])
    for T in (0.5, 1.0, 3.0):
        p = np.exp((z - z.max()) / T)
        p /= p.sum()
        us = (np.arange(2000) + 0.5) / 2000
        frac = np.bincount([oracle.sample_logits(z, T, u) for u in us], minlength=4) / len(us)
        assert np.abs(frac - p).max() < 1e-3
    # a very low temperature is greedy
    assert all(oracle.sample_logits(z, 1e-3, u) == 1 for u in (0.0, 0.5, 0.999))


@pytest.mark.parametrize("seed", [0, 1])
def test_first_emitted_token_is_distributed_as_p0(seed):
    """K = 1, V = 5: integrate the acceptance rule over the draft d_1 ~ q_1
    and over both uniforms on a midpoint grid; the first emitted token (d_1
    if accepted, else the final token) has distribution p_0, the second
    (after an acceptance: the bonus) distribution p_1."""
    rng = np.random.default_rng(seed)
    V, T = 5, 0.8
    pz = rng.normal(size=(2, V)) * 1.5
    qz = rng.normal(size=(1, V)) * 1.5
    p0 = np.exp(pz[0] / T) / np.exp(pz[0] / T).sum()
    p1 = np.exp(pz[1] / T) / np.exp(pz[1] / T).sum()
    q1 = np.exp(qz[0] / T) / np.exp(qz[0] / T).sum()
    n = 300
    grid = (np.arange(n) + 0.5) / n
    first = np.zeros(V)
    bonus = np.zeros(V)
    acc = 0.0
    for d in range(V):
        for ua in grid:
            for uf in grid:
                m, tok = oracle.spec_accept(pz, qz, [d], T, [ua], uf)
                wgt = q1[d] / (n * n)
                if m == 1:
                    first[d] += wgt
                    bonus[tok] += wgt
                    acc += wgt
                else:
                    first[tok] += wgt
    assert np.abs(first - p0).max() < 5e-3
    # acceptance probability sum_d min(q, p) and the bonus distribution
    assert abs(acc - np.minimum(q1, p0).sum()) < 5e-3
    assert np.abs(bonus / acc - p1).max() < 5e-3


def test_acceptance_rule_cases():
    V, T = 3, 1.0
    pz = np.log(np.array([[0.5, 0.3, 0.2], [0.1, 0.1, 0.8]]))
    qz = np.log(np.array([[0.25, 0.6, 0.15]]))
    # p(0)/q(0) = 2: always accepted, then the bonus from p_1
    assert oracle.spec_accept(pz, qz, [0], T, [0.999], 0.95) == (1, 2)
    # p(1)/q(1) = 0.5: accepted for u < 0.5 only
    assert oracle.spec_accept(pz, qz, [1], T, [0.49], 0.0)[0] == 1
    m, tok = oracle.spec_accept(pz, qz, [1], T, [0.51], 0.0)
    # residual max(0, p - q) = [0.25, 0, 0.05]: u = 0 draws token 0, u = 0.9 token 2
    assert m == 0 and tok == 0
    assert oracle.spec_accept(pz, qz, [1], T, [0.51], 0.9) == (0, 2)
    # a draft that is not a token is never accepted
    assert oracle.spec_accept(pz, qz, [7], T, [0.0], 0.0)[0] == 0

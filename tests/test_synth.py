"""The seeded input generator: Philox4x32-10 known answers, the compiled host
generator against the numpy specification, and the value maps."""
import json
import os

import numpy as np
import pytest

import synth
from synth import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    cases = json.load(open(os.path.join(GOLD, "philox4x32_10_kat.json")))["cases"]
    for c in cases:
        ctr = [np.array([int(x, 16)], np.uint64) for x in c["ctr"]]
        k0, k1 = (int(x, 16) for x in c["key"])
        out = synth.philox4x32_10(*ctr, k0, k1)
        assert [format(int(o[0]), "08x") for o in out] == c["out"]


def test_host_generator_matches_spec():
    for start in (0, 123456789, (1 << 32) - 3):
        a = synth.normal_f32(5000, 11, 42, 0.02, start=start)
        b = np.empty(5000, np.float32)
        synth.host_fill_normal(b, 11, 42, 0.02, start=start)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        c = np.empty(5000, np.uint16)
        synth.host_fill_normal(c, 11, 42, 0.02, start=start)
        assert np.array_equal(synth.f32_to_bf16_bits(a), c)


def test_normal_moments():
    x = synth.normal_f32(1 << 20, 0, 7, 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() - 0.02) < 1e-4
    # Irwin-Hall(8) tails are bounded at sqrt(24) sigma
    assert np.abs(x).max() <= 0.02 * np.sqrt(24.0) + 1e-6


def test_bf16_rounding_nearest_even():
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 1 + 2 ** -8 + 2 ** -20], np.float32)
    got = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(v))
    assert got.tolist() == [1.0, 1.0, 1 + 2 ** -6, -2.5, 1 + 2 ** -7]


def test_tokens_range_and_spread():
    t = synth.tokens(100000, 151936, 1, 0)
    assert t.min() >= 0 and t.max() < 151936
    assert abs(t.mean() / 151936 - 0.5) < 0.01


def test_planting_lengths_laws():
    a = workloads.plant_lengths(400, 2, 32, "geom6")
    assert a.min() >= 0 and a.max() <= 32
    assert 5.0 < a.mean() < 7.0          # clipped Geom(1/7): 5.957
    u = workloads.plant_lengths(400, 2, 32, "uniform32")
    assert u.min() >= 0 and u.max() <= 32 and 14.0 < u.mean() < 18.0


def test_planted_drafts_accept_exactly_a():
    rng = np.random.default_rng(0)
    V, K, steps, B = 50, 8, 30, 3
    traj = rng.integers(0, V, size=(B, 400)).astype(np.int32)
    a = workloads.plant_lengths(steps, B, K, "geom6")
    d = workloads.plant_drafts(traj, 1, a, K, V)
    for b in range(B):
        e = 1
        for s in range(steps):
            t = traj[b, e:e + K + 1]
            k = int(a[s, b])
            m = 0
            while m < K and d[s, b, m] == t[m]:
                m += 1
            assert m == k
            assert d[s, b].min() >= 0 and d[s, b].max() < V
            e += k + 1

"""Pins of the oracle's bf16 rounding points.

The pages give the model as a frozen Qwen3-8B backbone with a diffusion
attention path (atlas.scime.ai page, "Approach"), run in bf16; the reading
taken for its precision is: bf16 weights, an fp32 (here float64) residual
stream, and a bf16 rounding (fp32 first, then nearest even) at every GEMM
input (the attention-norm, FFN-norm and final-norm outputs, the attention
output, the SwiGLU product), at q and k after QK-norm and RoPE, and at the
cached / block K and V.

Each test composes one or two bf16 layers from numpy and the textbook
formulas (RMSNorm, rotate-half RoPE, softmax attention, SiLU), with the
bf16 rounding written out independently of the oracle, and requires the
oracle's logits to agree to 1e-9.  Every gain is drawn away from 1, so a
frozen tensor used in place of a diffusion one, or a gain dropped, fails as
well.  The mutation test compiles copies of the oracle with one rounding
step removed at a time and checks that some composition then fails: no
rounding point is left unpinned.
"""
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits
from synth import workloads
from tests import helpers as H

TOL = 1e-9


def bf16(x):
    """Round to bf16 the way the model stores values: float64 -> fp32
    (nearest even), then fp32 -> bf16 (nearest even on the upper 16 bits)."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_bf16_rounding_helper_matches_definition():
    # halfway cases go to even; values land on the bf16 grid
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -3.0, 0.1])
    assert np.array_equal(bf16(x)[:5], [1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7, -3.0])
    assert bf16(x)[5] == oracle.round_bf16(0.1)


def rms(x, g, eps):
    return x / np.sqrt((x * x).mean(-1, keepdims=True) + eps) * g


def rope_rows(x, pos, theta):
    """Rotate-half RoPE of x [..., hd] at position pos."""
    hd = x.shape[-1]
    h = hd // 2
    ang = pos * theta ** (-2.0 * np.arange(h) / hd)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], -1)


def attend(q, K, V):
    s = K @ q / np.sqrt(q.size)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


class Ref:
    """A numpy composition of the bf16 model with the rounding points
    switchable (all on = the reading; the oracle must match it)."""

    def __init__(self, shp, w, rnd=bf16):
        self.s = shp
        self.rnd = rnd
        self.T = lambda t: H.as_f64(shp, H.tensor(shp, w, t))
        self.Lt = lambda l, j: H.as_f64(shp, H.layer_tensor(shp, w, l, j))

    def qkv(self, l, h, pos, frozen):
        s = self.s
        sq, sk, sv, sqn, skn = (2, 3, 4, 6, 7) if frozen else (8, 9, 10, 12, 13)
        u = self.rnd(rms(h, self.Lt(l, 0), s.eps))
        R = len(pos)
        q = (u @ self.Lt(l, sq).reshape(s.hq * s.hd, s.d).T).reshape(R, s.hq, s.hd)
        k = (u @ self.Lt(l, sk).reshape(s.hkv * s.hd, s.d).T).reshape(R, s.hkv, s.hd)
        v = (u @ self.Lt(l, sv).reshape(s.hkv * s.hd, s.d).T).reshape(R, s.hkv, s.hd)
        for r, p in enumerate(pos):
            q[r] = rope_rows(rms(q[r], self.Lt(l, sqn), s.eps), p, s.theta)
            k[r] = rope_rows(rms(k[r], self.Lt(l, skn), s.eps), p, s.theta)
        return self.rnd(q), self.rnd(k), self.rnd(v)

    def tail(self, l, h, o, frozen):
        s = self.s
        o = self.rnd(o.reshape(len(h), -1))
        h = h + o @ self.Lt(l, 5 if frozen else 11).reshape(s.d, s.hq * s.hd).T
        u = self.rnd(rms(h, self.Lt(l, 1), s.eps))
        gate = u @ self.Lt(l, 14).reshape(s.F, s.d).T
        up = u @ self.Lt(l, 15).reshape(s.F, s.d).T
        act = self.rnd(gate / (1.0 + np.exp(-gate)) * up)
        return h + act @ self.Lt(l, 16).reshape(s.d, s.F).T

    def logits(self, h):
        s = self.s
        z = self.rnd(rms(h, self.T(2), s.eps))
        return z @ self.T(1).reshape(s.V, s.d).T

    def frozen(self, tokens):
        """Causal AR rows at positions 0..R-1; returns logits and the
        per-layer cache (K, V) [R, hkv, hd]."""
        s = self.s
        grp = s.hq // s.hkv
        h = self.T(0).reshape(s.V, s.d)[tokens]
        cache = []
        pos = list(range(len(tokens)))
        for l in range(s.L):
            q, k, v = self.qkv(l, h, pos, True)
            cache.append((k, v))
            o = np.zeros((len(tokens), s.hq, s.hd))
            for r in pos:
                for i in range(s.hq):
                    o[r, i] = attend(q[r, i], k[:r + 1, i // grp], v[:r + 1, i // grp])
            h = self.tail(l, h, o, True)
        return self.logits(h), cache

    def masks(self, cache, K):
        """K mask rows at positions n+1..n+K (n + 1 = cached slots), each
        seeing every cached slot and the whole block."""
        s = self.s
        grp = s.hq // s.hkv
        n1 = cache[0][0].shape[0]
        h = np.tile(self.T(3), (K, 1))
        pos = list(range(n1, n1 + K))
        for l in range(s.L):
            q, k, v = self.qkv(l, h, pos, False)
            keys = np.concatenate([cache[l][0], k])
            vals = np.concatenate([cache[l][1], v])
            o = np.zeros((K, s.hq, s.hd))
            for r in range(K):
                for i in range(s.hq):
                    o[r, i] = attend(q[r, i], keys[:, i // grp], vals[:, i // grp])
            h = self.tail(l, h, o, False)
        return self.logits(h)


def gains_away_from_one(shp, w, seed=31):
    w = w.copy()
    lay, _ = oracle.weight_layout(shp)
    rng = np.random.default_rng(seed)
    for t, off, n, gain in lay:
        if gain:
            g = (1.0 + 0.25 * rng.standard_normal(n)).astype(np.float32)
            w[off:off + n] = f32_to_bf16_bits(g)
    return w


@pytest.fixture(scope="module")
def bf16_model():
    shp = H.shape("small")                       # bf16, d 512, 8 q / 2 kv heads of 128, 2 layers
    w = gains_away_from_one(shp, H.weights(shp))
    return shp, w


def check_frozen(shp, w):
    """Prefill rows 0..R-1 (frozen view, causal, K/V cached)."""
    toks = workloads.prompts(1, 4, shp.V, seed=32)[0]
    lg, _ = oracle.Model(shp, w).seq(8).ar_rows(toks, 0)
    want, _ = Ref(shp, w).frozen(toks)
    return np.abs(lg - want).max()


def check_masks(shp, w, K=3):
    """Mask rows of the diffusion view over a cache of the prompt plus the
    staged anchor."""
    toks = workloads.prompts(1, 4, shp.V, seed=33)[0]
    m = oracle.Model(shp, w)
    seq = m.seq(16)
    n = len(toks) - 1
    seq.ar_rows(toks, 0)                          # slots 0..n: prompt rows and the anchor
    lg, _ = seq.draft_rows(n, K)
    ref = Ref(shp, w)
    _, cache = ref.frozen(toks)
    want = ref.masks(cache, K)
    return np.abs(lg - want).max()


def test_bf16_frozen_rows_composition(bf16_model):
    assert check_frozen(*bf16_model) < TOL


def test_bf16_mask_rows_composition(bf16_model):
    assert check_masks(*bf16_model) < TOL


def test_rounding_points_matter_at_this_tolerance(bf16_model):
    """Dropping any one rounding point from the numpy composition moves the
    logits far beyond the tolerance (so the compositions above pin each)."""
    shp, w = bf16_model
    toks = workloads.prompts(1, 4, shp.V, seed=32)[0]
    want, _ = Ref(shp, w).frozen(toks)
    got, _ = Ref(shp, w, rnd=lambda x: np.asarray(x, np.float64)).frozen(toks)
    assert np.abs(got - want).max() > 1e-5


# ---------------------------------------------------------------- mutation
def _rounding_sites(src):
    """Line numbers of the oracle's arithmetic rounding statements (the
    attention-tap copies are not arithmetic and are skipped)."""
    out = []
    for i, line in enumerate(src.splitlines()):
        if re.match(r"\s*store_round\(m, (\w+),", line) and "tap" not in line:
            out.append(i)
    return out


def test_every_rounding_point_is_pinned(tmp_path, bf16_model):
    """Compile the oracle with one rounding statement removed at a time; for
    every such mutant, one of the compositions must fail."""
    shp, w = bf16_model
    src = open(oracle.SRC_PATH).read()
    sites = _rounding_sites(src)
    # normed rows (attention, FFN, final), q, k, v, attention output, SwiGLU product
    assert len(sites) == 8, sites
    lines = src.splitlines()
    for j, i in enumerate(sites):
        mut = list(lines)
        mut[i] = "  /* rounding removed */"
        cpath = tmp_path / f"mut{j}.c"
        cpath.write_text("\n".join(mut) + "\n")
        so = str(tmp_path / f"libmut{j}.so")
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", so,
                               str(cpath), "-lm"])
        with oracle.using_library(so):
            err = max(check_frozen(shp, w), check_masks(shp, w))
        assert err > 1e-6, (lines[i].strip(), err)
        os.remove(so)


class Ref32(Ref):
    """The same composition in float32: float32 weights (exact: they are
    bf16), residual stream, matrix products and softmax, with the same bf16
    rounding points -- the arithmetic an fp32-accumulating implementation of
    the reading performs, written independently of the GPU kernels."""

    def __init__(self, shp, w):
        super().__init__(shp, w)
        t64, l64, memo = self.T, self.Lt, {}

        def T(t):
            if ("T", t) not in memo:
                memo[("T", t)] = t64(t).astype(np.float32)
            return memo[("T", t)]

        def Lt(l, j):
            if ("L", l, j) not in memo:
                memo[("L", l, j)] = l64(l, j).astype(np.float32)
            return memo[("L", l, j)]

        self.T, self.Lt = T, Lt
        self.rnd = lambda x: bf16(x).astype(np.float32)


def last_row_logits(ref, toks, dtype):
    """Prefill of toks through ref's layers (frozen view, causal); the last
    row's logits."""
    s = ref.s
    grp = s.hq // s.hkv
    h = ref.T(0).reshape(s.V, s.d)[toks].astype(dtype)
    pos = list(range(len(toks)))
    for l in range(s.L):
        q, k, v = (x.astype(dtype) for x in ref.qkv(l, h, pos, True))
        o = np.zeros((len(toks), s.hq, s.hd), dtype)
        for r in pos:
            for i in range(s.hq):
                o[r, i] = attend(q[r, i], k[:r + 1, i // grp], v[:r + 1, i // grp])
        h = ref.tail(l, h, o, True).astype(dtype)
    z = ref.rnd(rms(h[-1:], ref.T(2), s.eps))
    return (z @ ref.T(1).reshape(s.V, s.d).T)[0].astype(np.float64)


@pytest.mark.slow
def test_float32_accumulation_alone_moves_full_width_logits_by_about_the_tolerance():
    """Why the free-running GPU comparisons sit near 2e-2 at the Qwen3-8B
    width: one layer (d 4096, 32/8 heads, SwiGLU 12288, vocabulary 151936), a
    52-token prompt.  The float64 composition gives the oracle's prefill
    logits exactly; the float32 composition, with the same rounding points,
    differs from them by about 1e-2 at the maximum over the 151936 logits
    (measured 0.0186, mean 0.0031): float32 sums flip some bf16 roundings,
    and the flips carry through the norms to the logits.  The GPU's
    deviations at these prompt lengths (0.0096-0.0212, mean about 0.003) are
    of the same size."""
    shp = H.shape("qwen3_8b", L=1)
    w = H.weights(shp)
    toks = workloads.prompts(1, 52, shp.V, seed=21)[0]
    _, lo = oracle.Model(shp, w).seq(64).prefill(toks, want_logits=True)
    lo = np.asarray(lo, np.float64).reshape(-1)[-shp.V:]
    assert np.abs(last_row_logits(Ref(shp, w), toks, np.float64) - lo).max() < TOL
    d32 = np.abs(last_row_logits(Ref32(shp, w), toks, np.float32) - lo)
    assert 5e-3 < d32.max() < 3e-2, d32.max()
    assert d32.mean() < 5e-3, d32.mean()

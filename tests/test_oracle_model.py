"""Pins of the oracle's model and step against what the pages fix:
the lossless guarantee, the acceptance rule, cache growth, the draft pass
writing nothing to the cache, the K = 0 reduction, and structural
reductions of the diffusion view."""
import numpy as np
import pytest

import oracle
from synth import workloads
from tests import helpers as H


@pytest.fixture(scope="module")
def tiny():
    shp = H.shape("tiny")
    w = H.weights(shp)
    return shp, w, oracle.Model(shp, w)


@pytest.fixture(scope="module")
def small():
    shp = H.shape("small")
    w = H.weights(shp)
    return shp, w, oracle.Model(shp, w)


def test_tiny_orthrus_equals_greedy_ar_128(tiny):
    """Lossless guarantee on the tiny fp32 model: 128 tokens (HN item page
    'Idea'; abstract on the opentrain.ai page)."""
    shp, w, m = tiny
    prompt = workloads.prompts(1, 64, shp.V)[0]
    ar = m.ar_generate(prompt, 128)
    out, acc, lens = m.generate(prompt, 128, shp.K)
    assert np.array_equal(out, ar)
    # cache growth: len before step s = P + emitted_before - 1
    emitted = 1
    for s in range(len(acc)):
        assert lens[s] == 64 + emitted - 1
        emitted += acc[s] + 1


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
def test_lossless_for_any_diffusion_weights(tiny, seed):
    shp, w, _ = tiny
    m = oracle.Model(shp, H.reseed_diffusion(shp, w, 100 + seed))
    prompt = workloads.prompts(1, 24, shp.V, seed=seed)[0]
    assert np.array_equal(m.generate(prompt, 40, shp.K)[0], m.ar_generate(prompt, 40))


def test_lossless_with_zero_diffusion_weights(tiny):
    shp, w, _ = tiny
    w0 = w.copy()
    for l in range(shp.L):
        for s in H.DIFF_SLOTS:
            H.layer_tensor(shp, w0, l, s)[:] = 0
    m = oracle.Model(shp, w0)
    prompt = workloads.prompts(1, 20, shp.V)[0]
    assert np.array_equal(m.generate(prompt, 30, shp.K)[0], m.ar_generate(prompt, 30))


@pytest.mark.parametrize("model", ["tiny", "small"])
@pytest.mark.parametrize("kind", ["all", "none", "partial"])
def test_planted_drafts_lossless_and_accept(request, model, kind):
    """Planted drafts force any accept length; the output stays greedy AR and
    each step accepts exactly the planted length (contract planting)."""
    shp, w, m = request.getfixturevalue(model)
    P, n_new, K = 12, 60, shp.K
    prompt = workloads.prompts(1, P, shp.V, seed=9)[0]
    traj = m.ar_generate(prompt, n_new + 2 * K + 2)[None, :]
    steps = n_new
    if kind == "all":
        a = np.full((steps, 1), K, np.int32)
    elif kind == "none":
        a = np.zeros((steps, 1), np.int32)
    else:
        a = workloads.plant_lengths(steps, 1, K, "geom6")
    # trajectories must cover the planted steps: only use as many as fit
    e, s_ok = 1, 0
    while s_ok < steps and e + a[s_ok, 0] + 1 + K + 1 <= traj.shape[1]:
        e += a[s_ok, 0] + 1
        s_ok += 1
    a = a[:s_ok]
    planted = workloads.plant_drafts(traj, 1, a, K, shp.V)[:, 0, :]
    out, acc, lens = m.generate(prompt, n_new, K, planted=planted, max_steps=s_ok)
    got = len(out) if len(acc) == 0 else min(n_new, 1 + int((acc + 1).sum()))
    assert np.array_equal(out[:got], traj[0, :got])
    assert np.array_equal(acc, a[:len(acc), 0])


def test_step_invariants_and_draft_writes_nothing(tiny):
    """Per step: len grows by m+1, commit indices are [n, n+m], pass 1 leaves
    cache[0, n) untouched, the emitted tokens are d_1..d_m then a_m."""
    shp, w, m = tiny
    K = shp.K
    prompt = workloads.prompts(1, 30, shp.V, seed=4)[0]
    seq = m.seq(30 + 200)
    pending = seq.prefill(prompt)
    assert seq.len == 30
    for _ in range(12):
        n = seq.len
        c0 = seq.checksum(n)
        lg, d = seq.draft_rows(n - 1, K)      # a draft-only pass over the committed cache
        assert seq.checksum(n) == c0 and seq.len == n
        r = seq.step(pending, K)
        mm = r["m"]
        assert r["n"] == n and r["len"] == n + 1 + mm
        assert seq.checksum(n) == c0                      # committed prefix unchanged
        assert np.array_equal(r["emitted"][:mm], r["drafts"][:mm])
        assert r["emitted"][mm] == r["ar"][mm]
        assert mm == oracle.accept(r["drafts"], r["ar"])
        assert r["pending"] == r["ar"][mm]
        pending = r["pending"]


def test_k0_is_plain_greedy(tiny):
    shp, w, m = tiny
    prompt = workloads.prompts(1, 16, shp.V, seed=5)[0]
    out, acc, _ = m.generate(prompt, 25, 0)
    assert np.array_equal(out, m.ar_generate(prompt, 25))
    assert (acc == 0).all()


def _tied(shp, w):
    """Diffusion projections and gains := the frozen ones."""
    w = w.copy()
    for l in range(shp.L):
        for fro, dif in ((2, 8), (3, 9), (4, 10), (5, 11), (6, 12), (7, 13)):
            H.layer_tensor(shp, w, l, dif)[:] = H.layer_tensor(shp, w, l, fro)
    return w


@pytest.mark.parametrize("model", ["tiny", "small"])
def test_draft_view_reduces_to_verify_when_tied(request, model):
    """With the diffusion weights tied to the frozen ones, the true next tokens
    as block inputs and a causal block mask, the mask rows see exactly what
    the verify rows see, so their logits are identical."""
    shp, w, _ = request.getfixturevalue(model)
    m = oracle.Model(shp, _tied(shp, w))
    K = 6
    prompt = workloads.prompts(1, 10, shp.V, seed=6)[0]
    seq = m.seq(64)
    pending = seq.prefill(prompt)
    n = seq.len
    nxt = np.array([3, 17, 5, 99 % shp.V, 42, 7], np.int32)
    seq.ar_rows(np.array([pending], np.int32), n)      # anchor staged at slot n
    ld, _ = seq.draft_rows(n, K, in_tokens=nxt, causal=True)
    lv, _ = seq.ar_rows(nxt, n + 1)
    assert np.array_equal(ld, lv)


def test_block_is_bidirectional():
    # one layer: block K/V come straight from the inputs, so the last row's
    # keys are the same under both masks
    shp = H.shape("tiny", L=1)
    m = oracle.Model(shp, H.weights(shp))
    K = 5
    prompt = workloads.prompts(1, 9, shp.V, seed=7)[0]
    seq = m.seq(40)
    seq.prefill(prompt)
    n = seq.len - 1
    toks = np.array([1, 2, 3, 4, 5], np.int32)
    lb, _ = seq.draft_rows(n, K, in_tokens=toks, causal=False)
    lc, _ = seq.draft_rows(n, K, in_tokens=toks, causal=True)
    assert np.array_equal(lb[K - 1], lc[K - 1])     # last row sees the whole block either way
    assert np.abs(lb[0] - lc[0]).max() > 1e-6       # first row sees later rows only if bidirectional


def test_gqa_head_grouping():
    """hq=4 over hkv=2 equals hq=4 over hkv=4 with each KV head duplicated for
    its two query heads: query head h reads KV head floor(h / (hq/hkv))."""
    a = H.shape("tiny", L=1)
    wa = H.weights(a)
    b = H.shape("tiny", L=1, hkv=4)
    lay_b, tot_b = oracle.weight_layout(b)
    wb = np.zeros(tot_b, np.float32)
    lay_a, _ = oracle.weight_layout(a)
    for (t, off, n, _), (tb, offb, nb, _) in zip(lay_a, lay_b):
        src = wa[off:off + n]
        if nb == n:
            wb[offb:offb + nb] = src
        else:                                           # K/V projection [hkv*hd][d]
            rows = src.reshape(a.hkv, a.hd, a.d)
            wb[offb:offb + nb] = np.repeat(rows, 2, axis=0).reshape(-1)
    prompt = workloads.prompts(1, 7, a.V, seed=8)[0]
    la = oracle.Model(a, wa).seq(16).ar_rows(prompt, 0)[0]
    lb = oracle.Model(b, wb).seq(16).ar_rows(prompt, 0)[0]
    assert np.allclose(la, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("model", ["tiny", "small"])
def test_residual_only_model_closed_form(request, model):
    """With every O and down projection zero, each row's logits are
    RMSNorm(E[x]) . W_lm (the bf16 model rounds the normed row to bf16)."""
    shp, w, _ = request.getfixturevalue(model)
    w0 = w.copy()
    for l in range(shp.L):
        for s in (5, 11, 16):
            H.layer_tensor(shp, w0, l, s)[:] = 0
    m = oracle.Model(shp, w0)
    toks = workloads.prompts(1, 5, shp.V, seed=10)[0]
    lg, am = m.seq(8).ar_rows(toks, 0)
    E = H.as_f64(shp, H.tensor(shp, w0, 0)).reshape(shp.V, shp.d)
    Wl = H.as_f64(shp, H.tensor(shp, w0, 1)).reshape(shp.V, shp.d)
    x = E[toks]
    z = x / np.sqrt((x * x).mean(1, keepdims=True) + shp.eps)
    if shp.bf16:
        z = np.vectorize(oracle.round_bf16)(z)
    want = z @ Wl.T
    assert np.allclose(lg, want, rtol=0, atol=1e-9)
    assert np.array_equal(am, want.argmax(1))


def test_one_layer_wiring_fp32():
    """One fp32 layer composed from the pinned primitives and numpy matmuls:
    the oracle's projections, QK-norm, RoPE positions, GQA, residuals and
    SwiGLU are wired as the definition says."""
    shp = H.shape("tiny", L=1)
    w = H.weights(shp)
    m = oracle.Model(shp, w)
    toks = workloads.prompts(1, 3, shp.V, seed=11)[0]
    lg, _ = m.seq(4).ar_rows(toks, 0)
    T = lambda t: H.as_f64(shp, H.tensor(shp, w, t))
    Lt = lambda s: H.as_f64(shp, H.layer_tensor(shp, w, 0, s))
    d, hd, hq, hkv = shp.d, shp.hd, shp.hq, shp.hkv
    h = T(0).reshape(shp.V, d)[toks]
    u = np.stack([oracle.rmsnorm(r, Lt(0), shp.eps) for r in h])
    q = u @ Lt(2).reshape(hq * hd, d).T
    k = u @ Lt(3).reshape(hkv * hd, d).T
    v = u @ Lt(4).reshape(hkv * hd, d).T
    q = q.reshape(3, hq, hd); k = k.reshape(3, hkv, hd); v = v.reshape(3, hkv, hd)
    for p in range(3):
        for i in range(hq):
            q[p, i] = oracle.rope(oracle.rmsnorm(q[p, i], Lt(6), shp.eps), p)
        for g in range(hkv):
            k[p, g] = oracle.rope(oracle.rmsnorm(k[p, g], Lt(7), shp.eps), p)
    o = np.zeros((3, hq, hd))
    for p in range(3):
        for i in range(hq):
            g = i // (hq // hkv)
            o[p, i] = oracle.attention(q[p, i], k[:p + 1, g], v[:p + 1, g])
    h = h + o.reshape(3, -1) @ Lt(5).reshape(d, hq * hd).T
    u = np.stack([oracle.rmsnorm(r, Lt(1), shp.eps) for r in h])
    gate = u @ Lt(14).reshape(shp.F, d).T
    up = u @ Lt(15).reshape(shp.F, d).T
    act = gate / (1 + np.exp(-gate)) * up
    h = h + act @ Lt(16).reshape(d, shp.F).T
    z = np.stack([oracle.rmsnorm(r, T(2), shp.eps) for r in h])
    want = z @ T(1).reshape(shp.V, d).T
    assert np.allclose(lg, want, rtol=0, atol=1e-10)


def test_one_layer_diffusion_wiring_fp32():
    """The mask rows of one fp32 layer composed from the pinned primitives
    and numpy matmuls: the mask embedding as input, the diffusion Q/K/V/O and
    QK-norm gains, RoPE at positions n+1..n+K, attention over the cache slots
    [0, n] (prompt plus the staged anchor) and every block key, and the
    shared norms, FFN and LM head.  Every gain is drawn away from 1, so a
    frozen gain or matrix used in place of a diffusion one changes the
    logits."""
    shp = H.shape("tiny", L=1)
    w = H.weights(shp).copy()
    lay, _ = oracle.weight_layout(shp)
    rng = np.random.default_rng(12)
    for t, off, n, gain in lay:
        if gain:
            w[off:off + n] = 1.0 + 0.25 * rng.standard_normal(n).astype(np.float32)
    m = oracle.Model(shp, w)
    K = 4
    prompt = workloads.prompts(1, 3, shp.V, seed=13)[0]
    seq = m.seq(16)
    pending = seq.prefill(prompt)
    n = seq.len
    seq.ar_rows(np.array([pending], np.int32), n)           # anchor at slot n
    lg, am = seq.draft_rows(n, K)

    T = lambda t: H.as_f64(shp, H.tensor(shp, w, t))
    Lt = lambda s: H.as_f64(shp, H.layer_tensor(shp, w, 0, s))
    d, hd, hq, hkv, grp = shp.d, shp.hd, shp.hq, shp.hkv, shp.hq // shp.hkv

    def qkv(h, pos, sq, sk, sv, sqn, skn):
        R = len(pos)
        u = np.stack([oracle.rmsnorm(r, Lt(0), shp.eps) for r in h])
        q = (u @ Lt(sq).reshape(hq * hd, d).T).reshape(R, hq, hd)
        k = (u @ Lt(sk).reshape(hkv * hd, d).T).reshape(R, hkv, hd)
        v = (u @ Lt(sv).reshape(hkv * hd, d).T).reshape(R, hkv, hd)
        for r, p in enumerate(pos):
            for i in range(hq):
                q[r, i] = oracle.rope(oracle.rmsnorm(q[r, i], Lt(sqn), shp.eps), p)
            for g in range(hkv):
                k[r, g] = oracle.rope(oracle.rmsnorm(k[r, g], Lt(skn), shp.eps), p)
        return q, k, v

    def tail(h, o, so):
        h = h + o.reshape(len(h), -1) @ Lt(so).reshape(d, hq * hd).T
        u = np.stack([oracle.rmsnorm(r, Lt(1), shp.eps) for r in h])
        gate = u @ Lt(14).reshape(shp.F, d).T
        up = u @ Lt(15).reshape(shp.F, d).T
        h = h + (gate / (1 + np.exp(-gate)) * up) @ Lt(16).reshape(d, shp.F).T
        z = np.stack([oracle.rmsnorm(r, T(2), shp.eps) for r in h])
        return z @ T(1).reshape(shp.V, d).T

    # the cache slots 0..n: frozen view over the prompt and the anchor token
    toks = np.append(prompt, pending)
    _, kc, vc = qkv(T(0).reshape(shp.V, d)[toks], range(n + 1), 2, 3, 4, 6, 7)
    # the block: K copies of the mask embedding at positions n+1..n+K
    hb = np.tile(T(3), (K, 1))
    qb, kb, vb = qkv(hb, range(n + 1, n + 1 + K), 8, 9, 10, 12, 13)
    keys, vals = np.concatenate([kc, kb]), np.concatenate([vc, vb])
    o = np.zeros((K, hq, hd))
    for r in range(K):
        for i in range(hq):
            o[r, i] = oracle.attention(qb[r, i], keys[:, i // grp], vals[:, i // grp])
    want = tail(hb, o, 11)
    assert np.allclose(lg, want, rtol=0, atol=1e-10)
    assert np.array_equal(am, want.argmax(1))


@pytest.mark.parametrize("model", ["tiny", "small"])
def test_layer_entry_points_compose_to_the_step(request, model):
    """The per-layer entry points, chained from the embeddings with a cache
    loaded slot by slot from another sequence, give exactly the logits of the
    whole-pass routines (anchor, mask and verify rows of one step)."""
    shp, w, m = request.getfixturevalue(model)
    K = 5
    prompt = workloads.prompts(1, 9, shp.V, seed=14)[0]
    a = m.seq(32)
    pending = a.prefill(prompt)
    n = a.len
    b = m.seq(32)
    for l in range(shp.L):
        k, v = a.read_kv(l, n)
        b.load_kv(l, k, v)
    b.len = n
    r = a.step(pending, K)
    E = H.as_f64(shp, H.tensor(shp, w, 0)).reshape(shp.V, shp.d)
    # anchor row at n, then the mask rows over [0, n] + block, then verify
    h = E[[pending]]
    for l in range(shp.L):
        h, _ = b.ar_layer(l, h, n)
    lg, am = m.final(h)
    assert np.array_equal(lg[0], r["logits_anchor"]) and am[0] == r["ar"][0]
    hm = np.tile(H.as_f64(shp, H.tensor(shp, w, 3)), (K, 1))
    for l in range(shp.L):
        hm, _ = b.draft_layer(l, hm, n)
    lg, am = m.final(hm)
    assert np.array_equal(lg, r["logits_draft"]) and np.array_equal(am, r["drafts"])
    hv = E[r["drafts"]]
    for l in range(shp.L):
        hv, _ = b.ar_layer(l, hv, n + 1)
    lg, am = m.final(hv)
    assert np.array_equal(lg, r["logits_verify"]) and np.array_equal(am, r["ar"][1:])


def test_layer_tail_entry_point_matches_the_layer(tiny):
    """oc_layer_tail from a layer's own attention output reproduces the
    whole layer (frozen and diffusion views)."""
    shp, w, m = tiny
    prompt = workloads.prompts(1, 6, shp.V, seed=15)[0]
    seq = m.seq(32)
    seq.prefill(prompt)
    n = seq.len
    E = H.as_f64(shp, H.tensor(shp, w, 0)).reshape(shp.V, shp.d)
    h = E[[3]]
    h1, o = seq.ar_layer(0, h, n)
    assert np.array_equal(m.layer_tail(0, h, o), h1)
    hm = np.tile(H.as_f64(shp, H.tensor(shp, w, 3)), (4, 1))
    hm1, om = seq.draft_layer(0, hm, n)
    assert np.array_equal(m.layer_tail(0, hm, om, diffusion=True), hm1)
    assert not np.array_equal(m.layer_tail(0, hm, om, diffusion=False), hm1)


@pytest.mark.parametrize("model", ["tiny", "small"])
def test_any_block_size_schedule_is_lossless(request, model):
    """Dynamic K (openai-hub.net article, "Future Directions", item 1): a
    different block size every step, 0 and the full K included, still emits
    exactly greedy AR decoding, grows the cache by m+1 and accepts m <= k."""
    shp, w, m = request.getfixturevalue(model)
    sched = [shp.K, 3, 0, 5, 1, shp.K, 2, 7 % (shp.K + 1), 0, 4]
    prompt = workloads.prompts(1, 11, shp.V, seed=16)[0]
    n_new = 40
    want = m.ar_generate(prompt, n_new)
    seq = m.seq(11 + n_new + shp.K + 4)
    pend = seq.prefill(prompt)
    out = [pend]
    s = 0
    while len(out) < n_new:
        k = sched[s % len(sched)]
        n = seq.len
        r = seq.step(pend, k)
        assert 0 <= r["m"] <= k and seq.len == n + 1 + r["m"]
        out.extend(r["emitted"].tolist())
        pend = r["pending"]
        s += 1
    assert np.array_equal(np.array(out[:n_new]), want)


def test_two_step_denoised_drafts_are_lossless(tiny):
    """Drafts from a second diffusion pass over the first pass's argmax tokens
    (the 2-step variant) change only how much is accepted: the output is
    still greedy AR decoding."""
    shp, w, m = tiny
    K = shp.K
    prompt = workloads.prompts(1, 10, shp.V, seed=17)[0]
    n_new = 30
    seq = m.seq(10 + n_new + K + 4)
    pend = seq.prefill(prompt)
    out = [pend]
    while len(out) < n_new:
        n = seq.len
        seq.ar_rows(np.array([pend], np.int32), n)
        _, d1 = seq.draft_rows(n, K)
        _, d2 = seq.draft_rows(n, K, in_tokens=d1)
        r = seq.step(pend, K, planted=d2)
        out.extend(r["emitted"].tolist())
        pend = r["pending"]
    assert np.array_equal(np.array(out[:n_new]), m.ar_generate(prompt, n_new))

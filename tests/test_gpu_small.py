"""GPU parity on the small bf16 model (the bf16 MFMA kernels at the big
model's head size and GQA group): the draft/verify output equals the GPU's
own plain greedy decoding exactly; tokens, drafts and accept lengths equal
the oracle's wherever the oracle's top-1/top-2 margin exceeds the tolerance;
logits within 2e-2."""
import numpy as np
import pytest
import torch

from lossless_decoding_amd import _lib as C
from synth import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

TOL = 2e-2


@pytest.mark.parametrize("B", [1, 3])
def test_small_orthrus_equals_gpu_greedy(B):
    sh = workloads.SHAPES["small"]
    prompt = workloads.prompts(B, 40, sh["V"], seed=5)
    eng = U.engine("small", max_batch=B, max_ctx=1024)
    ar = U.engine("small", K=0, max_batch=B, max_ctx=1024)
    got, recs = eng.generate(prompt, 96, record=True)
    want, _ = ar.generate(prompt, 96)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kind", ["all", "none", "geom6", "uniform32"])
def test_small_planted_drafts(kind):
    """Planted drafts force the accept length; output stays greedy and every
    step accepts exactly the planted count (commit and discard paths)."""
    sh = workloads.SHAPES["small"]
    K, B = sh["K"], 2
    prompt = workloads.prompts(B, 24, sh["V"], seed=6)
    ar = U.engine("small", K=0, max_batch=B, max_ctx=2048)
    traj, _ = ar.generate(prompt, 400)
    steps = 8
    if kind == "all":
        a = np.full((steps, B), K, np.int32)
    elif kind == "none":
        a = np.zeros((steps, B), np.int32)
    else:
        a = workloads.plant_lengths(steps, B, K, kind)
    planted = workloads.plant_drafts(traj, 1, a, K, sh["V"])
    eng = U.engine("small", max_batch=B, max_ctx=2048)
    n_new = 1 + int((a + 1).sum(0).min())
    got, recs = eng.generate(prompt, n_new, planted=planted, record=True)
    assert np.array_equal(got, traj[:, :n_new])
    for s, r in enumerate(recs):
        assert np.array_equal(r["m"], a[s])
        assert np.array_equal(r["len"], r["n"] + 1 + a[s])


def test_small_anchor_and_verify_rows_bitwise_equal_plain_decoding():
    """Batch invariance: the anchor row (computed with 32 mask rows) and the
    verify rows (32 at once) give the same logits, bit for bit, as one-row
    greedy decoding of the same tokens."""
    sh = workloads.SHAPES["small"]
    K, V = sh["K"], sh["V"]
    prompt = workloads.prompts(1, 30, V, seed=7)
    ar = U.engine("small", K=0, max_ctx=512)
    lg_ar = torch.zeros(1, V, device="cuda")
    ar.set_debug(lg_ar, None, 1)
    ar.prefill(prompt)
    rows_ar = []
    toks = [int(ar.pending[0])]
    for _ in range(K + 1):
        ar.step()
        torch.cuda.synchronize()
        rows_ar.append(lg_ar[0].clone())
        toks.append(int(ar.pending[0]))
    eng = U.engine("small", max_ctx=512)
    lg = torch.zeros(K + 1, V, device="cuda")
    eng.set_debug(lg, None, K + 1)
    eng.prefill(prompt)
    eng.draft()
    torch.cuda.synchronize()
    assert torch.equal(lg[U.anchor_row(K)], rows_ar[0])   # anchor row
    eng.drafts[0].copy_(torch.tensor(toks[1:K + 1], dtype=torch.int32))
    eng.verify()
    torch.cuda.synchronize()
    for i in range(K):
        assert torch.equal(lg[i], rows_ar[i + 1]), i      # verify row i
    assert int(eng.accept[0]) == K


def test_small_step_parity_with_oracle():
    """Step by step against the oracle while the two agree on every token;
    a disagreement is only allowed at an oracle near-tie (margin <= tol) with
    the GPU choosing the oracle's runner-up, and ends the comparison."""
    sh = workloads.SHAPES["small"]
    K, V = sh["K"], sh["V"]
    prompt = workloads.prompts(1, 48, V, seed=8)
    om = U.oracle_model("small")
    seq = om.seq(600)
    pend_o, lg0 = seq.prefill(prompt[0], want_logits=True)
    eng = U.engine("small", max_ctx=600)
    lg = torch.zeros(K + 1, V, device="cuda")
    eng.set_debug(lg, None, K + 1)
    eng.prefill(prompt)
    assert int(eng.pending[0]) == pend_o or U.margin(lg0) <= TOL
    compared = 0
    for step in range(10):
        eng.draft()
        torch.cuda.synchronize()
        gd = lg.cpu().numpy().astype(np.float64)
        g_drafts = eng.drafts[0].cpu().numpy().copy()
        eng.verify()
        torch.cuda.synchronize()
        gv = lg[:K].cpu().numpy().astype(np.float64)
        eng.commit()
        torch.cuda.synchronize()
        r = seq.step(pend_o, K)
        assert np.abs(gd[U.anchor_row(K)] - r["logits_anchor"]).max() < TOL
        assert np.abs(gd[:K] - r["logits_draft"]).max() < TOL
        diverged = False
        for i in range(K):
            if g_drafts[i] != r["drafts"][i]:
                row = r["logits_draft"][i]
                assert U.margin(row) <= TOL and np.argsort(row)[-2] == g_drafts[i]
                diverged = True
                break
        if diverged:
            break
        # verify rows are comparable up to the accepted prefix and one more
        g_ar = eng.ar[0].cpu().numpy()
        m = r["m"]
        np.testing.assert_array_less(np.abs(gv[:m + 1] - r["logits_verify"][:m + 1]).max(), TOL)
        if not np.array_equal(g_ar[:m + 2], r["ar"][:m + 2]):
            j = int(np.nonzero(g_ar[:m + 2] != r["ar"][:m + 2])[0][0])
            row = r["logits_anchor"] if j == 0 else r["logits_verify"][j - 1]
            assert U.margin(row) <= TOL
            break
        assert int(eng.accept[0]) == m
        assert int(eng.seq_len[0]) == r["len"]
        pend_o = r["pending"]
        compared += 1
    assert compared >= 3


def test_small_repeated_passes_are_bitwise_identical():
    """The split-K GEMMs combine partials written by other workgroups; any
    stale read would show up as run-to-run differences."""
    sh = workloads.SHAPES["small"]
    K, V, B = sh["K"], sh["V"], 3
    prompt = workloads.prompts(B, 20, V, seed=12)
    eng = U.engine("small", max_batch=B, max_ctx=256)
    rows = U.anchor_row(K, B) + B
    lg = torch.zeros(rows, V, device="cuda")
    eng.set_debug(lg, None, rows)
    ref = None
    for it in range(25):
        eng.prefill(prompt)
        eng.draft()
        torch.cuda.synchronize()
        d = lg.clone()
        eng.verify()
        torch.cuda.synchronize()
        v = lg[:B * K].clone()
        eng.commit()
        if ref is None:
            ref = (d, v)
            assert torch.isfinite(d).all() and torch.isfinite(v).all()
        else:
            assert torch.equal(d, ref[0]) and torch.equal(v, ref[1]), it


def test_launch_timing_classes_and_capacity():
    """orthrus_timing_enable / orthrus_timing_read: the gate/up GEMM (timed
    by its own dispatch) and the attention class (events around the launch)
    report one launch per layer and pass with positive time (the prefill
    ends with an anchor-row pass, a draft pass); launches past the capacity
    are not timed and the read says so; timing off records nothing; the
    tokens are those of an untimed context."""
    sh = workloads.SHAPES["small"]
    L = sh["L"]
    prompt = workloads.prompts(1, 40, sh["V"], seed=17)
    ref = U.engine("small", max_ctx=512)
    want, _ = ref.generate(prompt, 24)
    eng = U.engine("small", max_ctx=512)
    gu_d, gu_v = C.timing_class("draft", "gate_up"), C.timing_class("verify", "gate_up")
    at_v = C.timing_class("verify", "attention")
    C.orthrus_timing_enable(eng.ctx, (1 << gu_d) | (1 << gu_v) | (1 << at_v), 1000)
    got, _ = eng.generate(prompt, 24)
    tim, dropped = C.orthrus_timing_read(eng.ctx)
    assert np.array_equal(got, want)
    steps = tim[("verify", "gate_up")][1] // L
    assert steps >= 1 and not dropped
    for key, passes in ((("draft", "gate_up"), steps + 1), (("verify", "gate_up"), steps),
                        (("verify", "attention"), steps)):
        ms, n = tim[key]
        assert n == passes * L and ms > 0.0, (key, ms, n)
    assert set(tim) == {("draft", "gate_up"), ("verify", "gate_up"), ("verify", "attention")}
    # capacity: only the first L draft gate/up launches are timed
    C.orthrus_timing_enable(eng.ctx, 1 << gu_d, L)
    eng.draft(); eng.verify(); eng.commit()
    eng.draft(); eng.verify(); eng.commit()
    tim, dropped = C.orthrus_timing_read(eng.ctx)
    assert dropped and tim[("draft", "gate_up")][1] == L
    C.orthrus_timing_enable(eng.ctx, 0, 0)
    eng.draft(); eng.verify(); eng.commit()
    tim, dropped = C.orthrus_timing_read(eng.ctx)
    assert tim == {} and not dropped


def test_small_block_of_63_masks():
    """The largest block (K = 63: 64 tokens x 4 heads = 256 attention rows per
    sequence and KV head in the draft pass, i.e. two row groups of eight
    16-row tiles).  Planted drafts, lengths uniform on 0..63, all accepted
    exactly, output equal to the GPU's greedy decoding; and one step against
    the oracle: anchor, mask and verify logits within 2e-2, drafts and AR
    tokens under the near-tie rule, the same accept length."""
    sh = workloads.SHAPES["small"]
    K, V, B, steps = 63, sh["V"], 3, 5
    prompt = workloads.prompts(B, 30, V, seed=65)
    ar = U.engine("small", K=0, max_batch=B, max_ctx=1024)
    traj, _ = ar.generate(prompt, 1 + steps * (K + 1) + K + 2)
    a = workloads.plant_lengths(steps, B, K, "uniform32")   # uniform on 0..K
    planted = workloads.plant_drafts(traj, 1, a, K, V)
    eng = U.engine("small", K=K, max_batch=B, max_ctx=1024)
    n_new = 1 + int((a + 1).sum(0).min())
    got, recs = eng.generate(prompt, n_new, planted=planted, record=True)
    assert np.array_equal(got, traj[:, :n_new])
    for s, r in enumerate(recs):
        assert np.array_equal(r["m"], a[s])

    # one free-running step of sequence 0 against the oracle
    om = U.oracle_model("small")
    seq = om.seq(256)
    pend_o, _ = seq.prefill(prompt[0], want_logits=True)
    one = U.engine("small", K=K, max_batch=1, max_ctx=256)
    RA = U.anchor_row(K)
    lg = torch.zeros(RA + 1, V, device="cuda")
    one.set_debug(lg, None, RA + 1)
    one.prefill(prompt[:1])
    torch.cuda.synchronize()
    assert int(one.pending[0]) == pend_o
    one.draft()
    torch.cuda.synchronize()
    gd = lg.cpu().numpy().astype(np.float64)
    drafts = one.drafts[0].cpu().numpy().copy()
    one.verify()
    torch.cuda.synchronize()
    gv = lg[:K].cpu().numpy().astype(np.float64)
    g_ar = one.ar[0].cpu().numpy().copy()
    g_m = int(one.accept[0])
    r = seq.step(pend_o, K)
    assert np.abs(gd[RA] - r["logits_anchor"]).max() < TOL
    assert np.abs(gd[:K] - r["logits_draft"]).max() < TOL
    ties = 0
    for i in range(K):
        if drafts[i] != r["drafts"][i]:
            row = r["logits_draft"][i]
            assert U.margin(row) <= TOL and np.argsort(row)[-2] == drafts[i]
            ties += 1
    if ties == 0:
        m = r["m"]
        assert g_m == m
        assert np.abs(gv[:m + 1] - r["logits_verify"][:m + 1]).max() < TOL
        assert g_ar[0] == r["ar"][0] or U.margin(r["logits_anchor"]) <= TOL

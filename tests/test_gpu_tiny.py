"""GPU parity on the tiny fp32 check model (2 layers, d 256, vocab 1024,
K = 8): tokens, drafts, AR tokens, accept lengths and commit indices are
bit-exact against the CPU oracle; logits and attention outputs within 1e-4."""
import numpy as np
import pytest
import torch

from lossless_decoding_amd.layout import vt_cols

from synth import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

TOL = 1e-4


def test_tiny_128_tokens_equal_oracle_greedy():
    """The check model's pass condition: 128 generated tokens equal plain
    greedy decoding (lossless guarantee)."""
    sh = workloads.SHAPES["tiny"]
    prompt = workloads.prompts(1, 64, sh["V"])
    want = U.oracle_model("tiny").ar_generate(prompt[0], 128)
    eng = U.engine("tiny", max_ctx=512)
    got, recs = eng.generate(prompt, 128, record=True)
    assert np.array_equal(got[0], want)
    ar = U.engine("tiny", K=0, max_ctx=512)
    got0, _ = ar.generate(prompt, 128)
    assert np.array_equal(got0[0], want)
    # cache growth per step: m + 1, commit index = old length
    for r in recs:
        assert r["commit_start"][0] == r["n"][0]
        assert r["len"][0] == r["n"][0] + 1 + r["m"][0]


def test_tiny_step_parity_with_oracle():
    sh = workloads.SHAPES["tiny"]
    K, V, L = sh["K"], sh["V"], sh["L"]
    qd = sh["hq"] * sh["hd"]
    prompt = workloads.prompts(1, 64, V, seed=3)
    om = U.oracle_model("tiny")
    seq = om.seq(400)
    tap = om.set_attn_tap(K + 1)
    pend_o = seq.prefill(prompt[0])
    eng = U.engine("tiny", max_ctx=400)
    RA = U.anchor_row(K)
    rows = RA + 1
    lg = torch.zeros(rows, V, device="cuda")
    at = torch.zeros(L, rows, qd, device="cuda")
    eng.set_debug(lg, at, rows)
    eng.prefill(prompt)
    assert int(eng.pending[0]) == pend_o
    for step in range(16):
        n = int(eng.seq_len[0])
        assert n == seq.len
        eng.draft()
        torch.cuda.synchronize()
        g_draft = lg.cpu().numpy().astype(np.float64)
        g_drafts = eng.drafts[0].cpu().numpy()
        eng.verify()
        torch.cuda.synchronize()
        g_verify = lg[:K].cpu().numpy().astype(np.float64)
        g_attn = at[:, :K].cpu().numpy().astype(np.float64)
        eng.commit()
        torch.cuda.synchronize()
        r = seq.step(pend_o, K)
        np.testing.assert_allclose(g_draft[RA], r["logits_anchor"], atol=TOL, rtol=0)
        np.testing.assert_allclose(g_draft[:K], r["logits_draft"], atol=TOL, rtol=0)
        np.testing.assert_allclose(g_verify, r["logits_verify"], atol=TOL, rtol=0)
        np.testing.assert_allclose(g_attn, tap[:, :K], atol=TOL, rtol=0)
        assert np.array_equal(g_drafts, r["drafts"])
        assert np.array_equal(eng.ar[0].cpu().numpy(), r["ar"])
        assert int(eng.accept[0]) == r["m"]
        assert int(eng.commit_start[0]) == r["commit_start"] == n
        off = eng.out_off[:2].cpu().numpy()
        assert np.array_equal(eng.out_tokens[off[0]:off[1]].cpu().numpy(), r["emitted"])
        assert int(eng.seq_len[0]) == r["len"]
        pend_o = r["pending"]
        assert int(eng.pending[0]) == pend_o


def test_tiny_draft_leaves_committed_cache_untouched():
    sh = workloads.SHAPES["tiny"]
    prompt = workloads.prompts(1, 40, sh["V"], seed=4)
    eng = U.engine("tiny", max_ctx=256)
    eng.prefill(prompt)
    for _ in range(3):
        eng.step()
    torch.cuda.synchronize()
    n = int(eng.seq_len[0])
    cap = int(eng.sizes.kv_slots)
    hd, hkv, L = sh["hd"], sh["hkv"], sh["L"]
    kv = eng.kv.view(torch.float32).view(2, L, 1, hkv, cap * hd)
    # committed slots [0, n): K rows; V^T tiles of 64 keys (whole tiles
    # below n // 64, then the columns of keys j < n % 64 of the partial tile)
    vt = kv[1].view(L, 1, hkv, cap // 64, hd, 64)
    cols = torch.as_tensor(vt_cols()[:n % 64], device=kv.device)

    def committed():
        return (kv[0, ..., :n * hd].clone(), vt[..., :n // 64, :, :].clone(),
                vt[..., n // 64, :, :][..., cols].clone())

    before = committed()
    eng.draft()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(committed(), before))
    eng.verify(); eng.commit()
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(committed(), before))

"""The 2-step iterative denoising variant (atlas.scime.ai page, "Surprising
findings"; HN item page, "Results"): orthrus_draft_refine runs the
diffusion view again over the block with each mask row starting from its
current draft's embedding.  Tiny fp32 model: the refined drafts and their
logits against the oracle's diffusion view over the same input tokens
(oc_draft_rows with in_tokens), then verify/accept/commit of the refined
block against the oracle's step; the output stays greedy decoding.  bf16
model: 2- and 3-step generation equal the GPU's own greedy decoding."""
import numpy as np
import pytest
import torch

from synth import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu
TOL = 1e-4


def test_tiny_refined_block_matches_oracle():
    sh = workloads.SHAPES["tiny"]
    K, V = sh["K"], sh["V"]
    prompt = workloads.prompts(1, 48, V, seed=41)
    om = U.oracle_model("tiny")
    seq = om.seq(400)
    pend = seq.prefill(prompt[0])
    eng = U.engine("tiny", max_ctx=400)
    rows = U.anchor_row(K) + 1              # the draft pass's rows (masks, padding, anchor)
    lg = torch.zeros(rows, V, device="cuda")
    eng.set_debug(lg, None, rows)
    eng.prefill(prompt)
    assert int(eng.pending[0]) == pend
    out = [pend]
    for step in range(10):
        n = int(eng.seq_len[0])
        eng.draft()
        torch.cuda.synchronize()
        d1 = eng.drafts[0].cpu().numpy().copy()
        eng.refine()
        torch.cuda.synchronize()
        d2 = eng.drafts[0].cpu().numpy().copy()
        g2 = lg[:K].cpu().numpy().astype(np.float64)
        # the oracle: anchor staged at slot n, then the diffusion view over
        # the block with d1 as its inputs
        seq.ar_rows(np.array([pend], np.int32), n)
        l1, o1 = seq.draft_rows(n, K)
        assert np.array_equal(o1, d1), step
        l2, o2 = seq.draft_rows(n, K, in_tokens=d1)
        np.testing.assert_allclose(g2, l2, atol=TOL, rtol=0)
        assert np.array_equal(o2, d2), step
        eng.verify()
        eng.commit()
        torch.cuda.synchronize()
        r = seq.step(pend, K, planted=d2)
        assert np.array_equal(eng.ar[0].cpu().numpy(), r["ar"])
        assert int(eng.accept[0]) == r["m"] and int(eng.seq_len[0]) == r["len"] == n + 1 + r["m"]
        off = eng.out_off[:2].cpu().numpy()
        em = eng.out_tokens[off[0]:off[1]].cpu().numpy()
        assert np.array_equal(em, r["emitted"])
        out.extend(em.tolist())
        pend = r["pending"]
    assert np.array_equal(np.array(out), om.ar_generate(prompt[0], len(out)))


@pytest.mark.parametrize("steps", [2, 3])
def test_small_iterative_denoising_equals_gpu_greedy(steps):
    sh = workloads.SHAPES["small"]
    prompt = workloads.prompts(2, 30, sh["V"], seed=42)
    eng = U.engine("small", max_batch=2, max_ctx=1024)
    got, _ = eng.generate(prompt, 60, denoise_steps=steps)
    ar = U.engine("small", K=0, max_batch=2, max_ctx=1024)
    want, _ = ar.generate(prompt, 60)
    assert np.array_equal(got, want)


def test_refine_call_order():
    from lossless_decoding_amd import _lib as C
    eng = U.engine("tiny", max_ctx=128)
    eng.prefill(workloads.prompts(1, 8, workloads.SHAPES["tiny"]["V"], seed=43))
    with pytest.raises(C.OrthrusError) as e:
        eng.refine()                       # no outstanding draft
    assert e.value.code == C.ORTHRUS_ESTATE
    eng.draft(); eng.refine(); eng.refine(); eng.verify()
    with pytest.raises(C.OrthrusError) as e:
        eng.refine()                       # already verified
    assert e.value.code == C.ORTHRUS_ESTATE
    eng.commit()

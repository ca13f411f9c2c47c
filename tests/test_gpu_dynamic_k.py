"""Dynamic K (openai-hub.net article, "Future Directions", item 1: the block
size adjusted per step): orthrus_draft_block_k with a different k <= block_k
every step.  Tiny fp32 model: every step bit-exact against the oracle's step
with the same k (drafts, AR tokens, accept length, commit), and the output
equals greedy decoding.  bf16 model: a fixed schedule and the certainty
policy both equal the GPU's own greedy decoding."""
import numpy as np
import pytest
import torch

from lossless_decoding_amd.engine import CertaintyK
from synth import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCHED = [8, 3, 0, 5, 1, 8, 2, 7, 0, 4, 6]


def test_tiny_dynamic_k_steps_match_oracle():
    sh = workloads.SHAPES["tiny"]
    K, V = sh["K"], sh["V"]
    prompt = workloads.prompts(1, 40, V, seed=31)
    om = U.oracle_model("tiny")
    seq = om.seq(400)
    pend_o = seq.prefill(prompt[0])
    eng = U.engine("tiny", max_ctx=400)
    eng.prefill(prompt)
    assert int(eng.pending[0]) == pend_o
    out = [pend_o]
    for step, k in enumerate(SCHED * 2):
        n = int(eng.seq_len[0])
        eng.drafts.fill_(-7)
        eng.draft(k)
        eng.verify()
        eng.commit()
        torch.cuda.synchronize()
        r = seq.step(pend_o, k)
        assert np.array_equal(eng.drafts[0, :k].cpu().numpy(), r["drafts"]), step
        assert (eng.drafts[0, k:].cpu().numpy() == -7).all()          # columns past k untouched
        assert np.array_equal(eng.ar[0, :k + 1].cpu().numpy(), r["ar"]), step
        m = int(eng.accept[0])
        assert m == r["m"] and 0 <= m <= k
        assert int(eng.commit_start[0]) == n and int(eng.seq_len[0]) == r["len"] == n + 1 + m
        off = eng.out_off[:2].cpu().numpy()
        emitted = eng.out_tokens[off[0]:off[1]].cpu().numpy()
        assert np.array_equal(emitted, r["emitted"])
        out.extend(emitted.tolist())
        pend_o = r["pending"]
        assert int(eng.pending[0]) == pend_o
    assert np.array_equal(np.array(out), om.ar_generate(prompt[0], len(out)))


@pytest.mark.parametrize("policy", ["schedule", "certainty"])
def test_small_dynamic_k_equals_gpu_greedy(policy):
    sh = workloads.SHAPES["small"]
    K = sh["K"]
    prompt = workloads.prompts(2, 30, sh["V"], seed=32)
    eng = U.engine("small", max_batch=2, max_ctx=1024)
    pol = (lambda s, m: [K, 3, 0, 17, 1, 32, 9][s % 7]) if policy == "schedule" else CertaintyK(K)
    got, recs = eng.generate(prompt, 60, record=True, k_policy=pol)
    ar = U.engine("small", K=0, max_batch=2, max_ctx=1024)
    want, _ = ar.generate(prompt, 60)
    assert np.array_equal(got, want)
    for r in recs:
        assert (r["m"] <= r["k"]).all()
        assert (r["len"] == r["n"] + 1 + r["m"]).all()


@pytest.mark.slow
def test_qwen3_8b_width_dynamic_k_and_refine_with_planted_drafts():
    """Dynamic K and the 2-step denoising pass at the Qwen3-8B width (one
    layer, d 4096, vocabulary 151936) and the batch shapes of the 8 x 32768
    workload (8 sequences: a 264-row draft pass at k = 32 takes the row-split
    GEMMs, smaller k the column-split ones).  Each step drafts a block of k
    from a schedule (0 and 32 included), every other step runs the refine
    pass, then planted drafts with accept lengths min(a, k) (a uniform on
    0..32) replace the block: every step accepts exactly its planted length,
    and the emitted tokens are the GPU's own greedy decoding."""
    from lossless_decoding_amd import _lib as C
    from lossless_decoding_amd.engine import Engine
    from synth.device import fill_weights_device

    sh = workloads.SHAPES["qwen3_8b"]
    K, V, B = sh["K"], sh["V"], 8
    ks = np.array([32, 5, 17, 0, 32, 9, 1, 32], np.int32)
    steps = len(ks)
    cfg = U.cfg_of("qwen3_8b", max_batch=B, max_ctx=512, n_layers=1)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    prompt = workloads.prompts(B, 20, V, seed=61)
    a = np.minimum(workloads.plant_lengths(steps, B, K, "uniform32"), ks[:, None])
    need = 1 + int((a + 1).sum(0).max()) + K + 2
    twin = Engine(U.cfg_of("qwen3_8b", K=0, max_batch=B, max_ctx=512, n_layers=1), w)
    traj, _ = twin.generate(prompt, need)
    twin.close()
    planted = workloads.plant_drafts(traj, 1, a, K, V)

    eng = Engine(cfg, w)
    eng.prefill(prompt)
    outs = [[int(t)] for t in eng.pending[:B].cpu().tolist()]
    for s in range(steps):
        k = int(ks[s])
        n = eng.seq_len[:B].cpu().numpy().copy()
        eng.draft(k)
        if s % 2 == 1 and k > 0:
            eng.refine()
        if k > 0:
            eng.drafts[:B, :k].copy_(torch.as_tensor(planted[s][:, :k], device="cuda"))
        eng.verify()
        eng.commit()
        torch.cuda.synchronize()
        acc = eng.accept[:B].cpu().numpy()
        assert np.array_equal(acc, a[s]), (s, k, acc, a[s])
        assert np.array_equal(eng.seq_len[:B].cpu().numpy(), n + 1 + acc)
        off = eng.out_off[:B + 1].cpu().numpy()
        tok = eng.out_tokens[:off[-1]].cpu().numpy()
        for b in range(B):
            outs[b].extend(tok[off[b]:off[b + 1]].tolist())
    eng.close()
    del w
    for b in range(B):
        assert outs[b] == traj[b, :len(outs[b])].tolist(), b

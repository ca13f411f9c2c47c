"""GPU path properties: rejected slots and block scratch are never read
(NaN poison), ragged prompts, per-sequence batch invariance, many sequences
with ragged commits, call-order and capacity errors."""
import numpy as np
import pytest
import torch

from lossless_decoding_amd import _lib as C
from synth import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def vt_cols():
    j = np.arange(64)
    return (j // 32) * 32 + ((j % 16) // 4) * 8 + ((j % 32) // 16) * 4 + j % 4


def poison(eng, bf16):
    """NaN into every cache slot at or past each sequence's committed length
    and into the whole block scratch."""
    cfg = eng.cfg
    L, hkv, hd, maxB = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim, cfg.max_batch
    cap = int(eng.sizes.kv_slots)
    dt = torch.bfloat16 if bf16 else torch.float32
    nan = float("nan")
    kv = eng.kv.view(dt)[:2 * L * maxB * hkv * cap * hd].view(2, L, maxB, hkv, cap, hd)
    lens = eng.seq_len[:eng.B].cpu().tolist()
    cols = torch.as_tensor(vt_cols(), device="cuda")
    for b, n in enumerate(lens):
        kv[0, :, b, :, n:, :] = nan
        vt = kv[1, :, b].view(L, hkv, cap // 64, hd, 64)
        t0 = n // 64
        vt[:, :, t0 + 1:] = nan
        if n % 64:
            vt[:, :, t0, :, cols[n % 64:]] = nan
        else:
            vt[:, :, t0] = nan
    eng.scratch.view(dt).fill_(nan)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_rejected_slots_and_scratch_are_never_read(name):
    sh = workloads.SHAPES[name]
    B = 2
    prompt = workloads.prompts(B, 30, sh["V"], seed=13)
    ref = U.engine(name, max_batch=B, max_ctx=512)
    want, _ = ref.generate(prompt, 40)
    eng = U.engine(name, max_batch=B, max_ctx=512)
    eng.prefill(prompt)
    poison(eng, sh["bf16"])
    outs = [[int(t)] for t in eng.pending[:B].cpu().tolist()]
    while min(len(o) for o in outs) < 40:
        eng.draft(); eng.verify(); eng.commit()
        off = eng.out_off[:B + 1].cpu().numpy()
        tok = eng.out_tokens[:off[-1]].cpu().numpy()
        for b in range(B):
            outs[b].extend(tok[off[b]:off[b + 1]].tolist())
        C.orthrus_sync_lengths(eng.ctx, B, eng.seq_len[:B].cpu().numpy())
        poison(eng, sh["bf16"])
    got = np.array([o[:40] for o in outs])
    assert np.array_equal(got, want)


def test_ragged_prompts_and_batch_invariance():
    """Sequences of different prompt lengths in one batch produce exactly the
    tokens each produces alone (every row's arithmetic is independent of the
    batch), and Orthrus equals greedy."""
    sh = workloads.SHAPES["small"]
    plens = [17, 40, 29]
    full = workloads.prompts(3, 40, sh["V"], seed=14)
    eng = U.engine("small", max_batch=3, max_ctx=512)
    eng.prefill(full, prompt_len=plens)
    B = 3
    outs = [[int(t)] for t in eng.pending[:B].cpu().tolist()]
    while min(len(o) for o in outs) < 50:
        eng.draft(); eng.verify(); eng.commit()
        off = eng.out_off[:B + 1].cpu().numpy()
        tok = eng.out_tokens[:off[-1]].cpu().numpy()
        for b in range(B):
            outs[b].extend(tok[off[b]:off[b + 1]].tolist())
        C.orthrus_sync_lengths(eng.ctx, B, eng.seq_len[:B].cpu().numpy())
    for b in range(B):
        alone = U.engine("small", K=0, max_batch=1, max_ctx=512)
        want, _ = alone.generate(full[b:b + 1, :plens[b]], 50)
        assert np.array_equal(np.array(outs[b][:50]), want[0]), b


def test_sixteen_sequences_ragged_commits():
    """16 sequences, per-sequence uniform{0..32} planted accept lengths:
    per-sequence lengths, commit indices and outputs stay exact."""
    sh = workloads.SHAPES["small"]
    K, B = sh["K"], 16
    prompt = workloads.prompts(B, 24, sh["V"], seed=15)
    ar = U.engine("small", K=0, max_batch=B, max_ctx=1024)
    traj, _ = ar.generate(prompt, 320)
    steps = 6
    a = workloads.plant_lengths(steps, B, K, "uniform32")
    planted = workloads.plant_drafts(traj, 1, a, K, sh["V"])
    eng = U.engine("small", max_batch=B, max_ctx=1024)
    n_new = 1 + int((a + 1).sum(0).min())
    got, recs = eng.generate(prompt, n_new, planted=planted, record=True)
    assert np.array_equal(got, traj[:, :n_new])
    for s, r in enumerate(recs):
        assert np.array_equal(r["m"], a[s])
        assert np.array_equal(r["commit_start"], r["n"])
        assert np.array_equal(r["len"], r["n"] + 1 + a[s])


def test_call_order_and_capacity_errors():
    sh = workloads.SHAPES["tiny"]
    eng = U.engine("tiny", max_batch=2, max_ctx=80)
    prompt = workloads.prompts(2, 30, sh["V"], seed=16)
    with pytest.raises(C.OrthrusError) as e:           # never prefilled
        eng.draft()
    assert e.value.code in (C.ORTHRUS_ESTATE, C.ORTHRUS_EINVAL)
    eng.prefill(prompt)
    with pytest.raises(C.OrthrusError) as e:           # verify without a draft
        eng.verify()
    assert e.value.code == C.ORTHRUS_ESTATE
    eng.draft()
    with pytest.raises(C.OrthrusError) as e:           # two drafts in a row
        eng.draft()
    assert e.value.code == C.ORTHRUS_ESTATE
    eng.verify()
    with pytest.raises(C.OrthrusError) as e:           # commit is next, not verify
        eng.verify()
    assert e.value.code == C.ORTHRUS_ESTATE
    eng.commit()
    with pytest.raises(C.OrthrusError) as e:           # commit twice
        eng.commit()
    assert e.value.code == C.ORTHRUS_ESTATE
    # the host bound grows by K+1 per step: 30 + 5*9 + 9 > 80 on the 6th step
    for _ in range(4):
        eng.step()
    with pytest.raises(C.OrthrusError) as e:
        eng.draft()
    assert e.value.code == C.ORTHRUS_ECAPACITY
    # reading the lengths back tightens the bound and decoding continues
    C.orthrus_sync_lengths(eng.ctx, 2, eng.seq_len[:2].cpu().numpy())
    eng.step()
    with pytest.raises(C.OrthrusError) as e:           # a bound above the host's is refused
        C.orthrus_sync_lengths(eng.ctx, 2, np.array([79, 79], np.int32))
    assert e.value.code == C.ORTHRUS_EINVAL


def test_prompt_length_edges():
    """Prompts of 1 and 2 tokens and of exactly one prefill pass and one token
    more (prefill_rows, the prompt rows per sequence of one pass), ragged in
    one batch: each sequence's output equals its own greedy decoding alone,
    and the one-token prompt's first token comes from prefill logits within
    2e-2 of the oracle's."""
    sh = workloads.SHAPES["small"]
    V, B = sh["V"], 4
    eng = U.engine("small", max_batch=B, max_ctx=1024)
    pr = int(eng.sizes.prefill_rows)
    plens = [1, 2, pr, pr + 1]
    full = workloads.prompts(B, pr + 1, V, seed=17)
    lg = torch.zeros(B, V, device="cuda")
    eng.set_debug(lg, None, B)
    eng.prefill(full, prompt_len=plens)
    torch.cuda.synchronize()
    first = lg[0].cpu().numpy().astype(np.float64)      # the last prefill pass: one row per sequence
    outs = [[int(t)] for t in eng.pending[:B].cpu().tolist()]
    eng.set_debug(None, None, 0)
    while min(len(o) for o in outs) < 40:
        eng.draft(); eng.verify(); eng.commit()
        off = eng.out_off[:B + 1].cpu().numpy()
        tok = eng.out_tokens[:off[-1]].cpu().numpy()
        for b in range(B):
            outs[b].extend(tok[off[b]:off[b + 1]].tolist())
        C.orthrus_sync_lengths(eng.ctx, B, eng.seq_len[:B].cpu().numpy())
    for b in range(B):
        alone = U.engine("small", K=0, max_batch=1, max_ctx=1024)
        want, _ = alone.generate(full[b:b + 1, :plens[b]], 40)
        assert np.array_equal(np.array(outs[b][:40]), want[0]), (b, plens[b])
    om = U.oracle_model("small")
    pend, lo = om.seq(64).prefill(full[0, :1], want_logits=True)
    lo = np.asarray(lo, np.float64).reshape(-1)[-V:]
    assert np.abs(first - lo).max() < 2e-2
    assert outs[0][0] == pend or U.margin(lo) <= 2e-2

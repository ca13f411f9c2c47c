"""A draft -> verify -> commit step captured as a HIP graph (engine
capture_step / replay, orthrus_reserve_steps): every replay gives exactly
the tokens, lengths and pending tokens of the same step run eagerly, with
eager work and synchronisations between the replays; and the capacity
reservation refuses steps past max_ctx."""
import numpy as np
import pytest
import torch

from lossless_decoding_amd import _lib as C
from synth import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def state(eng, B):
    off = eng.out_off[:B + 1].cpu().numpy().copy()
    return (eng.out_tokens[:off[-1]].cpu().numpy().copy(), off, eng.seq_len[:B].cpu().numpy().copy(),
            eng.pending[:B].cpu().numpy().copy())


@pytest.mark.parametrize("planted", [False, True])
def test_graph_replays_equal_eager_steps(planted):
    sh = workloads.SHAPES["small"]
    B, K, steps = 2, sh["K"], 6
    prompt = workloads.prompts(B, 24, sh["V"], seed=61)
    rng = np.random.default_rng(62)
    plants = [torch.from_numpy(rng.integers(0, sh["V"], (B, K)).astype(np.int32)).cuda()
              for _ in range(steps)]
    if planted:                      # make some drafts right: copy the greedy continuation
        ref = U.engine("small", max_batch=B, max_ctx=512)
        want, _ = ref.generate(prompt, 8)
        for s in range(steps):
            plants[s][:, :4] = torch.from_numpy(np.asarray(want)[:, 1:5].astype(np.int32)).cuda()
    eager = U.engine("small", max_batch=B, max_ctx=512)
    eager.prefill(prompt)
    want_states = []
    for s in range(steps):
        eager.step(plants[s] if planted else None)
        torch.cuda.synchronize()
        want_states.append(state(eager, B))

    eng = U.engine("small", max_batch=B, max_ctx=512)
    eng.prefill(prompt)
    torch.cuda.synchronize()
    buf = torch.zeros(B, K, dtype=torch.int32, device="cuda")
    g = eng.capture_step(buf if planted else None)
    torch.cuda.synchronize()
    for s in range(steps):
        buf.copy_(plants[s])
        eng.replay(g)
        torch.cuda.synchronize()
        got = state(eng, B)
        for a, b in zip(got, want_states[s]):
            assert np.array_equal(a, b), s
        _ = (torch.arange(1000, device="cuda") * 3).sum().item()   # eager work between replays


def test_reserve_steps_refuses_past_capacity():
    sh = workloads.SHAPES["tiny"]
    eng = U.engine("tiny", max_batch=2, max_ctx=80)
    eng.prefill(workloads.prompts(2, 30, sh["V"], seed=63))
    K = sh["K"]
    with pytest.raises(C.OrthrusError) as e:       # 30 + 6 * (K + 1) > 80
        C.orthrus_reserve_steps(eng.ctx, 2, K, 6)
    assert e.value.code == C.ORTHRUS_ECAPACITY
    C.orthrus_reserve_steps(eng.ctx, 2, K, 2)      # 30 + 2 * 9 <= 80
    eng.draft()
    with pytest.raises(C.OrthrusError) as e:       # a step in flight
        C.orthrus_reserve_steps(eng.ctx, 2, K, 1)
    assert e.value.code == C.ORTHRUS_ESTATE


@pytest.mark.slow
def test_graph_replays_equal_eager_steps_at_the_headline_batch_shapes():
    """The same at the Qwen3-8B width (one layer) and the 8-sequence shapes of
    the 8 x 32768 workload, whose passes take the row-split GEMM launches,
    the row-split LM head with its separate argmax kernel, and the
    two-tiles-per-wave attention: replays with planted drafts (the first
    step's start with three tokens of the greedy continuation, the rest are
    random) give the eager steps' tokens, lengths and pending tokens
    exactly."""
    from lossless_decoding_amd.engine import Engine
    from synth.device import fill_weights_device

    sh = workloads.SHAPES["qwen3_8b"]
    B, K, V, steps = 8, sh["K"], sh["V"], 4
    cfg = U.cfg_of("qwen3_8b", max_batch=B, max_ctx=512, n_layers=1)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    prompt = workloads.prompts(B, 24, V, seed=63)
    ref = Engine(cfg, w)
    want, _ = ref.generate(prompt, 12)
    ref.close()
    rng = np.random.default_rng(64)
    plants = []
    for s in range(steps):
        p = rng.integers(0, V, (B, K)).astype(np.int32)
        if s == 0:
            p[:, :3] = np.asarray(want)[:, 1:4]
        plants.append(torch.from_numpy(p).cuda())
    eager = Engine(cfg, w)
    eager.prefill(prompt)
    want_states = []
    for s in range(steps):
        eager.step(plants[s])
        torch.cuda.synchronize()
        want_states.append(state(eager, B))
    eager.close()

    eng = Engine(cfg, w)
    eng.prefill(prompt)
    torch.cuda.synchronize()
    buf = torch.zeros(B, K, dtype=torch.int32, device="cuda")
    g = eng.capture_step(buf)
    torch.cuda.synchronize()
    for s in range(steps):
        buf.copy_(plants[s])
        eng.replay(g)
        torch.cuda.synchronize()
        got = state(eng, B)
        for a, b in zip(got, want_states[s]):
            assert np.array_equal(a, b), s
        _ = (torch.arange(1000, device="cuda") * 3).sum().item()   # eager work between replays
    assert (want_states[0][2] == 24 + 1 + 3).all()          # the first step accepted its three drafts
    eng.close()
    del w

"""The two large decode workloads at their full sizes: Qwen3-8B shape (36
layers, bf16), K = 32, 16 sequences after 8192-token prompts and 8 after
32768-token prompts, in the configuration bench.py times (same chunk rule,
planted drafts with the workload's accept-length law).

The oracle cannot prefill prompts this long (one layer over 1024 tokens
takes minutes on the host), so these tests check properties that hold at
any size:
  * lossless: draft/verify decoding emits exactly the tokens of the GPU's own
    greedy decoding (the K = 0 twin), and every planted block is accepted to
    its planted length;
  * batch invariance: a sequence decoded inside the full batch gets the same
    tokens and bit-identical verify logits as the same sequence decoded
    alone.
Attention at these shapes is checked against the oracle on sampled rows in
test_gpu_attention; the layer arithmetic is checked against the oracle at
the full model shape in test_gpu_qwen3_8b."""
import numpy as np
import pytest
import torch

from lossless_decoding_amd import _lib as C
from lossless_decoding_amd.engine import Engine, attn_chunk_for
from synth import workloads
from synth.device import fill_weights_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

STEPS = 3


@pytest.fixture(scope="module")
def weights8b_full():
    sh = workloads.SHAPES["qwen3_8b"]
    cfg = C.OrthrusConfig.make(sh["L"], sh["d"], sh["hq"], sh["hkv"], sh["hd"], sh["F"], sh["V"],
                               sh["K"], True, 1, 128, attn_chunk=64)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    yield w
    del w
    torch.cuda.empty_cache()


def make(sh, K, B, max_ctx, chunk, w):
    cfg = C.OrthrusConfig.make(sh["L"], sh["d"], sh["hq"], sh["hkv"], sh["hd"], sh["F"], sh["V"],
                               K, True, B, max_ctx, attn_chunk=chunk)
    return Engine(cfg, w)


def decode(eng, prompts, planted):
    """Prefill, then one planted draft/verify/commit step per planted[s];
    returns the emitted tokens of each sequence."""
    eng.prefill(prompts)
    B = eng.B
    outs = [[int(t)] for t in eng.pending[:B].cpu().tolist()]
    for s in range(planted.shape[0]):
        eng.step(torch.as_tensor(planted[s], dtype=torch.int32, device="cuda"))
        off = eng.out_off[:B + 1].cpu().numpy()
        tok = eng.out_tokens[:off[-1]].cpu().numpy()
        for b in range(B):
            outs[b].extend(tok[off[b]:off[b + 1]].tolist())
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("name", ["qwen3_8b_b16_c8192", "qwen3_8b_b8_c32768"])
def test_full_size_lossless_and_batch_invariant(name, weights8b_full):
    wl = workloads.WORKLOADS[name]
    sh = workloads.SHAPES[wl["shape"]]
    B, P, K, V = wl["B"], wl["P"], sh["K"], sh["V"]
    print(f"[{name}] B={B} P={P} K={K} steps={STEPS}", flush=True)
    a = workloads.plant_lengths(STEPS, B, K, wl["plant"])
    need = 1 + int((a + 1).sum(0).max()) + K + 2
    max_ctx = P + STEPS * (K + 1) + 64
    chunk = attn_chunk_for(max_ctx, B, sh["hkv"])
    prompts = workloads.prompts(B, P, V)

    # greedy trajectory from the K = 0 twin (same chunk size: same attention rows)
    ar = make(sh, 0, B, P + need + 8, chunk, weights8b_full)
    ar.prefill(prompts)
    traj = [ar.pending[:B].clone()]
    for _ in range(1, need):
        ar.step()
        traj.append(ar.pending[:B].clone())
    traj = torch.stack(traj, 1).cpu().numpy()
    ar.close()
    del ar
    planted = workloads.plant_drafts(traj, 1, a, K, V)

    eng = make(sh, K, B, max_ctx, chunk, weights8b_full)
    # the tap is written by passes that fit in it whole: the last pass is
    # verify, B*K rows, sequence-major (sequence 0's rows first)
    lg = torch.zeros(B * K, V, device="cuda")
    eng.set_debug(lg, None, B * K)
    got = decode(eng, prompts, planted)
    lens = eng.seq_len[:B].cpu().numpy()
    eng.close()
    del eng
    for b in range(B):
        n = 1 + int((a[:, b] + 1).sum())
        assert len(got[b]) == n, (b, len(got[b]), n)
        assert got[b] == traj[b, :n].tolist(), b
        assert lens[b] == P + n - 1, b

    # sequence 0 alone, same drafts: same tokens, bit-identical verify logits
    solo = make(sh, K, 1, max_ctx, chunk, weights8b_full)
    lg1 = torch.zeros(K, V, device="cuda")
    solo.set_debug(lg1, None, K)
    got1 = decode(solo, prompts[:1], planted[:, :1])
    solo.close()
    assert got1[0] == got[0]
    assert torch.equal(lg1, lg[:K])

"""The two large decode workloads at their full sizes: Qwen3-8B shape (36
layers, bf16), K = 32, 16 sequences after 8192-token prompts and 8 after
32768-token prompts, in the configuration bench.py times (same chunk rule,
planted drafts with the workload's accept-length law).

The oracle cannot prefill prompts this long (one layer over 1024 tokens
takes minutes on the host), so two kinds of checks run here:
  * properties that hold at any size.  Lossless: draft/verify decoding emits
    exactly the tokens of the GPU's own greedy decoding (the K = 0 twin), and
    every planted block is accepted to its planted length.  Batch
    invariance: a sequence decoded inside the full batch gets the same tokens
    and bit-identical verify logits as the same sequence decoded alone;
  * oracle parity on samples the oracle can compute: three steps on the
    planting table, teacher-forced at three layers (the GPU's own layer inputs
    and committed cache loaded into the oracle) for the first and the last
    sequence of the batch.
Attention at these shapes is also checked against the oracle on sampled rows
in test_gpu_attention; every layer is checked against the oracle at the full
model shape (batch 1, short prompt) in test_gpu_qwen3_8b."""
import numpy as np
import pytest
import torch

import oracle

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


CHECK_LAYERS = (0, 18, 35)


@pytest.mark.parametrize("name", ["qwen3_8b_b16_c8192", "qwen3_8b_b8_c32768"])
def test_full_size_teacher_forced_against_oracle(name, weights8b_full):
    """Oracle parity at the full sizes, in the launch configuration bench.py
    times, on the workload's planting table: prefill of the whole batch, then
    three draft/verify/commit steps whose verify passes take the planted
    drafts.  At every step, for the first and the last sequence, at layers 0,
    18 and 35 of both passes, the oracle (float64, the GPU's committed cache
    of that layer loaded into it) recomputes the attention of the anchor,
    mask and verify rows from the GPU's layer-input rows and compares it with
    the GPU's before rounding, and recomputes the rest of the layer from the
    GPU's layer input and bf16 attention output; the final logits come from
    the GPU's last residual rows.  All within 2e-2; every draft and AR token
    is the oracle's argmax or, at an oracle near-tie, its runner-up (counted;
    the oracle follows the GPU's state); accept lengths are the planted ones
    and the oracle's prefix rule, and each commit moves a sequence by exactly
    m + 1 from its length."""
    from lossless_decoding_amd.layout import untile_v
    from tests import gpu_util as U
    from tests.test_gpu_qwen3_8b import TOL, check_token

    wl = workloads.WORKLOADS[name]
    sh = workloads.SHAPES[wl["shape"]]
    B, P, K, V = wl["B"], wl["P"], sh["K"], sh["V"]
    L, d, hkv, hd = sh["L"], sh["d"], sh["hkv"], sh["hd"]
    qd = sh["hq"] * hd
    a = workloads.plant_lengths(STEPS, B, K, wl["plant"])
    need = 1 + int((a + 1).sum(0).max()) + K + 2
    max_ctx = P + STEPS * (K + 1) + 64
    chunk = attn_chunk_for(max_ctx, B, hkv)
    print(f"[{name}] teacher-forced: B={B} P={P} K={K} chunk={chunk} layers={CHECK_LAYERS} "
          f"steps={STEPS}", flush=True)
    prompts = workloads.prompts(B, P, V)
    ar0 = make(sh, 0, B, P + need + 8, chunk, weights8b_full)
    ar0.prefill(prompts)
    traj = [ar0.pending[:B].clone()]
    for _ in range(1, need):
        ar0.step()
        traj.append(ar0.pending[:B].clone())
    traj = torch.stack(traj, 1).cpu().numpy()
    ar0.close()
    del ar0
    planted = workloads.plant_drafts(traj, 1, a, K, V)

    eng = make(sh, K, B, max_ctx, chunk, weights8b_full)
    RA = U.anchor_row(K, B)
    rows = RA + B
    lg = torch.zeros(rows, V, device="cuda")
    atb = torch.zeros(L, rows, qd, dtype=torch.bfloat16, device="cuda")
    resid = torch.zeros(L + 1, rows, d, device="cuda")
    at32 = torch.zeros(L, rows, qd, device="cuda")
    eng.set_debug(lg, atb, rows)
    eng.set_debug_layers(resid, at32, rows)
    eng.prefill(prompts)
    torch.cuda.synchronize()
    assert (eng.seq_len[:B].cpu().numpy() == P).all()

    lay = list(CHECK_LAYERS)
    lay1 = [l + 1 for l in CHECK_LAYERS]

    def grab(nrows):
        """The checked layers' taps of one pass, on the host (float64)."""
        f = lambda t: t.float().cpu().numpy().astype(np.float64)   # noqa: E731
        return dict(R=f(resid[lay, :nrows]), R1=f(resid[lay1, :nrows]), RL=f(resid[L, :nrows]),
                    A32=f(at32[lay, :nrows]), AB=f(atb[lay, :nrows]), lg=f(lg[:nrows]))

    cap = int(eng.sizes.kv_slots)
    kv = eng.kv.view(torch.bfloat16)[:2 * L * eng.cfg.max_batch * hkv * cap * hd]
    kv = kv.view(2, L, eng.cfg.max_batch, hkv, cap, hd)
    m = U.oracle_model(wl["shape"])
    worst = dict(attn=0.0, h=0.0, logits=0.0)
    events = 0

    def check_sequence(b, n, gd, gv, drafts, ar, acc):
        """Sequence b's rows of one step against the oracle (cache [0, n))."""
        nonlocal events
        seq = m.seq(n + K + 2)
        for l in CHECK_LAYERS:
            k = kv[0, l, b, :, :n].float().cpu().numpy().astype(np.float64)
            v = untile_v(kv[1, l, b].reshape(hkv, cap // 64, hd, 64))[:, :n]
            seq.load_kv(l, k, v.float().cpu().numpy().astype(np.float64))
        seq.len = n
        mk, an = slice(b * K, (b + 1) * K), slice(RA + b, RA + b + 1)

        def hold(i, g, o_o, sl, diffusion):
            ea = np.abs(o_o - g["A32"][i, sl]).max()
            h_o = m.layer_tail(CHECK_LAYERS[i], g["R"][i, sl], g["AB"][i, sl], diffusion=diffusion)
            eh = np.abs(h_o - g["R1"][i, sl]).max()
            worst["attn"] = max(worst["attn"], ea)
            worst["h"] = max(worst["h"], eh)
            assert ea < TOL and eh < TOL, (b, n, CHECK_LAYERS[i], ea, eh)

        # draft pass: the anchor at slot n (its K/V into the oracle's slot n
        # of the layer), then the mask rows over [0, n] and the block
        for i, l in enumerate(CHECK_LAYERS):
            _, o_a = seq.ar_layer(l, gd["R"][i, an], n)
            hold(i, gd, o_a, an, False)
            _, o_m = seq.draft_layer(l, gd["R"][i, mk], n)
            hold(i, gd, o_m, mk, True)
        lo, _ = m.final(np.concatenate([gd["RL"][mk], gd["RL"][an]]))
        e = np.abs(lo - np.concatenate([gd["lg"][mk], gd["lg"][an]])).max()
        worst["logits"] = max(worst["logits"], e)
        assert e < TOL, (b, n, e)
        events += sum(check_token(drafts[b, i], lo[i]) for i in range(K))
        events += check_token(ar[b, 0], lo[K])
        # verify pass over the planted drafts: rows at n+1 .. n+K, causal over
        # the cache, the anchor's slot n included
        for i, l in enumerate(CHECK_LAYERS):
            _, o_v = seq.ar_layer(l, gv["R"][i, mk], n + 1)
            hold(i, gv, o_v, mk, False)
        lo, _ = m.final(gv["RL"][mk])
        e = np.abs(lo - gv["lg"][mk]).max()
        worst["logits"] = max(worst["logits"], e)
        assert e < TOL, (b, n, e)
        events += sum(check_token(ar[b, 1 + i], lo[i]) for i in range(K))
        del seq

    for step in range(STEPS):
        n0 = eng.seq_len[:B].cpu().numpy().copy()
        eng.draft()
        torch.cuda.synchronize()
        gd = grab(rows)
        drafts = eng.drafts[:B].cpu().numpy().copy()
        eng.drafts[:B].copy_(torch.as_tensor(planted[step], device="cuda"))
        eng.verify()
        torch.cuda.synchronize()
        gv = grab(B * K)
        ar = eng.ar[:B].cpu().numpy().copy()
        acc = eng.accept[:B].cpu().numpy().copy()
        for b in sorted({0, B - 1}):
            check_sequence(b, int(n0[b]), gd, gv, drafts, ar, acc)
            assert acc[b] == oracle.accept(planted[step][b], ar[b]) == a[step, b], (step, b)
        eng.commit()
        torch.cuda.synchronize()
        assert np.array_equal(eng.commit_start[:B].cpu().numpy(), n0)
        assert np.array_equal(eng.seq_len[:B].cpu().numpy(), n0 + 1 + acc)
        assert np.array_equal(eng.pending[:B].cpu().numpy(), ar[np.arange(B), acc])
    eng.close()
    print(f"[{name}] teacher-forced layers {CHECK_LAYERS} x {STEPS} steps: max |attention| "
          f"{worst['attn']:.2e}, max |layer output| {worst['h']:.2e}, max |logits| "
          f"{worst['logits']:.2e}, near-tie events {events}", flush=True)

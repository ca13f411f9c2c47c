"""The allocation-free form of kernel (a) (orthrus_block_attention_noalloc:
its chunk partials in the library's static device scratch) against the
workspace form (orthrus_block_attention), bit for bit: the same kernels on
the same inputs.  Two calls in a row, the second smaller, so that the second
reuses the scratch the first left behind; and a call beyond the scratch's
limit is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from lossless_decoding_amd import _lib as C
from lossless_decoding_amd.layout import tile_block_v, tile_v
from synth import workloads
from synth.device import fill_normal_device

pytestmark = pytest.mark.gpu
HD = 128


def inputs(B, rows, hq, hkv, lk, kb, seed):
    cap = max(64, (lk + 63) // 64 * 64)
    st = workloads.attn_inputs_stream(B, lk) + seed
    q = torch.empty(B, rows, hq, HD, dtype=torch.bfloat16, device="cuda")
    fill_normal_device(q, workloads.ATTN_SEED, st, 1.0, synth.P_ATTN)
    kc = torch.zeros(B, hkv, cap, HD, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    if lk:
        t = torch.empty(B, hkv, lk, HD, dtype=torch.bfloat16, device="cuda")
        fill_normal_device(t, workloads.ATTN_SEED, st + 1, 1.0, synth.P_ATTN)
        kc[:, :, :lk] = t
        fill_normal_device(t, workloads.ATTN_SEED, st + 2, 1.0, synth.P_ATTN)
        vc[:, :, :lk] = t
    kpad = (kb + 31) // 32 * 32
    kbk = torch.zeros(B, hkv, kpad, HD, dtype=torch.bfloat16, device="cuda")
    t = torch.empty(B, hkv, kb, HD, dtype=torch.bfloat16, device="cuda")
    fill_normal_device(t, workloads.ATTN_SEED, st + 3, 1.0, synth.P_ATTN)
    kbk[:, :, :kb] = t
    fill_normal_device(t, workloads.ATTN_SEED, st + 4, 1.0, synth.P_ATTN)
    return q, kc, tile_v(vc), kbk, tile_block_v(t, kpad), cap


def both(B, rows, hq, hkv, lk, kb, seed):
    q, kc, vt, kbk, vbt, cap = inputs(B, rows, hq, hkv, lk, kb, seed)
    s = torch.cuda.current_stream().cuda_stream
    ref = torch.zeros(B, rows, hq, HD, dtype=torch.bfloat16, device="cuda")
    wsb = C.orthrus_attention_workspace(B, rows, hq, hkv, lk)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    C.orthrus_block_attention(B, rows, hq, hkv, q.data_ptr(), kc.data_ptr(), vt.data_ptr(), cap, lk,
                              kbk.data_ptr(), vbt.data_ptr(), kb, ref.data_ptr(), ws.data_ptr(),
                              wsb, s)
    got = torch.full_like(ref, float("nan"))
    C.orthrus_block_attention_noalloc(B, rows, hq, hkv, q.data_ptr(), kc.data_ptr(), vt.data_ptr(),
                                      cap, lk, kbk.data_ptr(), vbt.data_ptr(), kb, got.data_ptr(), s)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_block_attention_matches_workspace_form_twice():
    # first call: 16 sequences x 4000 keys (two-tile launch, ragged block)
    ref, got = both(16, 32, 32, 8, 4000, 17, 21)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # second call, smaller: 2 sequences x 300 keys (one-tile launch); the
    # scratch still holds the first call's partials
    ref, got = both(2, 32, 32, 8, 300, 32, 22)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_noalloc_block_attention_refuses_beyond_scratch():
    need = C.orthrus_attention_workspace(64, 36, 32, 8, 32768)
    assert need > (48 << 20)
    rc = C.lib().orthrus_block_attention_noalloc(64, 36, 32, 8, 1, 1, 1, 32768, 32768, 1, 1, 32,
                                                 1, None)
    assert rc == C.ORTHRUS_ECAPACITY

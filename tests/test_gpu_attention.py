"""Kernel (a) alone: block-draft attention through orthrus_block_attention
against the oracle's attention (float64 on the same bf16 inputs).  The
inputs are N(0, 1) from the seeded generator; rows see every cache key and
every block key (the mask-row view).  Tolerance 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from lossless_decoding_amd import _lib as C
from synth import workloads
from synth.device import fill_normal_device
from lossless_decoding_amd.layout import tile_v, tile_block_v

pytestmark = pytest.mark.gpu
TOL = 2e-2
HD = 128


def make(B, rows, hq, hkv, lk, kb, seed_base):
    cap = max(64, (lk + 63) // 64 * 64)
    q = torch.empty(B, rows, hq, HD, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, hkv, cap, HD, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(B, hkv, cap, HD, dtype=torch.bfloat16, device="cuda")
    kbk = torch.empty(B, hkv, max(kb, 1), HD, dtype=torch.bfloat16, device="cuda")
    vbk = torch.empty(B, hkv, max(kb, 1), HD, dtype=torch.bfloat16, device="cuda")
    st = workloads.attn_inputs_stream(B, lk) + seed_base
    fill_normal_device(q, workloads.ATTN_SEED, st, 1.0, synth.P_ATTN)
    if lk:
        kk = torch.empty(B, hkv, lk, HD, dtype=torch.bfloat16, device="cuda")
        fill_normal_device(kk, workloads.ATTN_SEED, st + 1, 1.0, synth.P_ATTN)
        kc[:, :, :lk] = kk
        fill_normal_device(kk, workloads.ATTN_SEED, st + 2, 1.0, synth.P_ATTN)
        vc[:, :, :lk] = kk
    fill_normal_device(kbk, workloads.ATTN_SEED, st + 3, 1.0, synth.P_ATTN)
    fill_normal_device(vbk, workloads.ATTN_SEED, st + 4, 1.0, synth.P_ATTN)
    return q, kc, vc, kbk, vbk, cap


def run(B, rows, hq, hkv, lk, kb, q, kc, vc, kbk, vbk, cap):
    kpad = (kb + 31) // 32 * 32
    vt = tile_v(vc)
    vbt = tile_block_v(vbk[:, :, :kb], kpad) if kb else None
    kbp = torch.zeros(B, hkv, kpad, HD, dtype=torch.bfloat16, device="cuda") if kb else None
    if kb:
        kbp[:, :, :kb] = kbk[:, :, :kb]
    out = torch.zeros(B, rows, hq, HD, dtype=torch.bfloat16, device="cuda")
    wsb = C.orthrus_attention_workspace(B, rows, hq, hkv, lk)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device="cuda")
    C.orthrus_block_attention(B, rows, hq, hkv, q.data_ptr(), kc.data_ptr(), vt.data_ptr(), cap,
                              lk, kbp.data_ptr() if kb else None, vbt.data_ptr() if kb else None,
                              kb, out.data_ptr(), ws.data_ptr(), wsb,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out


def oracle_row(q, kc, vc, kbk, vbk, b, r, h, lk, kb, G):
    g = h // G
    keys = np.concatenate([kc[b, g, :lk], kbk[b, g, :kb]]).astype(np.float64)
    vals = np.concatenate([vc[b, g, :lk], vbk[b, g, :kb]]).astype(np.float64)
    return oracle.attention(q[b, r, h].astype(np.float64), keys, vals)


@pytest.mark.parametrize("lk,kb", [(300, 32), (64, 32), (0, 32), (1000, 0), (577, 17)])
def test_block_attention_small_all_rows(lk, kb):
    B, rows, hq, hkv = 2, 32, 8, 2
    q, kc, vc, kbk, vbk, cap = make(B, rows, hq, hkv, lk, kb, 0)
    out = run(B, rows, hq, hkv, lk, kb, q, kc, vc, kbk, vbk, cap).float().cpu().numpy()
    qn, kn, vn = q.float().cpu().numpy(), kc.float().cpu().numpy(), vc.float().cpu().numpy()
    kbn, vbn = kbk.float().cpu().numpy(), vbk.float().cpu().numpy()
    err = 0.0
    for b in range(B):
        for r in range(rows):
            for h in range(hq):
                want = oracle_row(qn, kn, vn, kbn, vbn, b, r, h, lk, kb, hq // hkv)
                err = max(err, float(np.abs(out[b, r, h] - want).max()))
    assert err < TOL, err


@pytest.mark.slow
@pytest.mark.parametrize("B,rows,lk", [(16, 32, 32768), (16, 33, 8192), (8, 33, 32768)])
def test_block_attention_full_size_sampled(B, rows, lk):
    """Full sizes: the largest microbenchmark point (16 sequences x 32768
    cached keys, 32 query tokens) and the draft pass of the two large decode
    workloads (16 x 8192 and 8 x 32768 cached keys, 33 query tokens: anchor
    and 32 masks); 32 query heads over 8 KV heads, 32 block keys.  Sampled
    (sequence, row, head) outputs against the oracle."""
    hq, hkv, kb = 32, 8, 32
    G = hq // hkv
    print(f"[attention] B={B} rows={rows} lk={lk}", flush=True)
    q, kc, vc, kbk, vbk, cap = make(B, rows, hq, hkv, lk, kb, 0)
    out = run(B, rows, hq, hkv, lk, kb, q, kc, vc, kbk, vbk, cap)
    rng = np.random.default_rng(lk + rows)
    for _ in range(8):
        b, r, h = int(rng.integers(B)), int(rng.integers(rows)), int(rng.integers(hq))
        g = h // G
        keys = torch.cat([kc[b, g, :lk], kbk[b, g, :kb]]).float().cpu().numpy().astype(np.float64)
        vals = torch.cat([vc[b, g, :lk], vbk[b, g, :kb]]).float().cpu().numpy().astype(np.float64)
        want = oracle.attention(q[b, r, h].float().cpu().numpy().astype(np.float64), keys, vals)
        got = out[b, r, h].float().cpu().numpy()
        assert np.abs(got - want).max() < TOL, (b, r, h)


@pytest.mark.parametrize("lk,kb", [(4000, 17), (4096, 1)])
def test_block_attention_two_tile_launch_ragged(lk, kb):
    """A launch of 512 workgroups (16 sequences x 8 KV heads x 4 chunks)
    runs two query tiles per wave and streams the draft block after the
    last chunk's cache keys: a partial last cache tile (4000 keys: 32 keys
    in the last tile) and a ragged block (17 keys), or a whole last tile and
    a one-key block.  Sampled (sequence, row, head) outputs against the
    oracle."""
    B, rows, hq, hkv = 16, 32, 32, 8
    G = hq // hkv
    q, kc, vc, kbk, vbk, cap = make(B, rows, hq, hkv, lk, kb, 7)
    out = run(B, rows, hq, hkv, lk, kb, q, kc, vc, kbk, vbk, cap)
    rng = np.random.default_rng(lk + kb)
    for _ in range(16):
        b, r, h = int(rng.integers(B)), int(rng.integers(rows)), int(rng.integers(hq))
        g = h // G
        keys = torch.cat([kc[b, g, :lk], kbk[b, g, :kb]]).float().cpu().numpy().astype(np.float64)
        vals = torch.cat([vc[b, g, :lk], vbk[b, g, :kb]]).float().cpu().numpy().astype(np.float64)
        want = oracle.attention(q[b, r, h].float().cpu().numpy().astype(np.float64), keys, vals)
        got = out[b, r, h].float().cpu().numpy()
        assert np.abs(got - want).max() < TOL, (b, r, h)


def _reference_rows(q, kc, vc, kbk, vbk, b, g, lk, kb, qrows, G):
    """Oracle outputs of query rows qrows = [(token, head)] of sequence b,
    all reading KV head g: every cache key and every block key."""
    keys = torch.cat([kc[b, g, :lk], kbk[b, g, :kb]]).float().cpu().numpy().astype(np.float64)
    vals = torch.cat([vc[b, g, :lk], vbk[b, g, :kb]]).float().cpu().numpy().astype(np.float64)
    qs = np.stack([q[b, t, h] for t, h in qrows]).astype(np.float64)
    return oracle.attention_many(qs, keys, vals)


@pytest.mark.slow
@pytest.mark.parametrize("lk,B", workloads.ATTN_GRID)
def test_block_attention_microbenchmark_grid(lk, B):
    """Every point of the block-attention microbenchmark (32 query tokens x
    32 query heads over 8 KV heads, 32 block keys, Lk cached keys, bf16
    N(0, 1) inputs).  B in {1, 4}: every (sequence, token, head) output
    against the oracle.  B = 16: for every sequence, the four heads of one
    KV head (rotating over the KV heads) at tokens 0..31 step 3 plus the last
    token 31, which covers all eight 16-row query tiles (every row group of
    either launch form) of that (sequence, KV head): 16 x 12 x 4 = 768
    outputs."""
    rows, hq, hkv, kb = 32, 32, 8, 32
    G = hq // hkv
    print(f"[attention grid] B={B} lk={lk}", flush=True)
    q, kc, vc, kbk, vbk, cap = make(B, rows, hq, hkv, lk, kb, 11)
    out = run(B, rows, hq, hkv, lk, kb, q, kc, vc, kbk, vbk, cap)
    err = 0.0
    if B <= 4:
        pairs = [(b, g, [(t, g * G + j) for t in range(rows) for j in range(G)])
                 for b in range(B) for g in range(hkv)]
    else:
        toks = sorted(set(range(0, rows, 3)) | {rows - 1})
        pairs = [(b, b % hkv, [(t, (b % hkv) * G + j) for t in toks for j in range(G)])
                 for b in range(B)]
    n = 0
    qn = q.float().cpu().numpy()
    on = out.float().cpu().numpy()
    for b, g, qrows in pairs:
        want = _reference_rows(qn, kc, vc, kbk, vbk, b, g, lk, kb, qrows, G)
        got = np.stack([on[b, t, h] for t, h in qrows])
        err = max(err, float(np.abs(got - want).max()))
        n += len(qrows)
    assert n >= (B * rows * hq if B <= 4 else 256)
    assert err < TOL, err


@pytest.mark.parametrize("lk,kb", [(700, 64), (0, 64)])
def test_block_attention_64_rows_all_rows(lk, kb):
    """The largest block: 64 query tokens and 64 block keys (256 rows per KV
    head at a group of 4), every output against the oracle."""
    B, rows, hq, hkv = 2, 64, 8, 2
    q, kc, vc, kbk, vbk, cap = make(B, rows, hq, hkv, lk, kb, 5)
    out = run(B, rows, hq, hkv, lk, kb, q, kc, vc, kbk, vbk, cap).float().cpu().numpy()
    qn, kn, vn = q.float().cpu().numpy(), kc.float().cpu().numpy(), vc.float().cpu().numpy()
    kbn, vbn = kbk.float().cpu().numpy(), vbk.float().cpu().numpy()
    err = 0.0
    for b in range(B):
        for r in range(rows):
            for h in range(hq):
                want = oracle_row(qn, kn, vn, kbn, vbn, b, r, h, lk, kb, hq // hkv)
                err = max(err, float(np.abs(out[b, r, h] - want).max()))
    assert err < TOL, err

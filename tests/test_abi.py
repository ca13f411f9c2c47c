"""The C ABI on the host (no GPU): the library loads, exports every entry
point include/orthrus.h declares, agrees with the oracle on the canonical
weight format, and reports the block scratch the pages describe."""
import ctypes
import json
import os
import re

import pytest

import oracle
from lossless_decoding_amd import _lib as C
from synth import workloads
from tests import helpers as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")


def cfg_of(name, max_batch=1, max_ctx=4096, **over):
    s = dict(workloads.SHAPES[name]); s.update(over)
    return C.OrthrusConfig.make(s["L"], s["d"], s["hq"], s["hkv"], s["hd"], s["F"], s["V"],
                                s["K"], s["bf16"], max_batch, max_ctx)


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "orthrus.h")).read()
    declared = set(re.findall(r"\b(orthrus_[a-z_]+)\s*\(", hdr))
    assert declared == set(C.EXPORTED)
    L = ctypes.CDLL(C.lib_path())
    for name in declared:
        assert hasattr(L, name), name


@pytest.mark.parametrize("name", ["tiny", "small", "qwen3_8b"])
def test_weight_format_matches_oracle(name):
    lay, total = C.weight_layout(cfg_of(name))
    olay, ototal = oracle.weight_layout(H.shape(name))
    assert total == ototal
    assert lay == olay


def test_block_scratch_is_pages_overhead():
    """Block K/V scratch at the Qwen3-8B shape, K = 32, one sequence, bf16:
    32 * 36 * 2 * 8 * 128 * 2 bytes = 4.5 MiB -- the pages' flat O(1) KV
    overhead (HN item page 'Results'; openai-hub.net 'KV Cache Overhead')."""
    g = json.load(open(os.path.join(GOLD, "pages_figures.json")))
    s = C.orthrus_query_sizes(cfg_of("qwen3_8b", max_batch=1, max_ctx=1024))
    assert workloads.SHAPES["qwen3_8b"]["K"] == g["block_size_K"]["value"]
    assert s.scratch_bytes == g["kv_overhead_mib"]["value"] * 2 ** 20
    # flat in the context length
    s2 = C.orthrus_query_sizes(cfg_of("qwen3_8b", max_batch=1, max_ctx=32768))
    assert s2.scratch_bytes == s.scratch_bytes


def test_trainable_fraction_is_pages_16_percent():
    """The diffusion path (own Q/K/V/O per layer, everything else shared)
    is about 16% of all parameters at the Qwen3-8B shape (HN item page
    'Results'; atlas.scime.ai 'Key results')."""
    g = json.load(open(os.path.join(GOLD, "pages_figures.json")))
    lay, _ = C.weight_layout(cfg_of("qwen3_8b"))
    total = sum(n for _, _, n, _ in lay)
    diff = sum(n for t, _, n, _ in lay if t >= 4 and (t - 4) % 17 in (8, 9, 10, 11, 12, 13))
    assert round(100 * diff / total) == g["trainable_fraction_percent"]["value"]


def test_tpf_accounting_matches_pages():
    """Tokens per forward with two forwards per step and the bonus token:
    (accept length + 1) / 2 reproduces the printed MATH-500 pair
    11.7 -> 6.35 (HN item page 'Results'; atlas.scime.ai 'Key results')."""
    from bench import tpf_from_accept
    g = json.load(open(os.path.join(GOLD, "pages_figures.json")))
    assert abs(tpf_from_accept(g["acceptance_length_math500"]["value"])
               - g["tpf_math500"]["value"]) < 1e-12


@pytest.mark.parametrize("field,val", [("n_layers", 0), ("head_dim", 64), ("d_model", 500),
                                       ("block_k", 64), ("max_batch", 0), ("n_kv_heads", 3),
                                       ("attn_chunk", 100), ("attn_chunk", 32), ("vocab", 2000)])
def test_invalid_configs_rejected(field, val):
    c = cfg_of("small")
    setattr(c, field, val)
    with pytest.raises(C.OrthrusError) as e:
        C.orthrus_query_sizes(c)
    assert e.value.code == C.ORTHRUS_EINVAL


def test_largest_block_accepted():
    """block_k up to 63 (one 64-key block tile, one 64-lane acceptance
    ballot) at the Qwen3-8B group of 4 query heads per KV head."""
    c = cfg_of("qwen3_8b")
    c.block_k = 63
    assert C.orthrus_query_sizes(c).kv_bytes > 0


def test_create_rejects_null_and_misaligned_pointers():
    c = cfg_of("tiny")
    with pytest.raises(C.OrthrusError) as e:
        C.orthrus_create(c, None, None, None, None, None, None)
    assert e.value.code == C.ORTHRUS_EINVAL
    with pytest.raises(C.OrthrusError) as e:
        C.orthrus_create(c, 4096 + 8, 8192, 8192, 8192, 8192, None)
    assert e.value.code == C.ORTHRUS_EINVAL


def test_call_order_errors_on_null_context_args():
    with pytest.raises(C.OrthrusError) as e:
        C.orthrus_draft_block(None, 1, None, None, None, None, None)
    assert e.value.code == C.ORTHRUS_EINVAL
    with pytest.raises(C.OrthrusError) as e:
        C.orthrus_block_attention(1, 200, 32, 8, 8, 8, 8, 64, 64, 8, 8, 32, 8, 8, 1 << 20, None)
    assert e.value.code == C.ORTHRUS_EINVAL


@pytest.mark.parametrize("batch,ctx,kvh,want", [
    (1, 4668, 8, 128),      # B = 1 decode: at most 64 chunks per sequence
    (16, 8619, 8, 2048),    # 16 x 8192 decode: <= 1100 workgroups, >= 1024 keys
    (8, 33096, 8, 2048),    # 8 x 32768 decode
    (4, 16384, 8, 1024),
    (16, 4096, 8, 1024),
    (16, 32768, 8, 4096),   # capped at 4096
    (1, 1600, 8, 128),      # B = 1 decode at a short context: the floor
    (1, 64, 2, 128),
])
def test_default_attention_chunk_rule(batch, ctx, kvh, want):
    """The chunk rule the header documents: the smallest power of two in
    [128, 4096] with <= 64 chunks per sequence and <= 1100 (chunk, KV head,
    sequence) workgroups, at least 1024 when 1024-key chunks still give 512
    workgroups (slots: the context's kv_slots)."""
    got = C.orthrus_default_attn_chunk(batch, ctx, kvh)
    assert got == want
    # the context's kv_slots (include/orthrus.h, orthrus_sizes)
    slots = (ctx + 63) // 64 * 64
    nch = -(-slots // got)
    assert got & (got - 1) == 0 and 128 <= got <= 4096
    if got < 4096:
        assert nch <= 64 and batch * kvh * nch <= 1100
    if got > 128:     # the next smaller size breaks a condition
        half = got // 2
        n2 = -(-slots // half)
        long_ok = batch * kvh * (-(-slots // 1024)) >= 512
        assert n2 > 64 or batch * kvh * n2 > 1100 or (long_ok and half < 1024)


@pytest.mark.parametrize("batch,ctx,kvh,chunk", [
    (4, 16384, 8, 1024),    # the 256 MB kernel (a) points
    (16, 4096, 8, 1024),
    (16, 32768, 8, 8192),
    (8, 32768, 8, 4096),
    (1, 4096, 8, 64),
    (1, 0, 8, 64),          # block keys only: one chunk
])
def test_block_attention_chunk_rule(batch, ctx, kvh, chunk):
    """Kernel (a) alone sizes its workspace for its own chunk rule (the
    smallest power of two in [64, 16384] with <= 64 chunks and <= 512
    workgroups): partials for max(1, chunks) + 1 chunks of rows x G rows,
    each 128 fp32 plus (m, l), each array 256-byte aligned."""
    rows, hq = 32, 32
    nch = max(1, -(-ctx // chunk))
    pr = batch * kvh * (nch + 1) * rows * (hq // kvh)
    al = lambda n: (n + 255) // 256 * 256
    assert C.orthrus_attention_workspace(batch, rows, hq, kvh, ctx) == al(pr * 512) + al(pr * 8)
    if chunk > 64:    # the next smaller size breaks a condition
        n2 = -(-ctx // (chunk // 2))
        assert n2 > 64 or batch * kvh * n2 > 512


def test_default_attention_chunk_rejects_bad_args():
    with pytest.raises(C.OrthrusError):
        C.orthrus_default_attn_chunk(0, 1024, 8)
    with pytest.raises(C.OrthrusError):
        C.orthrus_default_attn_chunk(1, 1024, 0)


@pytest.mark.parametrize("batch,want", [(1, 256), (4, 256), (8, 256), (12, 160), (16, 128), (64, 32),
                                        (128, 32)])
def test_sizes_report_cache_slots_and_prefill_rows(batch, want):
    """orthrus_query_sizes: kv_slots is max_ctx rounded up to 64, and
    prefill_rows (prompt rows per sequence in one prefill pass) is 2048 /
    max_batch rounded down to a multiple of 32, clamped to [32, 256]."""
    s = C.orthrus_query_sizes(cfg_of("small", max_batch=batch, max_ctx=1000))
    assert s.kv_slots == 1024
    assert s.prefill_rows == want

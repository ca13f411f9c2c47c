"""Helpers for the GPU tests: engines over synth weights, oracle twins."""
import numpy as np
import torch

import oracle
from lossless_decoding_amd import _lib as C
from lossless_decoding_amd.engine import Engine
from synth import workloads
from synth.device import fill_weights_device
from tests import helpers as H


def cfg_of(name, K=None, max_batch=1, max_ctx=512, attn_chunk=128, **over):
    """Test contexts share one attention chunk size so that a K context and
    its K = 0 greedy twin are bit-comparable."""
    s = dict(workloads.SHAPES[name]); s.update(over)
    L = s.pop("n_layers", s["L"])
    return C.OrthrusConfig.make(L, s["d"], s["hq"], s["hkv"], s["hd"], s["F"], s["V"],
                                s["K"] if K is None else K, s["bf16"], max_batch, max_ctx,
                                attn_chunk=attn_chunk)


_WCACHE = {}


def device_weights(cfg, seed=workloads.WEIGHT_SEED):
    key = (cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn_dim,
           cfg.vocab, cfg.dtype, seed)
    if key not in _WCACHE:
        lay, total = C.weight_layout(cfg)
        _WCACHE[key] = fill_weights_device(lay, total, cfg.dtype == C.ORTHRUS_BF16, seed)
    return _WCACHE[key]


def engine(name, K=None, max_batch=1, max_ctx=512, seed=workloads.WEIGHT_SEED, **over):
    cfg = cfg_of(name, K, max_batch, max_ctx, **over)
    return Engine(cfg, device_weights(cfg, seed))


_OCACHE = {}


def oracle_model(name, seed=workloads.WEIGHT_SEED, **over):
    key = (name, seed, tuple(sorted(over.items())))
    if key not in _OCACHE:
        shp = H.shape(name, **over)
        _OCACHE[key] = oracle.Model(shp, H.weights(shp, seed))
    return _OCACHE[key]


def anchor_row(K, B=1, b=0):
    """Physical row of sequence b's anchor in a draft pass: the B*K mask rows
    come first, padded to a multiple of 16."""
    return (B * K + 15) // 16 * 16 + b


def margin(logits_row):
    """top-1 minus top-2 of one logits row."""
    s = np.sort(np.asarray(logits_row, np.float64))
    return s[-1] - s[-2]


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)

"""Workload descriptions and seeded input builders (shapes, prompts, planted
drafts, random-init weights).  No arithmetic of the decoding method lives
here: the planting only needs the greedy trajectory as data.

Model shapes
  tiny      -- 2 layers, d 256, 4 q / 2 kv heads of 64, SwiGLU 688, vocab
               1024, fp32, K = 8 (the CPU-seconds check model).
  small     -- 2 layers, d 512, 8 q / 2 kv heads of 128, SwiGLU 1024, vocab
               2048, bf16, K = 32: the bf16 kernels' parity model (same head
               size and GQA group of 4 as the big model, oracle in seconds).
  qwen3_8b  -- 36 layers, d 4096, 32 q / 8 kv heads of 128, SwiGLU 12288,
               vocab 151936, bf16, K = 32.
All matrices (and the mask embedding) are N(0, 0.02) from synth's
Irwin-Hall normal under weights seed 0, one Philox stream per canonical
tensor index; RMSNorm gains are 1.
"""
from __future__ import annotations

import numpy as np

from . import (P_PLANT, P_TOKENS, f32_to_bf16_bits, host_fill_normal, normal_f32, tokens,
               uniform_u32)

SHAPES = {
    "tiny": dict(L=2, d=256, hq=4, hkv=2, hd=64, F=688, V=1024, K=8, bf16=False),
    "small": dict(L=2, d=512, hq=8, hkv=2, hd=128, F=1024, V=2048, K=32, bf16=True),
    "qwen3_8b": dict(L=36, d=4096, hq=32, hkv=8, hd=128, F=12288, V=151936, K=32, bf16=True),
}

WEIGHT_SEED = 0
PROMPT_SEED = 1
PLANT_SEED = 2
ATTN_SEED = 3
SIGMA = 0.02

# Decode workloads: (shape, batch, prompt length, generated tokens, planting law)
WORKLOADS = {
    "tiny_b1": dict(shape="tiny", B=1, P=64, gen=128, plant=None),
    "qwen3_8b_b1_p512": dict(shape="qwen3_8b", B=1, P=512, gen=1024, plant="geom6"),
    "qwen3_8b_b16_c8192": dict(shape="qwen3_8b", B=16, P=8192, gen=256, plant="geom6"),
    "qwen3_8b_b8_c32768": dict(shape="qwen3_8b", B=8, P=32768, gen=128, plant="uniform32"),
}

# Attention microbenchmark grid (KV lengths x batch), bf16, 32 q / 8 kv heads of 128.
ATTN_GRID = [(lk, b) for b in (1, 4, 16) for lk in (1024, 4096, 16384, 32768)]


def fill_weights(layout, total: int, bf16: bool, seed: int = WEIGHT_SEED,
                 sigma: float = SIGMA) -> np.ndarray:
    """Canonical weight buffer on the host for a given layout
    [(tensor_index, offset, numel, is_gain)].  bf16 buffers are uint16."""
    w = np.zeros(total, np.uint16 if bf16 else np.float32)
    for t, off, n, gain in layout:
        view = w[off:off + n]
        if gain:
            view[:] = 0x3F80 if bf16 else 1.0
            continue
        try:
            host_fill_normal(view, seed, t, sigma)
        except RuntimeError:
            v = normal_f32(n, seed, t, sigma)
            view[:] = f32_to_bf16_bits(v) if bf16 else v
    return w


def prompts(B: int, P: int, V: int, seed: int = PROMPT_SEED) -> np.ndarray:
    """[B][P] int32 prompt ids uniform on [0, V); sequence b uses stream b."""
    return np.stack([tokens(P, V, seed, b, P_TOKENS) for b in range(B)]).astype(np.int32)


_GEOM_THRESH = (1 << 32) // 7       # P(success) = 1/7 per trial


def plant_lengths(steps: int, B: int, K: int, law: str, seed: int = PLANT_SEED) -> np.ndarray:
    """[steps][B] planted accept lengths a.
    geom6:     a = failures before the first success of Bernoulli(1/7)
               trials (mean 6), clipped to K.
    uniform32: a uniform on {0..K}."""
    a = np.zeros((steps, B), np.int32)
    for b in range(B):
        for s in range(steps):
            x = np.stack(uniform_u32(24, seed, b, P_PLANT, start=s * 24)).T.reshape(-1)
            if law == "geom6":
                k = 0
                while k < K and x[k] >= _GEOM_THRESH:
                    k += 1
                a[s, b] = k
            elif law == "uniform32":
                a[s, b] = int((int(x[0]) * (K + 1)) >> 32)
            else:
                raise ValueError(law)
    return a


def plant_drafts(traj: np.ndarray, first_emitted: int, a: np.ndarray, K: int, V: int,
                 seed: int = PLANT_SEED) -> np.ndarray:
    """Planted drafts [steps][B][K] from greedy trajectories.

    traj[b][j] is the (j+1)-th generated token of sequence b (traj[b][0] is
    the prefill's token).  With planted accept length a at step s and e
    tokens already emitted, the drafts are the next a true tokens, then a
    token guaranteed to differ from the true one, then uniform ids -- so the
    step accepts exactly a drafts.  Needs traj[b] long enough
    (first_emitted + sum(a+1) + K + 1 tokens)."""
    steps, B = a.shape
    out = np.zeros((steps, B, K), np.int32)
    # Philox blocks (4 words) per step: 24 up to K = 32 (x[64] the wrong
    # token, x[65..95] the fillers), more for larger blocks
    nblk = max(24, (64 + K + 3) // 4)
    for b in range(B):
        e = first_emitted
        for s in range(steps):
            x = np.stack(uniform_u32(nblk, seed, b, P_PLANT, start=s * nblk)).T.reshape(-1)
            k = int(a[s, b])
            t = traj[b, e:e + K + 1]          # true continuation t_1..t_{K+1}
            out[s, b, :k] = t[:k]
            if k < K:
                u = int((int(x[64]) * (V - 1)) >> 32)
                out[s, b, k] = (int(t[k]) + 1 + u) % V
                for i in range(k + 1, K):      # at most K - 1 words: x[65..]
                    out[s, b, i] = int((int(x[65 + (i - k - 1)]) * V) >> 32)
            e += k + 1
    return out


def attn_inputs_stream(B: int, lk: int) -> int:
    """Philox stream id of one attention-microbenchmark point."""
    return (B << 20) | (lk >> 10)

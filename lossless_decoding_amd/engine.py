"""A decode engine over liborthrus with torch as the device-memory and stream
provider.  Host-side sequencing only (prefill, then draft -> verify -> commit
steps); all computation is in the library's kernels."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as C


def attn_chunk_for(max_ctx: int, max_batch: int = 1, n_kv_heads: int = 8) -> int:
    """The library's default attention key chunk for a context of max_batch
    sequences x max_ctx slots over n_kv_heads KV heads.  Two contexts give
    bit-identical attention rows only with the same chunk size, so a context
    and its greedy (K = 0) twin, or a batch and one of its sequences alone,
    should share one value (pass it explicitly as attn_chunk)."""
    return C.orthrus_default_attn_chunk(max_batch, max_ctx, n_kv_heads)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _buf(nbytes: int, device) -> torch.Tensor:
    # 256-byte aligned raw device buffer (the caching allocator aligns to 512)
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Engine:
    """One context: packed weights, KV cache, block scratch and workspace.

    weights: a device tensor holding the canonical weight buffer (see
    orthrus_weight_tensor); it is only read during construction."""

    def __init__(self, cfg: C.OrthrusConfig, weights: torch.Tensor, device="cuda"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.sizes = C.orthrus_query_sizes(cfg)
        self.K = cfg.block_k
        self.packed = _buf(self.sizes.packed_bytes, self.device)
        self.kv = _buf(self.sizes.kv_bytes, self.device)
        self.scratch = _buf(self.sizes.scratch_bytes, self.device)
        self.ws = _buf(self.sizes.workspace_bytes, self.device)
        self.stream = torch.cuda.current_stream(self.device)
        self.ctx = C.orthrus_create(cfg, weights.data_ptr(), self.packed.data_ptr(),
                                    self.kv.data_ptr(), self.scratch.data_ptr(),
                                    self.ws.data_ptr(), self.stream.cuda_stream)
        B, K = cfg.max_batch, max(self.K, 1)
        i32 = dict(dtype=torch.int32, device=self.device)
        self.seq_len = torch.zeros(B, **i32)
        self.pending = torch.zeros(B, **i32)
        self.drafts = torch.zeros(B, K, **i32)
        self.ar = torch.zeros(B, self.K + 1, **i32)
        self.accept = torch.zeros(B, **i32)
        self.commit_start = torch.zeros(B, **i32)
        self.out_tokens = torch.zeros(B * (self.K + 1), **i32)
        self.out_off = torch.zeros(B + 1, **i32)
        self.B = 0

    def close(self):
        if getattr(self, "ctx", None):
            C.orthrus_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def s(self) -> int:
        return self.stream.cuda_stream

    def set_debug(self, logits: torch.Tensor | None, attn: torch.Tensor | None, rows: int):
        C.orthrus_set_debug(self.ctx, _ptr(logits), _ptr(attn), rows)

    def set_sampling(self, temperature: float, seed: int = 0):
        """T > 0: sampling with lossless rejection sampling; 0: greedy."""
        C.orthrus_set_sampling(self.ctx, float(temperature), int(seed))

    def set_debug_layers(self, resid: torch.Tensor | None, attn32: torch.Tensor | None, rows: int):
        C.orthrus_set_debug_layers(self.ctx, _ptr(resid), _ptr(attn32), rows)

    def prefill(self, prompts: np.ndarray, prompt_len=None):
        prompts = np.ascontiguousarray(prompts, np.int32)
        B, P = prompts.shape
        plen = np.full(B, P, np.int32) if prompt_len is None else np.asarray(prompt_len, np.int32)
        tok = torch.from_numpy(prompts).to(self.device)
        pl = torch.from_numpy(np.ascontiguousarray(plen)).to(self.device)
        self._prompt_dev = (tok, pl)
        C.orthrus_prefill(self.ctx, B, tok.data_ptr(), P, pl.data_ptr(), int(plen.max()),
                          self.seq_len.data_ptr(), self.pending.data_ptr(), self.s)
        self.B = B

    def draft(self, k: int | None = None):
        """Pass 1 with a block of k <= block_k masks (default block_k)."""
        C.orthrus_draft_block_k(self.ctx, self.B, self.K if k is None else int(k),
                                self.seq_len.data_ptr(), self.pending.data_ptr(),
                                self.drafts.data_ptr() if self.K else None, self.ar.data_ptr(),
                                self.s)

    def refine(self):
        """One more denoising pass over the outstanding block (2-step variant)."""
        C.orthrus_draft_refine(self.ctx, self.B, self.seq_len.data_ptr(), self.drafts.data_ptr(),
                               self.s)

    def verify(self):
        C.orthrus_verify_accept(self.ctx, self.B, self.seq_len.data_ptr(),
                                self.drafts.data_ptr() if self.K else None, self.ar.data_ptr(),
                                self.accept.data_ptr(), self.s)

    def commit(self):
        C.orthrus_commit_kv(self.ctx, self.B, self.accept.data_ptr(), self.ar.data_ptr(),
                            self.drafts.data_ptr() if self.K else None, self.seq_len.data_ptr(),
                            self.pending.data_ptr(), self.commit_start.data_ptr(),
                            self.out_tokens.data_ptr(), self.out_off.data_ptr(), self.s)

    def step(self, planted: torch.Tensor | None = None):
        self.draft()
        if planted is not None:
            self.drafts[:self.B].copy_(planted)
        self.verify()
        self.commit()

    def capture_step(self, planted: torch.Tensor | None = None) -> torch.cuda.CUDAGraph:
        """One greedy draft -> verify -> commit step of the current batch as
        a HIP graph (every call only enqueues work, none allocates or
        clears memory).  planted: optional device [B][K] int32 buffer whose
        contents replace the drafts at every replay (fill it before each
        replay).  Replay with graph.replay() on the engine's stream.  The
        launches are recorded as they are now: greedy decoding only (the
        sampling step counter is host state) and the batch size fixed.
        Replay it with replay(), which first reserves the step's capacity
        with the library (its host length bound, as an eager step would)."""
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(self.device)
        cap.wait_stream(self.stream)
        prev = self.stream
        try:
            with torch.cuda.graph(g, stream=cap):
                self.stream = cap
                self.step(planted)
        finally:
            self.stream = prev
        self.stream.wait_stream(cap)
        return g

    def replay(self, graph: torch.cuda.CUDAGraph, n: int = 1):
        """n replays of a captured step (capture_step), after reserving their
        capacity (ORTHRUS_ECAPACITY if a sequence could outgrow max_ctx)."""
        C.orthrus_reserve_steps(self.ctx, self.B, self.K, n)
        with torch.cuda.stream(self.stream):
            for _ in range(n):
                graph.replay()

    def generate(self, prompts: np.ndarray, n_new: int, planted=None, record=False, k_policy=None,
                 denoise_steps: int = 1):
        """Greedy generation of n_new tokens per sequence (token 1 is the
        prefill's).  planted: optional [steps][B][K] int32 drafts.  k_policy:
        optional block size per step (dynamic K): a callable (step index,
        accept lengths of the previous step or None) -> k <= block_k, e.g. a
        CertaintyK.  denoise_steps: diffusion passes per block (1 = single-step
        block projection; 2 = the 2-step iterative denoising variant).
        Returns (tokens [B][n_new], per-step records)."""
        self.prefill(prompts)
        B = self.B
        outs = [[int(t)] for t in self.pending[:B].cpu().tolist()]
        recs = []
        s = 0
        last_m = None
        while min(len(o) for o in outs) < n_new:
            n_before = self.seq_len[:B].clone() if record else None
            pl = None
            if planted is not None:
                if s >= planted.shape[0]:
                    break
                pl = torch.as_tensor(planted[s], dtype=torch.int32, device=self.device)
            k = self.K if k_policy is None else int(k_policy(s, last_m))
            self.draft(k)
            for _ in range(denoise_steps - 1):
                self.refine()
            if record:
                drafted = self.drafts[:B].clone()
            if pl is not None:
                self.drafts[:B].copy_(pl)
            self.verify()
            self.commit()
            last_m = self.accept[:B].cpu().numpy()
            off = self.out_off[:B + 1].cpu().numpy()
            C.orthrus_sync_lengths(self.ctx, B, self.seq_len[:B].cpu().numpy())
            tok = self.out_tokens[:off[-1]].cpu().numpy()
            for b in range(B):
                outs[b].extend(tok[off[b]:off[b + 1]].tolist())
            if record:
                recs.append(dict(k=k, n=n_before.cpu().numpy(), drafted=drafted.cpu().numpy(),
                                 drafts=self.drafts[:B].cpu().numpy(),
                                 ar=self.ar[:B].cpu().numpy(), m=self.accept[:B].cpu().numpy(),
                                 commit_start=self.commit_start[:B].cpu().numpy(),
                                 len=self.seq_len[:B].cpu().numpy()))
            s += 1
        return np.array([o[:n_new] for o in outs], np.int32), recs


class CertaintyK:
    """A dynamic-K policy: the pages propose adjusting K to the generation's
    certainty (openai-hub.net article, "Future Directions", item 1).  Taken
    here as: the accept lengths of the previous step measure how predictable
    the continuation is, so the next block holds twice the smallest accept
    length of the batch plus a margin, clamped to [k_min, k_max]; the first
    step uses k_max.  Any schedule is lossless (every emitted token is the
    AR argmax); K only changes how much work a step spends on drafts."""

    def __init__(self, k_max: int, k_min: int = 4, margin: int = 4):
        self.k_max, self.k_min, self.margin = k_max, min(k_min, k_max), margin

    def __call__(self, step: int, last_m) -> int:
        if last_m is None or len(last_m) == 0:
            return self.k_max
        k = 2 * int(np.min(last_m)) + self.margin
        return max(self.k_min, min(self.k_max, k))

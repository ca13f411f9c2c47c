"""ctypes binding of liborthrus.so.  Argument marshalling only: every step of
the decode path runs in the library's HIP kernels.  Loading fails loudly if
the library has not been built -- there is no fallback implementation."""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "liborthrus.so"

ORTHRUS_OK, ORTHRUS_EINVAL, ORTHRUS_ECAPACITY, ORTHRUS_ESTATE, ORTHRUS_EHIP = 0, -1, -2, -3, -4
ORTHRUS_F32, ORTHRUS_BF16 = 0, 1

EXPORTED = [
    "orthrus_query_sizes", "orthrus_weight_tensor", "orthrus_create", "orthrus_destroy",
    "orthrus_prefill", "orthrus_draft_block", "orthrus_draft_block_k", "orthrus_draft_refine", "orthrus_verify_accept", "orthrus_commit_kv",
    "orthrus_set_debug", "orthrus_set_debug_layers", "orthrus_set_sampling", "orthrus_sync_lengths", "orthrus_timing_enable", "orthrus_timing_read", "orthrus_block_attention", "orthrus_block_attention_noalloc", "orthrus_attention_workspace",
    "orthrus_default_attn_chunk", "orthrus_stream_read", "orthrus_gemm_plan", "orthrus_reserve_steps",
    "orthrus_strerror", "orthrus_last_hip_error",
]


class OrthrusError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = lib().orthrus_strerror(code).decode()
        if code == ORTHRUS_EHIP:
            msg += f" (hipError {lib().orthrus_last_hip_error()})"
        super().__init__(f"{fn}: {msg} ({code})")
        self.code = code


class OrthrusConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_dim", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_double),
                ("dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("attn_chunk", ctypes.c_int32)]

    @classmethod
    def make(cls, L, d, hq, hkv, hd, F, V, K, bf16, max_batch, max_ctx, theta=1e6, eps=1e-6,
             attn_chunk=0):
        return cls(L, d, hq, hkv, hd, F, V, K, theta, eps, ORTHRUS_BF16 if bf16 else ORTHRUS_F32,
                   max_batch, max_ctx, attn_chunk)


class OrthrusSizes(ctypes.Structure):
    _fields_ = [("weights_bytes", ctypes.c_uint64), ("packed_bytes", ctypes.c_uint64),
                ("kv_bytes", ctypes.c_uint64), ("scratch_bytes", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64), ("kv_slots", ctypes.c_uint64),
                ("prefill_rows", ctypes.c_uint64)]


_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def lib():
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(there is no non-HIP implementation of the decode path)")
        L = ctypes.CDLL(path)
        vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
        cfgp = ctypes.POINTER(OrthrusConfig)
        L.orthrus_query_sizes.argtypes = [cfgp, ctypes.POINTER(OrthrusSizes)]
        L.orthrus_weight_tensor.argtypes = [cfgp, i32, ctypes.POINTER(u64), ctypes.POINTER(u64)]
        L.orthrus_create.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(vp)]
        L.orthrus_destroy.argtypes = [vp]
        L.orthrus_prefill.argtypes = [vp, i32, vp, i32, vp, i32, vp, vp, vp]
        L.orthrus_draft_block.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        L.orthrus_draft_block_k.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
        L.orthrus_draft_refine.argtypes = [vp, i32, vp, vp, vp]
        L.orthrus_verify_accept.argtypes = [vp, i32, vp, vp, vp, vp, vp]
        L.orthrus_commit_kv.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orthrus_set_debug.argtypes = [vp, vp, vp, i32]
        L.orthrus_set_debug_layers.argtypes = [vp, vp, vp, i32]
        L.orthrus_set_sampling.argtypes = [vp, ctypes.c_float, ctypes.c_uint64]
        L.orthrus_sync_lengths.argtypes = [vp, i32, vp]
        L.orthrus_reserve_steps.argtypes = [vp, i32, i32, i32]
        L.orthrus_timing_enable.argtypes = [vp, ctypes.c_uint32, i32]
        L.orthrus_timing_read.argtypes = [vp, vp, vp]
        L.orthrus_block_attention.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, vp,
                                              i32, vp, vp, u64, vp]
        L.orthrus_block_attention_noalloc.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, i32, vp,
                                                      vp, i32, vp, vp]
        L.orthrus_attention_workspace.argtypes = [i32, i32, i32, i32, i32]
        L.orthrus_attention_workspace.restype = u64
        L.orthrus_default_attn_chunk.argtypes = [i32, i32, i32]
        L.orthrus_stream_read.argtypes = [vp, u64, vp, i32, vp]
        L.orthrus_gemm_plan.argtypes = [i32, i32, i32, i32, i32, vp]
        L.orthrus_default_attn_chunk.restype = i32
        L.orthrus_strerror.argtypes = [ctypes.c_int]
        L.orthrus_strerror.restype = ctypes.c_char_p
        L.orthrus_last_hip_error.argtypes = []
        _lib = L
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != ORTHRUS_OK:
        raise OrthrusError(fn, rc)


# ---- same-name wrappers (pointers are ints: device addresses) -----------
def orthrus_query_sizes(cfg: OrthrusConfig) -> OrthrusSizes:
    s = OrthrusSizes()
    _check("orthrus_query_sizes", lib().orthrus_query_sizes(ctypes.byref(cfg), ctypes.byref(s)))
    return s


def orthrus_weight_tensor(cfg: OrthrusConfig, index: int):
    off, n = ctypes.c_uint64(), ctypes.c_uint64()
    _check("orthrus_weight_tensor",
           lib().orthrus_weight_tensor(ctypes.byref(cfg), index, ctypes.byref(off), ctypes.byref(n)))
    return off.value, n.value


def orthrus_create(cfg, weights, packed, kv, scratch, workspace, stream):
    h = ctypes.c_void_p()
    _check("orthrus_create", lib().orthrus_create(ctypes.byref(cfg), weights, packed, kv, scratch,
                                                  workspace, stream, ctypes.byref(h)))
    return h.value


def orthrus_destroy(ctx):
    _check("orthrus_destroy", lib().orthrus_destroy(ctx))


def orthrus_prefill(ctx, batch, tokens, stride, prompt_len, max_prompt_len, seq_len, pending,
                    stream):
    _check("orthrus_prefill", lib().orthrus_prefill(ctx, batch, tokens, stride, prompt_len,
                                                    max_prompt_len, seq_len, pending, stream))


def orthrus_draft_block(ctx, batch, seq_len, pending, drafts, ar_tokens, stream):
    _check("orthrus_draft_block",
           lib().orthrus_draft_block(ctx, batch, seq_len, pending, drafts, ar_tokens, stream))


def orthrus_draft_block_k(ctx, batch, k, seq_len, pending, drafts, ar_tokens, stream):
    _check("orthrus_draft_block_k",
           lib().orthrus_draft_block_k(ctx, batch, k, seq_len, pending, drafts, ar_tokens, stream))


def orthrus_draft_refine(ctx, batch, seq_len, drafts, stream):
    _check("orthrus_draft_refine", lib().orthrus_draft_refine(ctx, batch, seq_len, drafts, stream))


def orthrus_verify_accept(ctx, batch, seq_len, drafts, ar_tokens, accept_len, stream):
    _check("orthrus_verify_accept",
           lib().orthrus_verify_accept(ctx, batch, seq_len, drafts, ar_tokens, accept_len, stream))


def orthrus_commit_kv(ctx, batch, accept_len, ar_tokens, drafts, seq_len, pending, commit_start,
                      out_tokens, out_off, stream):
    _check("orthrus_commit_kv",
           lib().orthrus_commit_kv(ctx, batch, accept_len, ar_tokens, drafts, seq_len, pending,
                                   commit_start, out_tokens, out_off, stream))


def orthrus_set_debug(ctx, logits, attn, rows_cap):
    _check("orthrus_set_debug", lib().orthrus_set_debug(ctx, logits, attn, rows_cap))


def orthrus_set_sampling(ctx, temperature: float, seed: int):
    _check("orthrus_set_sampling", lib().orthrus_set_sampling(ctx, temperature, seed))


def orthrus_set_debug_layers(ctx, resid, attn32, rows_cap):
    _check("orthrus_set_debug_layers", lib().orthrus_set_debug_layers(ctx, resid, attn32, rows_cap))


def orthrus_reserve_steps(ctx, batch, k, n_steps):
    _check("orthrus_reserve_steps", lib().orthrus_reserve_steps(ctx, batch, k, n_steps))


def orthrus_sync_lengths(ctx, batch, seq_len_host: np.ndarray):
    sl = np.ascontiguousarray(seq_len_host, np.int32)
    _check("orthrus_sync_lengths", lib().orthrus_sync_lengths(ctx, batch, sl.ctypes.data))


TIMING_CLASSES = 24
TIMING_PASSES = ("draft", "verify", "prefill")
TIMING_ROLES = ("qkv", "attention", "o_proj", "gate_up", "down", "lm_head", "small", "accept_commit")


def timing_class(pass_name: str, role: str) -> int:
    return TIMING_PASSES.index(pass_name) * 8 + TIMING_ROLES.index(role)


def orthrus_timing_enable(ctx, class_mask: int, capacity: int):
    _check("orthrus_timing_enable", lib().orthrus_timing_enable(ctx, class_mask, capacity))


def orthrus_timing_read(ctx):
    """{(pass, role): (ms_total, launches)} for every class with launches."""
    ms = np.zeros(TIMING_CLASSES, np.float64)
    n = np.zeros(TIMING_CLASSES, np.int64)
    rc = lib().orthrus_timing_read(ctx, ms.ctypes.data, n.ctypes.data)
    if rc not in (ORTHRUS_OK, ORTHRUS_ECAPACITY):
        _check("orthrus_timing_read", rc)
    out = {}
    for k in range(TIMING_CLASSES):
        if n[k]:
            out[(TIMING_PASSES[k // 8], TIMING_ROLES[k % 8])] = (float(ms[k]), int(n[k]))
    return out, rc == ORTHRUS_ECAPACITY


def orthrus_attention_workspace(batch, rows, hq, hkv, ctx_len) -> int:
    return lib().orthrus_attention_workspace(batch, rows, hq, hkv, ctx_len)


def orthrus_block_attention_noalloc(batch, rows, hq, hkv, q, k_cache, v_cache, cap, ctx_len,
                                    k_block, v_block, block_len, out, stream):
    _check("orthrus_block_attention_noalloc",
           lib().orthrus_block_attention_noalloc(batch, rows, hq, hkv, q, k_cache, v_cache, cap,
                                                 ctx_len, k_block, v_block, block_len, out, stream))


def orthrus_stream_read(buf, nbytes, out, n_workgroups, stream):
    _check("orthrus_stream_read", lib().orthrus_stream_read(buf, nbytes, out, n_workgroups, stream))


EP_RESID, EP_SWIGLU, EP_ARGMAX, EP_QKV = 1, 2, 3, 4


def orthrus_gemm_plan(m, m2, n, k, epilogue) -> dict:
    """The launch shape of a bf16 GEMM (see include/orthrus.h)."""
    plan = np.zeros(6, np.int32)
    _check("orthrus_gemm_plan", lib().orthrus_gemm_plan(m, m2, n, k, epilogue, plan.ctypes.data))
    return dict(MT=int(plan[0]), WV=int(plan[1]), split=bool(plan[2]), CT=int(plan[3]),
                workgroups=int(plan[4]), form=int(plan[5]))


def orthrus_default_attn_chunk(max_batch, max_ctx, n_kv_heads) -> int:
    r = lib().orthrus_default_attn_chunk(max_batch, max_ctx, n_kv_heads)
    _check("orthrus_default_attn_chunk", min(r, 0))
    return r


def orthrus_block_attention(batch, rows, hq, hkv, q, k_cache, v_cache, cap, ctx_len, k_block,
                            v_block, block_len, out, workspace, workspace_bytes, stream):
    _check("orthrus_block_attention",
           lib().orthrus_block_attention(batch, rows, hq, hkv, q, k_cache, v_cache, cap, ctx_len,
                                         k_block, v_block, block_len, out, workspace,
                                         workspace_bytes, stream))


GAIN_SLOTS = (0, 1, 6, 7, 12, 13)   # per-layer RMSNorm gains (plus global tensor 2)


def weight_layout(cfg: OrthrusConfig):
    """[(tensor_index, offset_elems, numel, is_gain)] and the total element
    count of the canonical weight buffer, as the library defines it."""
    _, total = orthrus_weight_tensor(cfg, -1)
    out = []
    for t in range(4 + 17 * cfg.n_layers):
        off, n = orthrus_weight_tensor(cfg, t)
        gain = t == 2 or (t >= 4 and (t - 4) % 17 in GAIN_SLOTS)
        out.append((t, off, n, gain))
    return out, total

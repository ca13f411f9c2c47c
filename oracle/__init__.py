"""ctypes front end of the CPU oracle (oracle/orthrus_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the product path.  See the C file's
header for what is computed and which passages of the pages it follows.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liborthrus_oracle.so")
SRC_PATH = os.path.join(_HERE, "orthrus_oracle.c")

N_GLOBAL = 4
PER_LAYER = 17
# gain tensors (RMSNorm weights): final norm (global 2) and per-layer slots
GAIN_SLOTS = (0, 1, 6, 7, 12, 13)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math: summation order kept)."""
    if force or not os.path.exists(LIB_PATH):
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", LIB_PATH, SRC_PATH, "-lm"])
    return LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("d", ctypes.c_int32), ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32), ("hd", ctypes.c_int32), ("F", ctypes.c_int32),
                ("V", ctypes.c_int32), ("K", ctypes.c_int32), ("theta", ctypes.c_double),
                ("eps", ctypes.c_double), ("bf16", ctypes.c_int32)]


@dataclass(frozen=True)
class ModelShape:
    L: int
    d: int
    hq: int
    hkv: int
    hd: int
    F: int
    V: int
    K: int
    bf16: bool
    theta: float = 1e6
    eps: float = 1e-6

    def c(self) -> _Cfg:
        return _Cfg(self.L, self.d, self.hq, self.hkv, self.hd, self.F, self.V, self.K,
                    self.theta, self.eps, int(self.bf16))


_lib = None
I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def _configure(L):
    """Argument and result types of the oracle's C entry points."""
    vp, i32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    sz = ctypes.POINTER(ctypes.c_size_t)
    L.oc_num_tensors.argtypes = [ctypes.POINTER(_Cfg)]
    L.oc_weight_layout.argtypes = [ctypes.POINTER(_Cfg), i32, sz, sz]
    L.oc_round_bf16.argtypes = [dbl]; L.oc_round_bf16.restype = dbl
    L.oc_rmsnorm.argtypes = [F64P, vp, i32, dbl, F64P]
    L.oc_rope.argtypes = [F64P, i32, ctypes.c_long, dbl]
    L.oc_attention_dense.argtypes = [F64P, F64P, F64P, i32, i32, F64P]
    L.oc_silu.argtypes = [dbl]; L.oc_silu.restype = dbl
    L.oc_argmax.argtypes = [F64P, i32]
    L.oc_accept.argtypes = [I32P, I32P, i32]
    L.oc_model_new.argtypes = [ctypes.POINTER(_Cfg), vp]; L.oc_model_new.restype = vp
    L.oc_model_free.argtypes = [vp]
    L.oc_model_set_attn_tap.argtypes = [vp, vp, i32]
    L.oc_seq_new.argtypes = [vp, i32]; L.oc_seq_new.restype = vp
    L.oc_seq_free.argtypes = [vp]
    L.oc_seq_len.argtypes = [vp]
    L.oc_seq_set_len.argtypes = [vp, i32]
    L.oc_seq_checksum.argtypes = [vp, i32]; L.oc_seq_checksum.restype = dbl
    L.oc_ar_rows.argtypes = [vp, vp, I32P, i32, i32, vp, vp]
    L.oc_draft_rows.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp]
    L.oc_prefill.argtypes = [vp, vp, I32P, i32, vp]
    L.oc_step.argtypes = [vp, vp, ctypes.c_int32, i32, vp, vp, I32P, vp, vp, vp, I32P,
                          ctypes.POINTER(ctypes.c_int32)]
    L.oc_ar_generate.argtypes = [vp, I32P, i32, i32, I32P]
    L.oc_generate.argtypes = [vp, I32P, i32, i32, i32, vp, i32, I32P, vp, vp]
    L.oc_attention_many.argtypes = [F64P, F64P, F64P, i32, i32, i32, F64P]
    L.oc_seq_load_kv.argtypes = [vp, i32, F64P, F64P, i32]
    L.oc_seq_read_kv.argtypes = [vp, i32, F64P, F64P, i32]
    L.oc_ar_layer.argtypes = [vp, vp, i32, F64P, i32, i32, vp]
    L.oc_draft_layer.argtypes = [vp, vp, i32, F64P, i32, i32, i32, vp]
    L.oc_final.argtypes = [vp, F64P, i32, vp, vp]
    L.oc_layer_tail.argtypes = [vp, i32, i32, F64P, F64P, i32]
    U32P = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
    L.oc_philox4x32_10.argtypes = [U32P, U32P, U32P]
    L.oc_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                             ctypes.c_uint32]
    L.oc_uniform.restype = dbl
    L.oc_draw.argtypes = [F64P, i32, dbl]
    L.oc_sample_logits.argtypes = [F64P, i32, dbl, dbl]
    L.oc_spec_accept.argtypes = [F64P, F64P, I32P, i32, i32, dbl, F64P, dbl,
                                 ctypes.POINTER(ctypes.c_int32)]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _configure(ctypes.CDLL(LIB_PATH))
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the oracle from another build of its source (the mutation tests
    compile copies with one step removed and check that a pin fails)."""
    global _lib
    saved = _lib
    _lib = _configure(ctypes.CDLL(path))
    try:
        yield _lib
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data


# ------------------------------------------------------------------ layout
def weight_layout(shape: ModelShape):
    """[(tensor_index, offset, numel, is_gain)] plus the total element count."""
    c = shape.c()
    n = lib().oc_num_tensors(ctypes.byref(c))
    off, num = ctypes.c_size_t(), ctypes.c_size_t()
    out = []
    for t in range(n):
        lib().oc_weight_layout(ctypes.byref(c), t, ctypes.byref(off), ctypes.byref(num))
        gain = t == 2 or (t >= N_GLOBAL and (t - N_GLOBAL) % PER_LAYER in GAIN_SLOTS)
        out.append((t, off.value, num.value, gain))
    lib().oc_weight_layout(ctypes.byref(c), -1, ctypes.byref(off), ctypes.byref(num))
    return out, num.value


def tensor_view(shape: ModelShape, w: np.ndarray, t: int) -> np.ndarray:
    lay, _ = weight_layout(shape)
    _, off, n, _ = lay[t]
    return w[off:off + n]


# ------------------------------------------------------------- primitives
def round_bf16(x: float) -> float:
    return lib().oc_round_bf16(float(x))


def rmsnorm(x, g=None, eps=1e-6):
    x = np.ascontiguousarray(x, np.float64)
    y = np.empty_like(x)
    gp = None
    if g is not None:
        g = np.ascontiguousarray(g, np.float64)
        gp = g.ctypes.data
    lib().oc_rmsnorm(x, gp, x.size, eps, y)
    return y


def rope(v, pos, theta=1e6):
    v = np.array(v, np.float64)
    lib().oc_rope(v, v.size, int(pos), theta)
    return v


def attention(q, K, V):
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    out = np.empty(q.size, np.float64)
    lib().oc_attention_dense(q, K, V, K.shape[0], q.size, out)
    return out


def attention_many(q, K, V):
    """attention() of every row of q [nq, hd] over the same keys."""
    q = np.ascontiguousarray(q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    out = np.empty_like(q)
    lib().oc_attention_many(q, K, V, q.shape[0], K.shape[0], q.shape[1], out)
    return out


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oc_philox4x32_10(c, k, out)
    return out


def uniform(seed: int, step: int, purpose: int, index: int, seq: int) -> float:
    return lib().oc_uniform(seed, step, purpose, index, seq)


def draw(w, u: float) -> int:
    w = np.ascontiguousarray(w, np.float64)
    return lib().oc_draw(w, w.size, u)


def sample_logits(z, T: float, u: float) -> int:
    z = np.ascontiguousarray(z, np.float64)
    return lib().oc_sample_logits(z, z.size, T, u)


def spec_accept(pz, qz, d, T: float, ua, uf: float):
    """(m, final token) of one sequence: pz [K+1, V], qz [K, V], drafts d [K]."""
    pz = np.ascontiguousarray(pz, np.float64)
    qz = np.ascontiguousarray(qz, np.float64)
    d = np.ascontiguousarray(d, np.int32)
    ua = np.ascontiguousarray(ua, np.float64)
    K, V = qz.shape
    tok = ctypes.c_int32()
    m = lib().oc_spec_accept(pz, qz, d, K, V, T, ua, uf, ctypes.byref(tok))
    return m, tok.value


def silu(x):
    return lib().oc_silu(float(x))


def argmax(x):
    return lib().oc_argmax(np.ascontiguousarray(x, np.float64), len(x))


def accept(d, a):
    d = np.ascontiguousarray(d, np.int32)
    a = np.ascontiguousarray(a, np.int32)
    assert a.size == d.size + 1
    return lib().oc_accept(d, a, d.size)


# ------------------------------------------------------------------- model
class Model:
    """An oracle model over a canonical weight buffer (numpy float32 for
    fp32 models, uint16 bf16 bit patterns for bf16 models)."""

    def __init__(self, shape: ModelShape, weights: np.ndarray):
        _, total = weight_layout(shape)
        want = np.uint16 if shape.bf16 else np.float32
        assert weights.dtype == want and weights.size >= total
        self.shape = shape
        self.w = np.ascontiguousarray(weights)
        self._c = shape.c()
        self.h = lib().oc_model_new(ctypes.byref(self._c), self.w.ctypes.data)
        self._free = lib().oc_model_free     # held so that teardown needs no module globals
        self._tap = None

    def __del__(self):
        if getattr(self, "h", None):
            self._free(self.h)
            self.h = None

    def set_attn_tap(self, rows: int):
        s = self.shape
        self._tap = np.zeros((s.L, rows, s.hq * s.hd), np.float64)
        lib().oc_model_set_attn_tap(self.h, self._tap.ctypes.data, rows)
        return self._tap

    def seq(self, cap: int) -> "Seq":
        return Seq(self, cap)

    def layer_tail(self, layer: int, h, o, diffusion=False):
        """Layer `layer` after attention (O projection + residual, FFN +
        residual) for rows h [R, d] with attention outputs o [R, hq*hd]:
        the layer outputs [R, d]."""
        h = np.array(h, np.float64, order="C")
        o = np.ascontiguousarray(o, np.float64)
        rc = lib().oc_layer_tail(self.h, layer, int(diffusion), h, o, h.shape[0])
        assert rc == 0, rc
        return h

    def final(self, h):
        """Final RMSNorm + LM head of rows h [R, d]: (logits [R, V], argmax [R])."""
        h = np.ascontiguousarray(h, np.float64)
        R = h.shape[0]
        lg = np.zeros((R, self.shape.V), np.float64)
        am = np.zeros(R, np.int32)
        lib().oc_final(self.h, h, R, lg.ctypes.data, am.ctypes.data)
        return lg, am

    def ar_generate(self, prompt, n_new: int) -> np.ndarray:
        prompt = np.ascontiguousarray(prompt, np.int32)
        out = np.zeros(n_new, np.int32)
        rc = lib().oc_ar_generate(self.h, prompt, prompt.size, n_new, out)
        assert rc == 0, rc
        return out

    def generate(self, prompt, n_new: int, K: int, planted=None, max_steps: int = 1 << 20):
        prompt = np.ascontiguousarray(prompt, np.int32)
        out = np.zeros(n_new, np.int32)
        cap_steps = min(max_steps, n_new + 1)
        acc = np.zeros(cap_steps, np.int32)
        lens = np.zeros(cap_steps, np.int32)
        pl = None if planted is None else np.ascontiguousarray(planted, np.int32)
        if pl is not None:
            cap_steps = min(cap_steps, pl.shape[0])
        steps = lib().oc_generate(self.h, prompt, prompt.size, n_new, K, _ptr(pl), cap_steps, out,
                                  acc.ctypes.data, lens.ctypes.data)
        assert steps >= 0, steps
        return out, acc[:steps], lens[:steps]


class Seq:
    def __init__(self, model: Model, cap: int):
        self.m = model
        self.h = lib().oc_seq_new(model.h, cap)
        self._free = lib().oc_seq_free
        self.cap = cap

    def __del__(self):
        if getattr(self, "h", None):
            self._free(self.h)
            self.h = None

    @property
    def len(self) -> int:
        return lib().oc_seq_len(self.h)

    @len.setter
    def len(self, v: int):
        lib().oc_seq_set_len(self.h, v)

    def checksum(self, upto: int) -> float:
        return lib().oc_seq_checksum(self.h, upto)

    def prefill(self, prompt, want_logits=False):
        prompt = np.ascontiguousarray(prompt, np.int32)
        lg = np.zeros(self.m.shape.V, np.float64) if want_logits else None
        tok = lib().oc_prefill(self.m.h, self.h, prompt, prompt.size, _ptr(lg))
        assert tok >= 0, tok
        return (tok, lg) if want_logits else tok

    def ar_rows(self, tokens, pos0: int):
        tokens = np.ascontiguousarray(tokens, np.int32)
        R, V = tokens.size, self.m.shape.V
        lg = np.zeros((R, V), np.float64)
        am = np.zeros(R, np.int32)
        rc = lib().oc_ar_rows(self.m.h, self.h, tokens, R, pos0, lg.ctypes.data, am.ctypes.data)
        assert rc == 0, rc
        return lg, am

    def load_kv(self, layer: int, k, v):
        """Cache slots [0, n) of one layer from K, V [hkv, n, hd]."""
        k = np.ascontiguousarray(k, np.float64)
        v = np.ascontiguousarray(v, np.float64)
        assert k.shape == v.shape and k.shape[0] == self.m.shape.hkv
        rc = lib().oc_seq_load_kv(self.h, layer, k, v, k.shape[1])
        assert rc == 0, rc

    def read_kv(self, layer: int, n: int):
        """Cache slots [0, n) of one layer as K, V [hkv, n, hd]."""
        s = self.m.shape
        k = np.zeros((s.hkv, n, s.hd), np.float64)
        v = np.zeros_like(k)
        rc = lib().oc_seq_read_kv(self.h, layer, k, v, n)
        assert rc == 0, rc
        return k, v

    def ar_layer(self, layer: int, h, pos0: int):
        """One frozen-view layer for rows at pos0.. from inputs h [R, d]:
        (layer outputs [R, d], attention output before rounding [R, hq*hd]);
        writes the rows' K/V into this layer's cache slots."""
        h = np.array(h, np.float64, order="C")
        s = self.m.shape
        o = np.zeros((h.shape[0], s.hq * s.hd), np.float64)
        rc = lib().oc_ar_layer(self.m.h, self.h, layer, h, h.shape[0], pos0, o.ctypes.data)
        assert rc == 0, rc
        return h, o

    def draft_layer(self, layer: int, h, n: int, causal=False):
        """One diffusion-view layer for the mask rows at n+1.. from inputs
        h [K, d] (keys: cache [0, n] plus the block)."""
        h = np.array(h, np.float64, order="C")
        s = self.m.shape
        o = np.zeros((h.shape[0], s.hq * s.hd), np.float64)
        rc = lib().oc_draft_layer(self.m.h, self.h, layer, h, n, h.shape[0], int(causal),
                                  o.ctypes.data)
        assert rc == 0, rc
        return h, o

    def draft_rows(self, n: int, K: int, in_tokens=None, causal=False):
        V = self.m.shape.V
        lg = np.zeros((K, V), np.float64)
        am = np.zeros(K, np.int32)
        it = None if in_tokens is None else np.ascontiguousarray(in_tokens, np.int32)
        rc = lib().oc_draft_rows(self.m.h, self.h, n, K, _ptr(it), int(causal), lg.ctypes.data,
                                 am.ctypes.data)
        assert rc == 0, rc
        return lg, am

    def step(self, pending: int, K: int, planted=None):
        """One draft/verify/accept/commit step; returns a dict of everything."""
        V = self.m.shape.V
        drafts = np.zeros(max(K, 1), np.int32)
        ar = np.zeros(K + 1, np.int32)
        la = np.zeros(V, np.float64)
        ld = np.zeros((max(K, 1), V), np.float64)
        lv = np.zeros((max(K, 1), V), np.float64)
        em = np.zeros(K + 1, np.int32)
        npend = ctypes.c_int32()
        pl = None if planted is None else np.ascontiguousarray(planted, np.int32)
        n0 = self.len
        m = lib().oc_step(self.m.h, self.h, int(pending), K, _ptr(pl), drafts.ctypes.data, ar,
                          la.ctypes.data, ld.ctypes.data, lv.ctypes.data, em, ctypes.byref(npend))
        assert m >= 0, m
        return dict(n=n0, m=m, drafts=drafts[:K], ar=ar, emitted=em[:m + 1], pending=npend.value,
                    logits_anchor=la, logits_draft=ld[:K], logits_verify=lv[:K],
                    commit_start=n0, len=self.len)

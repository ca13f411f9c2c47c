"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no arithmetic of the decoding method.  It only turns
(seed, stream, purpose, element index) into numbers, so that the CPU oracle
and the GPU library can be fed bit-identical inputs without either of them
reading the other's results.

Generator: Philox4x32-10, the counter-based generator published by Salmon,
Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
For element ``i`` of stream ``t`` with purpose ``p`` under seed ``s``:

    counter = (i mod 2^32, i div 2^32, t, p),  key = (s mod 2^32, s div 2^32)

and the four 32-bit outputs ``x0..x3`` are turned into values without any
transcendental function, so every platform reproduces them bit for bit:

* ``normal(sigma)``: Irwin-Hall sum of the eight 16-bit halves of x0..x3,
  centred and scaled to standard deviation ``sigma`` with ONE fp32 multiply:
  ``float(S - 262140) * float(sigma / sqrt(8 * (65536**2 - 1) / 12))``.
  The integer S is exact in fp32, so the product is correctly rounded once.
  (An approximately normal law with bounded +-4.9 sigma tails; the model is
  random-init, so only the mean and variance matter.)
* ``ones``: the constant 1.0 (RMSNorm gains).
* token ids uniform on [0, V): ``(x0 * V) >> 32`` (Lemire's multiply-shift).

bf16 values are the fp32 values rounded to nearest-even.

Three implementations exist: this numpy one (the specification, used for
small tensors), ``synth.c`` (host, OpenMP, for multi-GB tensors) and
``synth_dev.hip`` (device fill).  Tests check they agree bit for bit.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

# purposes (the 4th counter word)
P_WEIGHTS = 0
P_TOKENS = 1
P_PLANT = 2
P_ATTN = 3

IH_CENTER = 8 * 65535 // 2          # 262140, mean of the 8-term Irwin-Hall sum
IH_SD = float(np.sqrt(8.0 * (65536.0 ** 2 - 1.0) / 12.0))


def normal_scale(sigma: float) -> np.float32:
    """fp32 multiplier that maps the centred Irwin-Hall sum to std ``sigma``."""
    return np.float32(sigma / IH_SD)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32 with 10 rounds.  Inputs are uint64 arrays/scalars
    holding 32-bit values; returns four uint64 arrays of 32-bit values."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    k0 = np.uint64(k0)
    k1 = np.uint64(k1)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    mask = np.uint64(MASK32)
    s32 = np.uint64(32)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(PHILOX_W1)) & mask
        p0 = m0 * c0            # < 2^64, exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> s32, p0 & mask
        hi1, lo1 = p1 >> s32, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def _raw(n: int, seed: int, stream: int, purpose: int, start: int = 0):
    idx = np.arange(start, start + n, dtype=np.uint64)
    return philox4x32_10(idx & np.uint64(MASK32), idx >> np.uint64(32),
                         np.full(n, stream, np.uint64), np.full(n, purpose, np.uint64),
                         seed & MASK32, (seed >> 32) & MASK32)


def irwin_hall_sum(x0, x1, x2, x3):
    s = np.zeros(np.shape(x0), dtype=np.int64)
    for x in (x0, x1, x2, x3):
        x = x.astype(np.int64)
        s += (x & 0xFFFF) + (x >> 16)
    return s


def normal_f32(n: int, seed: int, stream: int, sigma: float, purpose: int = P_WEIGHTS,
               start: int = 0) -> np.ndarray:
    """``n`` fp32 values of element indices [start, start+n) of one stream."""
    s = irwin_hall_sum(*_raw(n, seed, stream, purpose, start))
    return (s - IH_CENTER).astype(np.float32) * normal_scale(sigma)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rnd = ((b >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((b + rnd) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tokens(n: int, vocab: int, seed: int, stream: int, purpose: int = P_TOKENS) -> np.ndarray:
    """``n`` token ids uniform on [0, vocab)."""
    x0, _, _, _ = _raw(n, seed, stream, purpose)
    return ((x0 * np.uint64(vocab)) >> np.uint64(32)).astype(np.int32)


def uniform_u32(n: int, seed: int, stream: int, purpose: int, start: int = 0):
    """All four 32-bit words for element indices [start, start+n)."""
    return _raw(n, seed, stream, purpose, start)


# --------------------------------------------------------------------------
# Optional compiled generators (same definition, faster for big tensors)
# --------------------------------------------------------------------------
_HERE = os.path.dirname(os.path.abspath(__file__))
_host_lib = None
_dev_lib = None


def host_lib():
    """ctypes handle to synth/libsynth.so (host OpenMP generator)."""
    global _host_lib
    if _host_lib is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_float, ctypes.c_int]
        lib.synth_fill_normal.restype = None
        _host_lib = lib
    return _host_lib


def dev_lib():
    """ctypes handle to synth/libsynth_dev.so (device fill kernels)."""
    global _dev_lib
    if _dev_lib is None:
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_dev_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                              ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                              ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.synth_dev_fill_normal.restype = ctypes.c_int
        lib.synth_dev_fill_const.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_float,
                                             ctypes.c_int, ctypes.c_void_p]
        lib.synth_dev_fill_const.restype = ctypes.c_int
        _dev_lib = lib
    return _dev_lib


def host_fill_normal(out: np.ndarray, seed: int, stream: int, sigma: float,
                     purpose: int = P_WEIGHTS, start: int = 0) -> None:
    """Fill a contiguous float32 or uint16(bf16) numpy array with the compiled
    host generator (same values as :func:`normal_f32`)."""
    assert out.flags.c_contiguous
    if out.dtype == np.float32:
        kind = 0
    elif out.dtype == np.uint16:
        kind = 1
    else:
        raise TypeError(out.dtype)
    host_lib().synth_fill_normal(out.ctypes.data, out.size, start, seed, stream, purpose,
                                 float(normal_scale(sigma)), kind)

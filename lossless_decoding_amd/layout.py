"""Host-side helpers for the library's documented cache layouts (plain torch
gathers; used by tests and benchmarks that build caches directly).

V is stored per 64-key tile transposed, [..., tiles, 128 dims, 64 keys]; key
j of a tile sits at column (j//32)*32 + ((j%16)//4)*8 + ((j%32)//16)*4 + j%4,
so one 16-byte LDS read gives an MFMA lane its 8 P.V keys (the layout
include/orthrus.h documents for orthrus_block_attention)."""
import numpy as np
import torch


def vt_cols() -> np.ndarray:
    j = np.arange(64)
    return (j // 32) * 32 + ((j % 16) // 4) * 8 + ((j % 32) // 16) * 4 + j % 4


def tile_v(v: torch.Tensor) -> torch.Tensor:
    """[..., L (multiple of 64), 128] logical -> [..., L/64, 128, 64] tiled."""
    *lead, L, d = v.shape
    t = v.reshape(*lead, L // 64, 64, d).transpose(-1, -2)       # [.., tiles, 128, 64 keys]
    out = torch.empty_like(t)
    out[..., torch.as_tensor(vt_cols(), device=v.device)] = t
    return out.contiguous()


def tile_block_v(v: torch.Tensor, kpad: int) -> torch.Tensor:
    """[..., Kb <= 64, 128] -> [..., 128, kpad] with the same key-to-column map."""
    *lead, Kb, d = v.shape
    out = torch.zeros(*lead, d, kpad, dtype=v.dtype, device=v.device)
    cols = torch.as_tensor(vt_cols()[:Kb], device=v.device)
    out[..., cols] = v.transpose(-1, -2)
    return out


def untile_v(vt: torch.Tensor) -> torch.Tensor:
    """[..., tiles, 128, 64] tiled -> [..., tiles * 64, 128] logical (inverse of tile_v)."""
    *lead, nt, d, _ = vt.shape
    cols = torch.as_tensor(vt_cols(), device=vt.device)
    return vt[..., cols].transpose(-1, -2).reshape(*lead, nt * 64, d)

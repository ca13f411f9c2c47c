"""Seeded inputs written straight into device memory (torch tensors) with
synth's device generator; the same values as the numpy specification."""
from __future__ import annotations

import torch

from . import P_WEIGHTS, dev_lib, normal_scale
from .workloads import SIGMA, WEIGHT_SEED


def fill_weights_device(layout, total: int, bf16: bool, seed: int = WEIGHT_SEED,
                        sigma: float = SIGMA, device="cuda") -> torch.Tensor:
    """Canonical weight buffer on the device.  layout: [(tensor_index,
    offset_elems, numel, is_gain)]."""
    dt = torch.int16 if bf16 else torch.float32
    w = torch.empty(total, dtype=dt, device=device)
    stream = torch.cuda.current_stream(device).cuda_stream
    esz = 2 if bf16 else 4
    L = dev_lib()
    for t, off, n, gain in layout:
        ptr = w.data_ptr() + off * esz
        if gain:
            rc = L.synth_dev_fill_const(ptr, n, 1.0, int(bf16), stream)
        else:
            rc = L.synth_dev_fill_normal(ptr, n, 0, seed, t, P_WEIGHTS,
                                         float(normal_scale(sigma)), int(bf16), stream)
        if rc != 0:
            raise RuntimeError(f"synth device fill failed ({rc})")
    return w


def fill_normal_device(t: torch.Tensor, seed: int, stream_id: int, sigma: float, purpose: int):
    """Fill a contiguous float32 or bf16 tensor in place."""
    assert t.is_contiguous() and t.dtype in (torch.float32, torch.bfloat16, torch.int16)
    kind = 0 if t.dtype == torch.float32 else 1
    rc = dev_lib().synth_dev_fill_normal(t.data_ptr(), t.numel(), 0, seed, stream_id, purpose,
                                         float(normal_scale(sigma)), kind,
                                         torch.cuda.current_stream(t.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth device fill failed ({rc})")

"""Shared test helpers: oracle models over synth's seeded weights."""
import numpy as np

import oracle
from synth import workloads

DIFF_SLOTS = (8, 9, 10, 11)          # diffusion Q/K/V/O matrices (per layer)


def shape(name, **over):
    d = dict(workloads.SHAPES[name])
    d.update(over)
    return oracle.ModelShape(**d)


def weights(shp, seed=workloads.WEIGHT_SEED):
    lay, total = oracle.weight_layout(shp)
    return workloads.fill_weights(lay, total, shp.bf16, seed)


def tensor(shp, w, t):
    return oracle.tensor_view(shp, w, t)


def layer_tensor(shp, w, layer, slot):
    return tensor(shp, w, oracle.N_GLOBAL + oracle.PER_LAYER * layer + slot)


def reseed_diffusion(shp, w, seed):
    """Replace only the diffusion-path matrices with those of another seed."""
    other = weights(shp, seed)
    w = w.copy()
    for l in range(shp.L):
        for s in DIFF_SLOTS:
            layer_tensor(shp, w, l, s)[:] = layer_tensor(shp, other, l, s)
    return w


def as_f64(shp, x):
    x = np.asarray(x)
    if shp.bf16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)

"""Orthrus dual-view decode step on MI355X (gfx950): ctypes binding of
liborthrus (include/orthrus.h) and a torch-memory engine around it."""
from ._lib import (ORTHRUS_BF16, ORTHRUS_F32, OrthrusConfig, OrthrusError, OrthrusSizes, lib,
                   lib_path)

__all__ = ["ORTHRUS_BF16", "ORTHRUS_F32", "OrthrusConfig", "OrthrusError", "OrthrusSizes", "lib",
           "lib_path"]

"""Fused int4 group-32 Mixture-of-Experts layer for AMD Instinct MI355X.

The layer runs in hand-written HIP kernels for gfx950 inside libqmoe.so
(C ABI: include/qmoe.h).  This package is its Python binding; it needs the
in-tree library and never falls back to another implementation.
"""
from ._binding import (QMOE_ERR_ARG, QMOE_ERR_DEVICE, QMOE_ERR_LAUNCH, QMOE_ERR_UNSUPPORTED,  # noqa: F401
                       QMOE_ERR_WORKSPACE, QMOE_OK, QmoeError, lib_path, load_library)

__all__ = ["Layer", "layer_from_numpy", "QmoeError", "load_library", "lib_path"]


def __getattr__(name):
    # the torch-facing wrapper is imported lazily so that the C ABI can be
    # loaded and inspected without initialising torch
    if name in ("Layer", "layer_from_numpy"):
        from . import layer
        return getattr(layer, name)
    raise AttributeError(name)

"""ctypes binding of libqmoe.so (the C ABI in include/qmoe.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the layer runs in the library's kernels.
If the library is missing this module raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libqmoe.so"

QMOE_OK = 0
QMOE_ERR_ARG = -1
QMOE_ERR_UNSUPPORTED = -2
QMOE_ERR_WORKSPACE = -3
QMOE_ERR_DEVICE = -4
QMOE_ERR_LAUNCH = -5


class QmoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"qmoe error {code}: {message}")
        self.code = code
        self.message = message


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("group_size", ctypes.c_int32), ("max_rows", ctypes.c_int32),
        ("w13", ctypes.c_void_p), ("s13", ctypes.c_void_p),
        ("w2", ctypes.c_void_p), ("s2", ctypes.c_void_p),
        ("shared_w13", ctypes.c_void_p), ("shared_s13", ctypes.c_void_p),
        ("shared_w2", ctypes.c_void_p), ("shared_s2", ctypes.c_void_p),
        ("local_first", ctypes.c_int32), ("local_count", ctypes.c_int32),
        ("scoring", ctypes.c_int32), ("routed_scale", ctypes.c_float), ("expert_bias", ctypes.c_void_p),
    ]


SCORING_SOFTMAX, SCORING_SIGMOID = 0, 1


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "forward_calls", "route_calls", "gemm_launches", "launches", "workspace_inits",
        "workspace_bytes_last", "workspace_bytes_peak", "prefill_tiles", "gemv_tiles",
        "gemv_nt_launches", "splitk_launches")]

    def as_dict(self) -> dict:
        return {n: int(getattr(self, n)) for n, _ in self._fields_}


class Receipt(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_uint64), ("M", ctypes.c_int64), ("regime", ctypes.c_int32),
                ("rows_per_item", ctypes.c_int32), ("nt_codes", ctypes.c_int32), ("shared_expert", ctypes.c_int32),
                ("launches", ctypes.c_int32), ("route_kernels", ctypes.c_int32), ("max_items", ctypes.c_int64),
                ("gate_up_blocks", ctypes.c_int64), ("down_blocks", ctypes.c_int64),
                ("combine_blocks", ctypes.c_int64), ("workspace_bytes", ctypes.c_uint64),
                ("static_scratch", ctypes.c_int32), ("router", ctypes.c_int32),
                ("splits_gate_up", ctypes.c_int32), ("splits_down", ctypes.c_int32)]

    def as_dict(self) -> dict:
        d = {n: int(getattr(self, n)) for n, _ in self._fields_}
        d["regime"] = {1: "gemv", 2: "tiles", 3: "mixed"}.get(d["regime"], d["regime"])
        return d


_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/qmoe.h
SIGNATURES = {
    "qmoe_version": (ctypes.c_int, []),
    "qmoe_last_error": (ctypes.c_char_p, []),
    "qmoe_layer_create": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(_VP)]),
    "qmoe_layer_destroy": (None, [_VP]),
    "qmoe_workspace_size": (ctypes.c_int, [_VP, _I64, ctypes.POINTER(_SZ)]),
    "qmoe_workspace_init": (ctypes.c_int, [_VP, _VP, _SZ, _VP]),
    "qmoe_forward": (ctypes.c_int, [_VP, _VP, _VP, _I64, _VP, _VP, _SZ, _VP]),
    "qmoe_forward_static": (ctypes.c_int, [_VP, _VP, _VP, _I64, _VP, _VP]),
    "qmoe_router_logits": (ctypes.c_int, [_VP, _VP, _VP, _I64, _VP, _VP]),
    "qmoe_forward_router": (ctypes.c_int, [_VP, _VP, _VP, _I64, _VP, _VP, _SZ, _VP]),
    "qmoe_route": (ctypes.c_int, [_VP, _VP, _VP, _I64, _VP, _SZ, _VP]),
    "qmoe_gate_up": (ctypes.c_int, [_VP, _I64, _VP, _SZ, _VP]),
    "qmoe_down": (ctypes.c_int, [_VP, _I64, _VP, _SZ, _VP]),
    "qmoe_combine": (ctypes.c_int, [_VP, _I64, _VP, _VP, _SZ, _VP]),
    "qmoe_read_routing": (ctypes.c_int, [_VP, _I64, _VP, _SZ, _VP, _VP, _VP, _VP, _VP, _VP]),
    "qmoe_read_intermediate": (ctypes.c_int, [_VP, _I64, _VP, _SZ, _I32, _VP, _VP]),
    "qmoe_dequant_debug": (ctypes.c_int, [_VP, _I32, _I32, _VP, _VP]),
    "qmoe_get_stats": (ctypes.c_int, [_VP, ctypes.POINTER(Stats)]),
    "qmoe_reset_stats": (ctypes.c_int, [_VP]),
    "qmoe_last_receipt": (ctypes.c_int, [_VP, ctypes.POINTER(Receipt)]),
    "qmoe_read_item_count": (ctypes.c_int, [_VP, _I64, _VP, _SZ, _VP, _VP]),
}

ABI_VERSION = 4  # QMOE_VERSION of include/qmoe.h
_lib = None


def lib_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library():
    """Load the in-tree libqmoe.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.qmoe_version() != ABI_VERSION:  # the structs above follow this version's header
        raise RuntimeError(f"{path} has ABI version {lib.qmoe_version()}, this binding expects "
                           f"{ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != QMOE_OK:
        raise QmoeError(rc, load_library().qmoe_last_error().decode())

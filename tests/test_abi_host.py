"""The C ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments before any device query."""
import ctypes
import os
import re

import pytest

from quantized_mixture_experts_top_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        pytest.fail("libqmoe.so is not built (run __graft_entry__.build())")
    return B.load_library()


def test_header_declares_the_boundary():
    names = _header_functions()
    for required in ("qmoe_layer_create", "qmoe_forward", "qmoe_route", "qmoe_gate_up", "qmoe_down",
                     "qmoe_combine", "qmoe_workspace_size", "qmoe_dequant_debug", "qmoe_last_error"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in _header_functions():
        assert hasattr(lib, name), name
    # and the binding mirrors the header one to one
    assert sorted(B.SIGNATURES) == _header_functions()


def test_version(lib):
    assert lib.qmoe_version() == B.ABI_VERSION == 4


def _desc(**kw):
    d = dict(E=8, H=256, I=128, top_k=2, group_size=32, max_rows=16,
             w13=0x1000, s13=0x2000, w2=0x3000, s2=0x4000,
             shared_w13=None, shared_s13=None, shared_w2=None, shared_s2=None)
    d.update(kw)
    desc = B.LayerDesc(d["E"], d["H"], d["I"], d["top_k"], d["group_size"], d["max_rows"],
                       d["w13"], d["s13"], d["w2"], d["s2"],
                       d["shared_w13"], d["shared_s13"], d["shared_w2"], d["shared_s2"])
    for f in ("local_first", "local_count", "scoring", "routed_scale", "expert_bias"):
        if f in d:
            setattr(desc, f, d[f])
    return desc


@pytest.mark.parametrize("field,value,needle", [
    ("E", 0, "E must"), ("E", 1025, "E must"), ("H", 33, "H must"), ("H", 0, "H must"),
    ("H", 160, "H must"), ("I", 48, "I must"), ("I", 96, "I must"), ("top_k", 0, "top_k"), ("top_k", 9, "top_k"), ("group_size", 64, "group_size"),
    ("max_rows", 0, "max_rows"), ("w13", None, "w13"), ("s13", None, "s13"), ("w2", None, "w2"),
    ("s2", None, "s2"), ("shared_w13", 0x5000, "shared expert"), ("w13", 0x1001, "aligned"),
    ("local_count", 9, "local experts"), ("scoring", 2, "scoring must"),
    ("expert_bias", 0x6000, "expert_bias is only"), ("routed_scale", -1.0, "routed_scale"),
    ("routed_scale", float("nan"), "routed_scale"), ("routed_scale", float("inf"), "routed_scale"),
])
def test_create_rejects_bad_fields(lib, field, value, needle):
    h = ctypes.c_void_p()
    rc = lib.qmoe_layer_create(ctypes.byref(_desc(**{field: value})), ctypes.byref(h))
    assert rc == B.QMOE_ERR_ARG
    assert needle in lib.qmoe_last_error().decode()
    assert not h.value


def test_library_reads_no_environment():
    """No kernel path is chosen from the environment: the library source
    calls no getenv."""
    src = open(os.path.join(ROOT, "quantized_mixture_experts_top_amd", "csrc", "qmoe.hip")).read()
    assert "getenv" not in src


def test_create_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.qmoe_layer_create(None, ctypes.byref(h)) == B.QMOE_ERR_ARG
    assert "desc" in lib.qmoe_last_error().decode()
    assert lib.qmoe_layer_create(ctypes.byref(_desc()), None) == B.QMOE_ERR_ARG


def test_valid_description_without_gpu_fails_on_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    rc = lib.qmoe_layer_create(ctypes.byref(_desc()), ctypes.byref(h))
    assert rc in (B.QMOE_ERR_DEVICE, B.QMOE_ERR_UNSUPPORTED)
    assert not h.value


def test_calls_on_null_layer(lib):
    n = ctypes.c_size_t()
    assert lib.qmoe_workspace_size(None, 1, ctypes.byref(n)) == B.QMOE_ERR_ARG
    assert lib.qmoe_forward(None, None, None, 1, None, None, 0, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_route(None, None, None, 1, None, 0, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_gate_up(None, 1, None, 0, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_down(None, 1, None, 0, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_combine(None, 1, None, None, 0, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_dequant_debug(None, 0, 0, None, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_reset_stats(None) == B.QMOE_ERR_ARG
    s = B.Stats()
    assert lib.qmoe_get_stats(None, ctypes.byref(s)) == B.QMOE_ERR_ARG
    assert lib.qmoe_workspace_init(None, None, 0, None) == B.QMOE_ERR_ARG
    r = B.Receipt()
    assert lib.qmoe_last_receipt(None, ctypes.byref(r)) == B.QMOE_ERR_ARG
    assert lib.qmoe_read_item_count(None, 1, None, 0, None, None) == B.QMOE_ERR_ARG
    assert lib.qmoe_forward_static(None, None, None, 1, None, None) == B.QMOE_ERR_ARG
    lib.qmoe_layer_destroy(None)  # no-op


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_HERE", str(tmp_path))
    with pytest.raises(RuntimeError, match="missing"):
        B.load_library()


def test_layer_rejects_short_weight_arrays(lib):
    """Creation copies the codes and scales into the tile order, so the
    torch wrapper refuses an array shorter than its full size before the
    library reads it (CPU tensors: the size check comes first)."""
    import torch
    from quantized_mixture_experts_top_amd import Layer
    E, H, I = 4, 256, 128
    full = dict(w13=torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8),
                s13=torch.zeros((E, 2 * I, H // 32), dtype=torch.int16),
                w2=torch.zeros((E, H, I // 2), dtype=torch.uint8),
                s2=torch.zeros((E, H, I // 32), dtype=torch.int16))
    for key in full:
        kw = dict(full)
        kw[key] = torch.zeros(128, dtype=torch.int16)
        with pytest.raises(ValueError, match=key):
            Layer(E=E, H=H, I=I, top_k=2, max_rows=16, **kw)
    with pytest.raises(ValueError, match="on the GPU"):
        Layer(E=E, H=H, I=I, top_k=2, max_rows=16, **full)

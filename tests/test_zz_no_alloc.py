"""The allocation-free entry point (qmoe_forward_static) against the
workspace entry point (qmoe_forward), through the C ABI: the same kernels
on the library's static scratch must give the same bits, call after call,
whatever the previous call left there."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import REL_TOL, dev, dev_bf16, expert_getter, make_layer, rel_err, say, shared_of
from oracle import moe as oracle_moe

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_forward_static_matches_forward():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_mixture_experts_top_amd._binding import QMOE_ERR_WORKSPACE
    shape = synth.LayerShape(E=64, H=1024, I=512, top_k=4, shared=True)
    layer, w = make_layer(shape, 21, 4096)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # 200 tokens: 128-row tiles, routing blocks meeting at a ticket; then 9
    # tokens: dot-product GEMV items, one routing block (a smaller call on
    # what the larger one left in the scratch); then 200 again
    for M in (200, 9, 200):
        say(f"static scratch forward M={M}")
        x = synth.hidden(30 + M, M, shape.H)
        lg = synth.logits(31 + M, M, shape.E)
        xd, ld = dev_bf16(x), dev(lg)
        want = layer.forward(xd, ld).clone()
        out = torch.full_like(want, float("nan"))
        rc = layer.lib.qmoe_forward_static(layer.handle, _p(xd), _p(ld), M, _p(out), st)
        assert rc == 0, layer.lib.qmoe_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))
        assert layer.receipt()["static_scratch"] == 1
        ref = oracle_moe.forward(x, lg, shape.top_k, expert_getter(w), shape.I, shared=shared_of(w))
        err = rel_err(out.float().cpu().numpy(), ref["out"])
        say(f"  bit-equal to qmoe_forward; rel err vs oracle {err:.3e}")
        assert err <= REL_TOL
    # a call whose workspace exceeds the static array is refused, nothing enqueued
    M = 4096
    need = layer.workspace_bytes(M)
    assert need > (32 << 20)
    x = torch.zeros((M, shape.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((M, shape.E), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    rc = layer.lib.qmoe_forward_static(layer.handle, _p(x), _p(lg), M, _p(out), st)
    assert rc == QMOE_ERR_WORKSPACE
    assert "static" in layer.lib.qmoe_last_error().decode()

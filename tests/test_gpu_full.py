"""Parity at the full layer size (E=384, H=7168, I=2048, top-8, int4
group-32), in the launch configuration the benchmark times: routing for
every token bit-exact, the output checked on a seeded sample of tokens
(each output row depends only on its own token and logits)."""
import numpy as np
import pytest

import synth
from helpers import REL_TOL, check_routing, dev, dev_bf16, rel_err, say, upload_full
from oracle import moe as oracle_moe

pytestmark = pytest.mark.gpu

SEED = 0
CASES = [
    # workload, M, number of sampled tokens (None = all)
    ("decode", 1, None),
    ("decode", 9, None),
    ("transition", 90, 6),
    ("transition", 256, 6),
    ("plateau", 1024, 6),
    ("plateau", 4096, 6),
    ("skew", 512, 6),
]


@pytest.fixture(scope="module")
def full():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_mixture_experts_top_amd import Layer
    say("uploading the full layer (384 experts, seed 0)")
    w = upload_full(SEED, synth.FULL)
    r = w["routed"]
    kw = dict(E=384, H=7168, I=2048, top_k=8, max_rows=4096, w13=r["w13"], s13=r["s13"], w2=r["w2"], s2=r["s2"])
    layers = {"routed": Layer(**kw), "shared": Layer(shared=w["shared"], **kw)}
    yield layers
    for l in layers.values():
        l.close()


@pytest.mark.parametrize("workload,M,nsample", CASES)
def test_full_size_parity(full, workload, M, nsample):
    wl = synth.WORKLOADS[workload]
    shape = wl.shape
    say(f"full size {workload} M={M}")
    layer = full["shared"] if shape.shared else full["routed"]
    inp = synth.inputs(SEED, shape, M, skew=wl.skew)
    out = layer.forward(dev_bf16(inp["x"]), dev(inp["logits"])).float().cpu().numpy()
    ref_route = oracle_moe.route(inp["logits"], shape.top_k)
    check_routing(layer, M, ref_route, shape.E)
    if nsample is None:
        tokens = np.arange(M)
    else:
        rng = np.random.default_rng(1000 + M)
        tokens = np.unique(np.concatenate([[0, M - 1], rng.choice(M, nsample, replace=False)]))
    get = lambda e: synth.expert(SEED, shape, e)
    shared = synth.expert(SEED, shape, "shared") if shape.shared else None
    ref = oracle_moe.forward(inp["x"], inp["logits"], shape.top_k, get, shape.I, shared=shared, tokens=tokens)
    err = rel_err(out[tokens], ref["out"])
    say(f"  tokens {tokens.tolist()} rel err {err:.3e}")
    assert err <= REL_TOL


@pytest.fixture(scope="module")
def tp8():
    """One GPU's share under 8-way tensor parallelism over I: all 384
    experts, I = 256 (synthetic weights of that shape)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_mixture_experts_top_amd import Layer
    shape = synth.TP8_SLICE
    say("uploading the tensor-parallel slice (384 experts, I=256, seed 0)")
    r = upload_full(SEED, shape)["routed"]
    layer = Layer(E=shape.E, H=shape.H, I=shape.I, top_k=shape.top_k, max_rows=4096,
                  w13=r["w13"], s13=r["s13"], w2=r["w2"], s2=r["s2"])
    yield layer
    layer.close()


@pytest.mark.parametrize("M,nsample", [(1, None), (9, None), (256, 6), (4096, 6)])
def test_tp8_slice_parity(tp8, M, nsample):
    shape = synth.TP8_SLICE
    say(f"tp8 slice M={M}")
    inp = synth.inputs(SEED, shape, M)
    out = tp8.forward(dev_bf16(inp["x"]), dev(inp["logits"])).float().cpu().numpy()
    check_routing(tp8, M, oracle_moe.route(inp["logits"], shape.top_k), shape.E)
    if nsample is None:
        tokens = np.arange(M)
    else:
        rng = np.random.default_rng(2000 + M)
        tokens = np.unique(np.concatenate([[0, M - 1], rng.choice(M, nsample, replace=False)]))
    ref = oracle_moe.forward(inp["x"], inp["logits"], shape.top_k, lambda e: synth.expert(SEED, shape, e),
                             shape.I, tokens=tokens)
    err = rel_err(out[tokens], ref["out"])
    say(f"  tokens {tokens.tolist()} rel err {err:.3e}")
    assert err <= REL_TOL

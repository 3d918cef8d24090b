"""Shared helpers of the GPU tests: seeded inputs on the device, the oracle
on the same inputs, and the comparison rules."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import synth
from oracle import moe as oracle_moe

REL_TOL = 1e-2  # max|gpu - oracle| / max|oracle| for floating-point outputs
W_REL_TOL = 1e-5  # routing weights: fp32 exp/divide on the GPU vs float64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def make_layer(shape: synth.LayerShape, seed: int, max_rows: int, weights: dict | None = None, **layer_kw):
    from quantized_mixture_experts_top_amd import layer_from_numpy
    w = weights if weights is not None else synth.all_experts(seed, shape)
    layer = layer_from_numpy(w, E=shape.E, H=shape.H, I=shape.I, top_k=shape.top_k,
                             max_rows=max_rows, device="cuda", **layer_kw)
    return layer, w


def expert_getter(w: dict):
    return lambda e: {k: w[k][e] for k in ("w13", "s13", "w2", "s2")}


def shared_of(w: dict):
    if "shared_w13" not in w:
        return None
    return {k: w["shared_" + k] for k in ("w13", "s13", "w2", "s2")}


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if scale == 0.0:
        return float(np.max(np.abs(got))) if got.size else 0.0
    return float(np.max(np.abs(got.astype(np.float64) - ref))) / scale


def check_routing(layer, M: int, ref: dict, E: int):
    """ids, counts, offsets and perm bit-exact; weights to W_REL_TOL."""
    r = {k: v.cpu().numpy() for k, v in layer.read_routing(M).items()}
    assert np.array_equal(r["ids"], ref["ids"]), "top-k ids differ"
    assert np.array_equal(r["counts"], ref["counts"]), "expert counts differ"
    assert np.array_equal(r["offsets"], ref["offsets"]), "expert offsets differ"
    assert np.array_equal(r["perm"], ref["perm"]), "sorted routing (perm) differs"
    if M:
        werr = np.max(np.abs(r["w"].astype(np.float64) - ref["w"]) / ref["w"])
        assert werr <= W_REL_TOL, f"routing weight rel err {werr:.2e}"
    return r


def upload_full(seed: int, shape: synth.LayerShape, threads: int = 16, chunk: int = 32) -> dict:
    """Generate the full layer's weights straight into device tensors, a
    chunk of experts at a time (bounded host memory)."""
    import torch
    H, I = shape.H, shape.I
    experts = list(shape.local_experts())  # an expert-parallel shard holds its own only
    E = len(experts)
    out = {
        "w13": torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda"),
        "s13": torch.empty((E, 2 * I, H // 32), dtype=torch.int16, device="cuda"),
        "w2": torch.empty((E, H, I // 2), dtype=torch.uint8, device="cuda"),
        "s2": torch.empty((E, H, I // 32), dtype=torch.int16, device="cuda"),
    }
    with ThreadPoolExecutor(threads) as ex:
        for e0 in range(0, E, chunk):
            es = [experts[i] for i in range(e0, min(E, e0 + chunk))]
            ws = list(ex.map(lambda e: synth.expert(seed, shape, e), es))
            for key in out:
                a = np.stack([w[key] for w in ws])
                if a.dtype == np.uint16:
                    a = a.view(np.int16)
                out[key][e0:e0 + len(es)].copy_(torch.from_numpy(a))
    sh = synth.expert(seed, shape, "shared")
    shared = {k: dev(v) for k, v in sh.items()}
    torch.cuda.synchronize()
    return {"routed": out, "shared": shared}

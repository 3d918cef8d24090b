"""Plain float64 definition of the fused int4 MoE layer (the oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU library.

Sources (pages, by title and section):

* "The MoE Throughput Lever: Quantifying the INT4 Marlin GEMM on Blackwell PRO
  6000", sections "The Context: Why This Measurement Matters" and "The
  Benchmark: What Was Measured": each token goes through its top-8 of 384
  experts; weights are INT4 with group size 32 and activations 16-bit
  ("wna16"); E=384, hidden 7168, intermediate 2048.
* "Detailed results" (DeepSeek-V4.1-Flash EXL3 recipe), section "Nsight
  Compute on the stock kernel": the layer counts tokens per expert (384
  counts) and scans them.
* "perf(exl3): accelerate fat-expert prefill" (PR #77), description and
  section "Rollout": sorted routing groups the routed pairs by expert; the
  gate and up projections are one stacked GEMM over a shared input; the
  results are scattered back ("direct"/"scatter" calls).

Readings where the pages are silent (each one is listed with its reason in
the design notes):

* scoring: softmax over all experts, then the selected top-k weights are
  renormalised to sum to 1; no bias correction, no routed scaling factor;
* selection on the fp32 logits, descending, ties to the lower expert index;
  slot j of a token is its j-th selected expert in that order;
* codes: byte j of a weight row holds input index 2j (low nibble) and 2j+1
  (high nibble); value = (code - 8) * scale, one fp16 scale per 32
  consecutive inputs (the contraction axis: H for gate/up, I for down);
* gate+up stacked as [E, 2I, H]: rows 0..I-1 gate, rows I..2I-1 up;
* activation: h = SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z));
* within an expert, routed rows are ordered by ascending token index;
* combine: out[t] = sum over j = 0..k-1 of w[t,j] * y(t,j), in j order; a
  shared expert, when present, is added afterwards with weight 1.0;
* optional sigmoid scoring (the pages state top-8 routing but no scoring
  function; this is the router of the model family whose shapes the pages
  benchmark, stated as an option): scores s = 1 / (1 + e^(-l)), selection by
  s + b (a per-expert bias that steers selection only), weights = the
  selected scores renormalised and times a routed scaling factor.

Everything is computed in float64.  Integer results (ids, counts, offsets,
perm) are exact.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
ZERO_POINT = 8


# ---------------------------------------------------------------- decoding


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (a bf16 is the top
    half of an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def decode_fp16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] 4-bit codes 0..15 (low nibble = even
    input index)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequant(packed: np.ndarray, scales_bits: np.ndarray) -> np.ndarray:
    """INT4 group-32 weights -> float64 [..., N, K]:
    W[n, k] = (code[n, k] - 8) * scale[n, k // 32].

    The product is exact in float64 (a 4-bit integer times an 11-bit fp16
    significand).  Source: "The MoE Throughput Lever ...", section "The
    Benchmark: What Was Measured" (INT4, group size 32); zero-point 8 and
    fp16 scales are the configuration's format."""
    q = unpack_codes(packed).astype(np.float64) - ZERO_POINT
    s = decode_fp16(scales_bits)
    if q.shape[-1] != s.shape[-1] * GROUP:
        raise ValueError("scale groups do not match the code row length")
    return q * np.repeat(s, GROUP, axis=-1)


# ----------------------------------------------------------------- routing


def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray) -> np.ndarray:
    """The router in front of the layer: logits[t, e] = sum_k x[t, k] *
    W_r[e, k], a plain product of the bf16 hidden states [M, H] with the bf16
    router weights [E, H], in float64 (exact products of two bf16 values).
    The pages state top-8 routing over 384 experts but neither the router
    nor its scoring ("The MoE Throughput Lever ...", section "The Context:
    Why This Measurement Matters"); this is the plainest reading: a linear
    map to one logit per expert, whose scores the softmax-then-top-k routing
    below consumes."""
    return decode_bf16(x_bits) @ decode_bf16(wr_bits).T


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logit, ties to the lower
    expert index, in that order.  [M, E] -> int32 [M, k].  (Also used with
    the sigmoid scoring's float32 selection keys in place of logits.)"""
    lg = np.asarray(logits, dtype=np.float32)
    M, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("top_k out of range")
    if not np.all(np.isfinite(lg)):
        raise ValueError("router logits must be finite")
    ids = np.empty((M, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(M):
        # lexsort: last key is primary -> sort by -logit, then by index
        order = np.lexsort((idx, -lg[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


def routing_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over all experts (float64, max subtracted), then the selected
    probabilities renormalised to sum to 1.  -> float64 [M, k]."""
    lg = np.asarray(logits, dtype=np.float64)
    z = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def count_and_scan(ids: np.ndarray, E: int):
    """counts[e] = number of routed (token, slot) pairs on expert e;
    offsets = exclusive prefix sum of counts, length E+1.  Source: "Detailed
    results", section "Nsight Compute on the stock kernel" (the 384 expert
    counts and their scan)."""
    counts = np.bincount(np.asarray(ids).ravel().astype(np.int64), minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    np.cumsum(counts, out=offsets[1:])
    return counts, offsets


def sort_slots(ids: np.ndarray, E: int):
    """Sorted routing: a stable sort of the flat slots f = t*k + j by expert.
    perm[pos] = f lists each expert's pairs contiguously, tokens ascending;
    inv_perm[f] = pos.  Source: "perf(exl3): accelerate fat-expert prefill",
    section "Rollout" (sorted routing)."""
    flat = np.asarray(ids).ravel().astype(np.int64)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return perm, inv


def sigmoid_scores(logits: np.ndarray) -> np.ndarray:
    """Scores of the sigmoid router: s = 1 / (1 + e^(-l)), float64 [M, E]."""
    return 1.0 / (1.0 + np.exp(-np.asarray(logits, dtype=np.float64)))


def sigmoid_selection_keys(logits: np.ndarray, bias=None) -> np.ndarray:
    """Selection keys of the sigmoid router: s + b per expert, taken in
    float32 (the precision the selection is made in): the score rounded to
    float32, plus the bias, rounded again.  [M, E] float32."""
    s32 = sigmoid_scores(logits).astype(np.float32)
    if bias is None:
        return s32
    return (s32 + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)


def sigmoid_weights(logits: np.ndarray, ids: np.ndarray, scale: float) -> np.ndarray:
    """The selected experts' scores renormalised to sum to 1, times the
    routed scaling factor (the bias does not enter).  -> float64 [M, k]."""
    sel = np.take_along_axis(sigmoid_scores(logits), ids.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True) * float(scale)


def route(logits: np.ndarray, k: int, scoring=None) -> dict:
    """All routing outputs of one call.  scoring: None (softmax over all
    experts, selected weights renormalised) or {"kind": "sigmoid", "bias":
    float [E] or None, "scale": routed scaling factor}."""
    E = np.asarray(logits).shape[1]
    if scoring is None or scoring.get("kind", "softmax") == "softmax":
        ids = select_topk(logits, k)
        w = routing_weights(logits, ids)
    elif scoring["kind"] == "sigmoid":
        ids = select_topk(sigmoid_selection_keys(logits, scoring.get("bias")), k)
        w = sigmoid_weights(logits, ids, scoring.get("scale", 1.0))
    else:
        raise ValueError(f"unknown scoring {scoring['kind']}")
    counts, offsets = count_and_scan(ids, E)
    perm, inv = sort_slots(ids, E)
    return {"ids": ids, "w": w, "counts": counts, "offsets": offsets, "perm": perm, "inv_perm": inv}


# ------------------------------------------------------------------ expert


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_mlp(X: np.ndarray, w: dict, I: int, return_h: bool = False):
    """One expert on rows X (float64 [n, H]): the stacked gate+up product,
    h = SiLU(gate) * up, then the down product.  w holds the packed
    w13/s13/w2/s2 of the expert.  Source: "perf(exl3): accelerate fat-expert
    prefill", description (stacked gate+up GEMM over one shared input);
    "The MoE Throughput Lever ...", section "The Benchmark: What Was Measured"
    (the MoE GEMM at hidden 7168, intermediate 2048)."""
    W13 = dequant(w["w13"], w["s13"])
    gu = X @ W13.T
    del W13
    h = silu(gu[:, :I]) * gu[:, I:]
    W2 = dequant(w["w2"], w["s2"])
    y = h @ W2.T
    return (y, h) if return_h else y


# ------------------------------------------------------------------- layer


def combine(w_row: np.ndarray, y_rows, shared_row=None) -> np.ndarray:
    """One token's output: sum over its slots j = 0..k-1, in j order, of
    w[j] * y[j] (y[j] the MLP output of its j-th selected expert), then the
    shared expert's row, when there is one, with weight 1.0.  Source: "perf(exl3):
    accelerate fat-expert prefill", description (results scattered back to
    their tokens) and the routing-weighted sum of the layer."""
    acc = np.zeros(np.asarray(y_rows[0]).shape, dtype=np.float64)
    for j in range(len(w_row)):
        acc += w_row[j] * y_rows[j]
    if shared_row is not None:
        acc = acc + shared_row
    return acc


def forward(x_bits: np.ndarray, logits: np.ndarray, k: int, get_expert, I: int,
            shared=None, tokens=None, return_h: bool = False, local=None, scoring=None) -> dict:
    """The layer: out[t] = sum_j w[t,j] * MLP_{ids[t,j]}(x[t]) (+ shared
    expert), float64.

    get_expert(e) returns expert e's packed weights; `shared` is the shared
    expert's packed weights or None.  Routing is computed for all tokens;
    the output only for `tokens` (default: all), which is exact because each
    output row depends only on its own token.  With return_h, h is returned
    per routed slot of the computed tokens (dict slot -> h row) for
    debugging.

    local = (first, count): one expert-parallel shard ("The MoE Throughput
    Lever ...", section "The Architectural Implication: Refining the Engine
    Design"): routing over all experts as above, but the sum takes only the
    slots routed to experts first .. first + count - 1 (the shard's partial
    output; the shards' outputs add up to the whole layer's).

    scoring: as in route()."""
    xf = decode_bf16(x_bits)
    M, H = xf.shape
    r = route(logits, k, scoring)
    ids, w = r["ids"], r["w"]
    sel = np.arange(M) if tokens is None else np.asarray(tokens, dtype=np.int64)
    Y = {}  # (t, j) -> y row
    Hs = {}
    # group the requested pairs by expert so each expert is decoded once
    lo, hi = (0, logits.shape[1]) if local is None else (local[0], local[0] + local[1])
    mine = lambda e: lo <= e < hi
    by_e = {}
    for t in sel:
        for j in range(k):
            if mine(int(ids[t, j])):
                by_e.setdefault(int(ids[t, j]), []).append((int(t), j))
    for e in sorted(by_e):
        pairs = by_e[e]
        X = xf[[t for t, _ in pairs]]
        out = expert_mlp(X, get_expert(e), I, return_h=return_h)
        y = out[0] if return_h else out
        for n, (t, j) in enumerate(pairs):
            Y[(t, j)] = y[n]
            if return_h:
                Hs[t * k + j] = out[1][n]
    Ys = expert_mlp(xf[sel], shared, I) if shared is not None and sel.size else None
    res = np.zeros((sel.size, H), dtype=np.float64)
    for n, t in enumerate(sel):
        js = [j for j in range(k) if mine(int(ids[t, j]))]
        if js:
            res[n] = combine(w[t][js], [Y[(int(t), j)] for j in js], None if Ys is None else Ys[n])
        elif Ys is not None:
            res[n] = Ys[n]
    r.update({"out": res, "tokens": sel})
    if return_h:
        r["h"] = Hs
    return r

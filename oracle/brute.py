"""Pure-Python float64 brute force of the fused int4 MoE layer, tiny shapes.

TEST INFRASTRUCTURE ONLY.  An independent evaluation of the same definition
as ``oracle.moe``, written differently on purpose so that a slip in one
(an index, a sign, a transposed operand, a dropped term) shows up as a
disagreement:

* no numpy: lists, ``math.exp`` and Python floats (IEEE binary64);
* every weight is decoded element by element from its byte and nibble;
* the layer is evaluated densely: every expert runs on every token and its
  output is multiplied by a routing mask (0 for unselected experts), instead
  of sorting and gathering the routed pairs;
* the top-k is chosen by repeated arg-max, not by a sort.

Use only where E*M*(3*H*I) is small (a few million multiply-adds).
"""
from __future__ import annotations

import math
import struct


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _fp16(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))[0]


def _weight(packed_row, scale_row, kk: int) -> float:
    byte = int(packed_row[kk >> 1])
    code = (byte >> 4) if (kk & 1) else (byte & 15)
    return (code - 8) * _fp16(scale_row[kk // 32])


def _topk_argmax(row, k):
    """Repeated arg-max; a strict '>' keeps the first (lowest) index on ties."""
    chosen = []
    for _ in range(k):
        best = -1
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best < 0 or float(v) > float(row[best]):
                best = e
        chosen.append(best)
    return chosen


def _mlp(x, w, H, I):
    gate_up = []
    for n in range(2 * I):
        s = 0.0
        for kk in range(H):
            s += x[kk] * _weight(w["w13"][n], w["s13"][n], kk)
        gate_up.append(s)
    h = []
    for i in range(I):
        g, u = gate_up[i], gate_up[I + i]
        h.append(g / (1.0 + math.exp(-g)) * u)
    y = []
    for n in range(H):
        s = 0.0
        for i in range(I):
            s += h[i] * _weight(w["w2"][n], w["s2"][n], i)
        y.append(s)
    return y


def layer(x_bits, logits, k, experts, H, I, shared=None):
    """x_bits [M][H] bf16 patterns, logits [M][E] floats, experts[e] dicts of
    nested lists/arrays.  Returns (out [M][H], ids [M][k], w [M][k])."""
    M = len(x_bits)
    E = len(experts)
    out, all_ids, all_w = [], [], []
    for t in range(M):
        x = [_bf16(b) for b in x_bits[t]]
        row = [float(v) for v in logits[t]]
        ids = _topk_argmax(row, k)
        m = max(row)
        p = [math.exp(v - m) for v in row]
        z = sum(p)
        p = [v / z for v in p]
        zs = sum(p[e] for e in ids)
        mask = [0.0] * E
        for e in ids:
            mask[e] = p[e] / zs
        acc = [0.0] * H
        for e in range(E):  # dense: every expert, masked
            y = _mlp(x, experts[e], H, I)
            for n in range(H):
                acc[n] += mask[e] * y[n]
        if shared is not None:
            y = _mlp(x, shared, H, I)
            for n in range(H):
                acc[n] += y[n]
        out.append(acc)
        all_ids.append(ids)
        all_w.append([mask[e] for e in ids])
    return out, all_ids, all_w


def router_logits(x_bits, wr_bits):
    """Router logits by explicit loops: logits[t][e] = sum over k of
    x[t][k] * W_r[e][k], each bf16 decoded from its bit pattern, summed in
    Python floats."""
    M, H = len(x_bits), len(x_bits[0])
    out = []
    for t in range(M):
        xs = [_bf16(x_bits[t][kk]) for kk in range(H)]
        row = []
        for wr in wr_bits:
            acc = 0.0
            for kk in range(H):
                acc += xs[kk] * _bf16(wr[kk])
            row.append(acc)
        out.append(row)
    return out


def _f32(v: float) -> float:
    """Round a Python float to the nearest float32 value."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def sigmoid_route(logits, k, bias=None, scale=1.0):
    """The sigmoid router by explicit loops: per expert the score
    1 / (1 + e^(-l)) and the selection key (score + bias) rounded to float32
    as the selection is made; the k largest keys by repeated arg-max (ties to
    the lower index); the selected scores renormalised times the scale.
    Returns (ids, weights) as lists."""
    all_ids, all_w = [], []
    for row in logits:
        scores = [1.0 / (1.0 + math.exp(-float(l))) for l in row]
        keys = [_f32(_f32(s) + (_f32(float(bias[e])) if bias is not None else 0.0)) for e, s in enumerate(scores)]
        ids = _topk_argmax(keys, k)
        tot = 0.0
        for e in ids:
            tot += scores[e]
        all_ids.append(ids)
        all_w.append([scores[e] / tot * scale for e in ids])
    return all_ids, all_w

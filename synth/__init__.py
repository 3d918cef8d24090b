"""Seeded synthetic inputs for the fused int4 Mixture-of-Experts layer.

This module is the only code shared by the CPU oracle and the GPU path.  It
draws random numbers and encodes them into the layer's input formats (bf16
hidden states, fp32 router logits, packed int4 codes, fp16 group scales); it
holds none of the layer's arithmetic.

Shapes follow the layer measured in "The MoE Throughput Lever: Quantifying the
INT4 Marlin GEMM on Blackwell PRO 6000", section "The Benchmark: What Was
Measured": 384 experts, hidden 7168, intermediate 2048, top-8, INT4 weights
with group size 32.  Value distributions (N(0,1) activations and logits,
uniform codes 0..15 around zero-point 8, scales uniform in [0.002, 0.02]) are
this repository's synthetic recipe; the pages print no weights.

Every tensor comes from its own PCG64 stream keyed by
SeedSequence([seed, tag, index]) so that one expert can be regenerated alone:

  tag 0  hidden states x            tag 1  router logits
  tag 2  gate+up codes  (per expert) tag 3  gate+up scales (per expert)
  tag 4  down codes     (per expert) tag 5  down scales    (per expert)
  tag 6..9  the shared expert's gate+up codes, scales, down codes, scales
  tag 10  router weights (bf16 [E, H])

Packed code bytes are the little-endian bytes of PCG64's raw 64-bit outputs;
each byte is uniform on 0..255, so both of its nibbles are uniform on 0..15.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GROUP = 32
ZIPF_S = 1.2

TAG_X, TAG_LOGITS = 0, 1
TAG_W13, TAG_S13, TAG_W2, TAG_S2 = 2, 3, 4, 5
TAG_SHARED_W13, TAG_SHARED_S13, TAG_SHARED_W2, TAG_SHARED_S2 = 6, 7, 8, 9
TAG_ROUTER = 10

SCALE_LO, SCALE_HI = 0.002, 0.02


@dataclasses.dataclass(frozen=True)
class LayerShape:
    E: int
    H: int
    I: int
    top_k: int
    shared: bool = False
    # expert-parallel shard: local experts [local_first, local_first + local_count)
    # of the E routed over (0 = all E)
    local_first: int = 0
    local_count: int = 0

    def local_experts(self) -> range:
        return range(self.local_first, self.local_first + (self.local_count or self.E))

    def expert_bytes(self) -> int:
        """Packed code bytes plus fp16 scale bytes of one expert."""
        codes = 2 * self.I * self.H // 2 + self.H * self.I // 2
        scales = 2 * (2 * self.I * self.H // GROUP + self.H * self.I // GROUP)
        return codes + scales


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    Ms: tuple
    skew: bool = False


TINY = LayerShape(E=8, H=256, I=128, top_k=2)
FULL = LayerShape(E=384, H=7168, I=2048, top_k=8)
FULL_SHARED = LayerShape(E=384, H=7168, I=2048, top_k=8, shared=True)
# one GPU's share of the same layer under 8-way tensor parallelism over I:
# every expert, an eighth of its intermediate width
TP8_SLICE = LayerShape(E=384, H=7168, I=256, top_k=8)
# one GPU's share under 8-way expert parallelism: routes over all 384
# experts, holds and computes experts 0..47
EP48_SLICE = LayerShape(E=384, H=7168, I=2048, top_k=8, local_first=0, local_count=48)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, (16,)),
    "decode": Workload("decode", FULL, (1, 9)),
    "transition": Workload("transition", FULL, (90, 256)),
    "plateau": Workload("plateau", FULL, (1024, 4096)),
    "skew": Workload("skew", FULL_SHARED, (512,), skew=True),
    "tp8": Workload("tp8", TP8_SLICE, (1, 9, 256, 4096)),
    "ep48": Workload("ep48", EP48_SLICE, (1, 9, 256, 4096)),
}


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


def _raw_bytes(seed: int, tag: int, index: int, n: int) -> np.ndarray:
    bg = np.random.PCG64(np.random.SeedSequence([seed, tag, index]))
    words = bg.random_raw((n + 7) // 8)
    return words.astype("<u8", copy=False).view(np.uint8)[:n].copy()


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs must be finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def hidden(seed: int, M: int, H: int) -> np.ndarray:
    """x: N(0,1) float32 rounded to bf16; uint16 bit patterns [M, H]."""
    return f32_to_bf16_bits(_rng(seed, TAG_X).standard_normal((M, H), dtype=np.float32))


def zipf_bias(E: int) -> np.ndarray:
    """log of an unnormalised Zipf(s=1.2) popularity over experts ranked
    0..E-1 (expert 0 most popular): -s*ln(e+1), as float32."""
    return (-ZIPF_S * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def logits(seed: int, M: int, E: int, skew: bool = False) -> np.ndarray:
    """Router logits: N(0,1) float32 [M, E]; the skewed workload adds the Zipf
    log-bias per expert (in float32)."""
    z = _rng(seed, TAG_LOGITS).standard_normal((M, E), dtype=np.float32)
    if skew:
        z = z + zipf_bias(E)[None, :]
    return z


def router_weights(seed: int, E: int, H: int) -> np.ndarray:
    """Router weights W_r: N(0, 1/H) float32 rounded to bf16, [E, H] (so that
    the logits of N(0,1) hidden states are about N(0,1)); uint16 patterns."""
    w = _rng(seed, TAG_ROUTER).standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    return f32_to_bf16_bits(w)


def _scales(seed: int, tag: int, index: int, rows: int, groups: int) -> np.ndarray:
    s = _rng(seed, tag, index).uniform(SCALE_LO, SCALE_HI, size=(rows, groups))
    return s.astype(np.float32).astype(np.float16).view(np.uint16)


def expert(seed: int, shape: LayerShape, e) -> dict:
    """One expert's packed weights.  e is an expert index or the string
    "shared" for the always-selected shared expert.

    w13 uint8 [2I, H/2], s13 uint16 (fp16 bits) [2I, H/32]: rows 0..I-1 gate,
    rows I..2I-1 up.  w2 uint8 [H, I/2], s2 uint16 [H, I/32].  Byte j of a row
    holds the code of input index 2j in its low nibble and 2j+1 in its high
    nibble."""
    H, I = shape.H, shape.I
    if e == "shared":
        tags, idx = (TAG_SHARED_W13, TAG_SHARED_S13, TAG_SHARED_W2, TAG_SHARED_S2), 0
    else:
        tags, idx = (TAG_W13, TAG_S13, TAG_W2, TAG_S2), int(e)
    w13 = _raw_bytes(seed, tags[0], idx, 2 * I * H // 2).reshape(2 * I, H // 2)
    s13 = _scales(seed, tags[1], idx, 2 * I, H // GROUP)
    w2 = _raw_bytes(seed, tags[2], idx, H * I // 2).reshape(H, I // 2)
    s2 = _scales(seed, tags[3], idx, H, I // GROUP)
    return {"w13": w13, "s13": s13, "w2": w2, "s2": s2}


def all_experts(seed: int, shape: LayerShape, threads: int = 8, out: dict | None = None) -> dict:
    """Stacked weights of all experts: w13 [E,2I,H/2], s13 [E,2I,H/32],
    w2 [E,H,I/2], s2 [E,H,I/32] (numpy; or written into the arrays of `out`).
    Shared-expert weights, when the shape has one, are under shared_*."""
    E, H, I = shape.E, shape.H, shape.I
    if out is None:
        out = {
            "w13": np.empty((E, 2 * I, H // 2), np.uint8),
            "s13": np.empty((E, 2 * I, H // GROUP), np.uint16),
            "w2": np.empty((E, H, I // 2), np.uint8),
            "s2": np.empty((E, H, I // GROUP), np.uint16),
        }

    def fill(e):
        w = expert(seed, shape, e)
        for key in ("w13", "s13", "w2", "s2"):
            out[key][e] = w[key]

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(E)))
    if shape.shared:
        w = expert(seed, shape, "shared")
        for key in ("w13", "s13", "w2", "s2"):
            out["shared_" + key] = w[key]
    return out


def expected_touched(E: int, k: int, M: int) -> float:
    """Expected number of distinct experts hit by M tokens that each pick k of
    E experts uniformly without replacement."""
    return E * (1.0 - (1.0 - k / E) ** M)


def inputs(seed: int, shape: LayerShape, M: int, skew: bool = False, logits_seed: int | None = None) -> dict:
    """Activations and logits of one call (weights are separate: expert())."""
    ls = seed if logits_seed is None else logits_seed
    return {"x": hidden(ls, M, shape.H), "logits": logits(ls, M, shape.E, skew)}


__all__ = [
    "GROUP", "LayerShape", "Workload", "WORKLOADS", "TINY", "FULL", "FULL_SHARED", "TP8_SLICE", "EP48_SLICE",
    "f32_to_bf16_bits", "hidden", "logits", "zipf_bias", "expert", "all_experts",
    "inputs", "expected_touched", "router_weights",
]

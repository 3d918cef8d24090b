"""GPU parity of each step of the HIP path against the CPU oracle at sizes
the oracle finishes in seconds: dequant (bit-exact), routing (bit-exact),
gate+up (h), down (weighted y) and the whole layer, on shapes that cover
both tile shapes, several K-steps, ragged tails, the shared expert and the
degenerate cases."""
import numpy as np
import pytest

import synth
from helpers import (REL_TOL, check_routing, dev, dev_bf16, expert_getter, make_layer, rel_err, say,
                     shared_of)
from oracle import moe as oracle_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------- dequant


def _crafted_expert(H, I, seed):
    """Every code 0..15 in every position class, scales over a wide sweep
    (the synthetic range's ends, random normal fp16 values, subnormals)."""
    rng = np.random.default_rng(seed)
    codes13 = (np.arange(2 * I * H) % 16).reshape(2 * I, H).astype(np.uint8)
    rng.shuffle(codes13, axis=1)
    codes2 = rng.integers(0, 16, size=(H, I), dtype=np.uint8)
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)

    def scales(shape):
        s = rng.uniform(2.0 ** -10, 16.0, size=shape).astype(np.float16).view(np.uint16)
        flat = s.reshape(-1)
        specials = np.array([np.float16(0.002).view(np.uint16), np.float16(0.02).view(np.uint16),
                             0x0001, 0x0200, 0x03FF, 0x0400, 0x3C00, 0x7BFF >> 2], dtype=np.uint16)
        flat[:specials.size] = specials
        return s
    return {"w13": pack(codes13), "s13": scales((2 * I, H // 32)), "w2": pack(codes2), "s2": scales((H, I // 32))}


def test_dequant_bit_exact_against_rne_of_exact_product():
    H, I, E = 256, 128, 2
    ex = [_crafted_expert(H, I, 100 + e) for e in range(E)]
    w = {k: np.stack([x[k] for x in ex]) for k in ex[0]}
    layer, _ = make_layer(synth.LayerShape(E=E, H=H, I=I, top_k=1), 0, 4, weights=w)
    for e in range(E):
        for which, (wk, sk) in enumerate((("w13", "s13"), ("w2", "s2"))):
            say(f"dequant expert={e} which={which}")
            got = layer.dequant_debug(e, which).cpu().numpy().view(np.uint16)
            exact = oracle_moe.dequant(w[wk][e], w[sk][e])  # float64, exact
            want = exact.astype(np.float16).view(np.uint16)  # one rounding to nearest even
            assert np.array_equal(got, want), f"expert {e} which {which}"


# ---------------------------------------------------------------- routing

ROUTE_CASES = [
    # E, k, M, logits kind
    (8, 2, 16, "normal"),
    (384, 8, 1, "normal"),
    (384, 8, 9, "normal"),
    (384, 8, 90, "normal"),
    (384, 8, 256, "normal"),
    (384, 8, 1024, "normal"),
    (384, 8, 4096, "normal"),
    (384, 8, 512, "zipf"),
    (64, 4, 300, "ties"),
    (1000, 32, 70, "normal"),
    (64, 1, 65, "normal"),
    (1, 1, 5, "normal"),
    (16, 16, 130, "normal"),
    (33, 3, 64, "zeros"),
]


def _logits(kind, seed, M, E):
    if kind == "zipf":
        return synth.logits(seed, M, E, skew=True)
    lg = synth.logits(seed, M, E)
    if kind == "ties":
        lg = (np.round(lg * 2.0) / 2.0).astype(np.float32)  # few distinct values: many ties
    if kind == "zeros":
        lg = np.where(np.abs(lg) < 0.7, np.float32(0.0), lg).astype(np.float32)
        lg[:, ::2] = np.where(lg[:, ::2] == 0, np.float32(-0.0), lg[:, ::2])  # +0 and -0 tie
    return lg


@pytest.mark.parametrize("E,k,M,kind", ROUTE_CASES)
def test_routing_bit_exact(E, k, M, kind):
    say(f"route E={E} k={k} M={M} {kind}")
    shape = synth.LayerShape(E=E, H=128, I=128, top_k=k)
    layer, _ = make_layer(shape, 1, M)
    x = synth.hidden(2, M, 128)
    lg = _logits(kind, 3, M, E)
    layer.route(dev_bf16(x), dev(lg))
    ref = oracle_moe.route(lg, k)
    check_routing(layer, M, ref, E)


def test_routing_repeatable_and_workspace_reuse():
    E, k = 384, 8
    shape = synth.LayerShape(E=E, H=128, I=128, top_k=k)
    layer, _ = make_layer(shape, 1, 4096)
    for M in (4096, 7, 1000, 7):  # shrinking and growing M on one workspace
        say(f"route reuse M={M}")
        lg = synth.logits(M, M, E)
        layer.route(dev_bf16(synth.hidden(M, M, 128)), dev(lg))
        check_routing(layer, M, oracle_moe.route(lg, k), E)


# ------------------------------------------------------------ whole layer

FWD_CASES = [
    # E, H, I, k, M, shared   (dot-product GEMV items of <= 2 rows when
    #                          4*M*k <= 7E, else 128-row MFMA tiles; the
    #                          GEMV reads codes non-temporal when M*k <= E
    #                          and there is no shared expert: the cases
    #                          with M=1 on 8 experts, M=20 on 64, M=2 on 16
    #                          and M=1 on 1, and the default cache policy in
    #                          the other GEMV cases)
    (8, 256, 128, 2, 16, False),     # the tiny configuration (tiles)
    (8, 256, 128, 2, 7, False),      # GEMV, several items per expert
    (8, 256, 128, 2, 1, False),      # GEMV, one row
    (16, 640, 384, 2, 37, False),    # tiles: K = 1 super-step + a partial one / a partial one
    (64, 128, 128, 2, 9, True),      # GEMV with a shared expert
    (4, 640, 384, 2, 300, False),    # tiles: 2 row tiles per expert, partial super-steps
    (4, 256, 128, 1, 200, True),     # tiles with a shared expert
    (4, 512, 256, 4, 20, False),     # top_k = E
    (8, 2048, 1536, 2, 64, False),   # tiles: several super-steps per wave in both GEMMs
    (3, 384, 1152, 2, 130, False),   # tiles: N not a multiple of the block width
    (64, 1152, 640, 2, 20, False),   # GEMV: whole + partial super-steps in both GEMMs
    (32, 2048, 1536, 4, 8, True),    # GEMV: 2-row items, shared expert
    (16, 256, 128, 8, 2, False),     # GEMV: top_k = 8, partial super-steps only
    (8, 512, 256, 2, 7, True),       # GEMV: experts with several items, shared expert
    (8, 256, 128, 2, 40, False),     # tiles on the tiny shape (2 row blocks)
    (16, 640, 384, 2, 72, True),     # tiles with a shared expert, partial super-steps
    (1, 256, 128, 1, 1, False),      # one expert, GEMV (a plain quantized SwiGLU MLP)
    (1, 256, 128, 1, 5, False),      # one expert, tiles
    (32, 256, 128, 32, 3, False),    # top_k = 32 = E (the largest top_k)
    (1024, 128, 128, 8, 20, True),   # 1024 experts (the most), shared expert
    (4, 13056, 128, 2, 3, False),    # the largest K the GEMV stages in LDS
    (4, 13184, 128, 1, 2, False),    # K past the GEMV's LDS: small M on tiles
    (16, 256, 1664, 2, 64, False),   # tiles: down items of <= 32 rows, 3 whole super-steps + a partial one
    (16, 256, 1024, 2, 64, True),    # tiles: down items of <= 32 rows, 2 whole super-steps; shared expert
    (4, 256, 128, 1, 300, False),    # tiles: items of 4, 5 and 6 row blocks
    (4, 256, 128, 1, 400, False),    # tiles: items of 6 and 7 row blocks
    # tiles with K >= 1536 in both products (3 whole super-steps: the
    # pipelined K loops) and 65-128 routed rows per expert (items of 5-8 row
    # blocks), every token compared; the shared expert adds items of 8 blocks
    (4, 1536, 1536, 1, 300, False),
    (4, 1536, 1536, 1, 300, True),
    (4, 1536, 1536, 1, 360, False),
    (4, 1536, 1536, 1, 360, True),
    (4, 1536, 1536, 1, 400, False),
    (4, 1536, 1536, 1, 400, True),
    (4, 1536, 1536, 1, 500, False),
    (4, 1536, 1536, 1, 500, True),
    # mixed calls (tiles, at most 4 rows per expert on average): experts of
    # 1-2 rows on the dot-product GEMV, the rest (and the shared expert) on
    # tiles, every token compared
    (64, 1024, 512, 4, 40, False),
    (64, 1024, 512, 4, 40, True),
    (32, 2048, 1536, 4, 30, True),   # 4 whole super-steps in gate+up, 3 in down
]


def _run_case(E, H, I, k, M, shared, seed=5):
    shape = synth.LayerShape(E=E, H=H, I=I, top_k=k, shared=shared)
    layer, w = make_layer(shape, seed, max(M, 1))
    x = synth.hidden(seed + 1, M, H)
    lg = synth.logits(seed + 2, M, E)
    ref = oracle_moe.forward(x, lg, k, expert_getter(w), I, shared=shared_of(w), return_h=True)
    return layer, w, x, lg, ref


def _item_blocks(counts, shared_rows):
    """Row blocks of 16 of each 128-row MFMA work item (the K loop each
    item runs through), over the routed experts and the shared expert."""
    blocks = []
    for c in list(counts) + ([shared_rows] if shared_rows else []):
        for r0 in range(0, int(c), 128):
            blocks.append((min(128, int(c) - r0) + 15) // 16)
    return sorted(set(blocks))


@pytest.mark.parametrize("E,H,I,k,M,shared", FWD_CASES)
def test_forward_parity(E, H, I, k, M, shared):
    say(f"forward E={E} H={H} I={I} k={k} M={M} shared={shared}")
    layer, w, x, lg, ref = _run_case(E, H, I, k, M, shared)
    out = layer.forward(dev_bf16(x), dev(lg)).float().cpu().numpy()
    check_routing(layer, M, ref, E)
    err = rel_err(out, ref["out"])
    tiles = layer.stats()["prefill_tiles"] > 0
    where = (f"tiles, items of {_item_blocks(ref['counts'], M if shared else 0)} row blocks" if tiles
             else "dot-product GEMV")
    say(f"  all {M} tokens; {where}; rel err out {err:.3e}")
    assert err <= REL_TOL


@pytest.mark.parametrize("E,H,I,k,M,shared", [FWD_CASES[3], FWD_CASES[5], FWD_CASES[6], FWD_CASES[10],
                                               FWD_CASES[11], FWD_CASES[13], FWD_CASES[15]])
def test_steps_match_oracle_intermediates(E, H, I, k, M, shared):
    """h = SiLU(gate)*up after the gate+up step and w*y after the down step,
    per routed slot, against the oracle's float64 values."""
    say(f"steps E={E} H={H} I={I} k={k} M={M} shared={shared}")
    layer, w, x, lg, ref = _run_case(E, H, I, k, M, shared)
    layer.route(dev_bf16(x), dev(lg))
    layer.gate_up(M)
    h = layer.read_intermediate(M, 0).cpu().numpy()
    T = M * k
    ref_h = np.stack([ref["h"][f] for f in range(T)])
    assert rel_err(h[:T], ref_h) <= REL_TOL
    layer.down(M)
    y = layer.read_intermediate(M, 1).cpu().numpy()
    xf = oracle_moe.decode_bf16(x)
    get = expert_getter(w)
    ref_y = np.zeros((T, H))
    for t in range(M):
        for j in range(k):
            e = int(ref["ids"][t, j])
            ref_y[t * k + j] = ref["w"][t, j] * oracle_moe.expert_mlp(xf[t:t + 1], get(e), I)[0]
    assert rel_err(y[:T], ref_y) <= REL_TOL
    if shared:
        ref_s = oracle_moe.expert_mlp(xf, shared_of(w), I)
        assert rel_err(y[T:], ref_s) <= REL_TOL
    out = layer.combine(M).float().cpu().numpy()
    assert rel_err(out, ref["out"]) <= REL_TOL


@pytest.mark.parametrize("M", [20, 2])  # 128-row tiles, dot-product items
def test_diagonal_weights_closed_form_on_gpu(M):
    """Top-1 with diagonal weights and power-of-two scales: the output is
    sd*su*x*SiLU(sg*x) on the first min(H, I) columns and 0 elsewhere."""
    import math
    H, I, E = 256, 128, 3
    codes13 = np.full((2 * I, H), 8, np.uint8)
    for i in range(I):
        codes13[i, i] = 9
        codes13[I + i, i] = 9
    codes2 = np.full((H, I), 8, np.uint8)
    for n in range(I):
        codes2[n, n] = 9
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    s13 = np.empty((2 * I, H // 32), np.uint16)
    s13[:I], s13[I:] = 0x3800, 0x4000  # 0.5, 2.0
    s2 = np.full((H, I // 32), 0x3400, np.uint16)  # 0.25
    one = {"w13": pack(codes13), "s13": s13, "w2": pack(codes2), "s2": s2}
    w = {k: np.stack([one[k]] * E) for k in one}
    layer, _ = make_layer(synth.LayerShape(E=E, H=H, I=I, top_k=1), 0, M, weights=w)
    x = synth.hidden(9, M, H)
    out = layer.forward(dev_bf16(x), dev(synth.logits(9, M, E))).float().cpu().numpy()
    xf = oracle_moe.decode_bf16(x)
    expect = np.zeros((M, H))
    for t in range(M):
        for n in range(I):
            v = xf[t, n]
            g = 0.5 * v
            expect[t, n] = 0.25 * (2.0 * v) * (g / (1.0 + math.exp(-g)))
    if M > 2:
        # MFMA tiles: a code-8 weight decodes to exactly zero
        assert np.all(out[:, I:] == 0.0)
    else:
        # dot-product GEMV: the zero point is taken back as 8 * sum(x) per
        # group, so all-8 rows leave only fp32 cancellation, far inside the bar
        assert np.max(np.abs(out[:, I:])) <= 2.0 ** -10 * np.max(np.abs(expect))
    assert rel_err(out, expect) <= REL_TOL


@pytest.mark.parametrize("case", [(16, 640, 384, 2, 37, False), (32, 2048, 1536, 4, 8, True)])
def test_repeat_runs_bitwise_identical(case):
    layer, w, x, lg, ref = _run_case(*case)
    xs, ls = dev_bf16(x), dev(lg)
    import torch
    a = layer.forward(xs, ls).clone()
    b = layer.forward(xs, ls).clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("E,H,I,k,M,m,path", [
    # GEMV both times: 30 tokens alone read the codes non-temporal, 40 do
    # not; neither call splits K (a split call adds its K shares in another
    # order, so its bits may differ from an unsplit one)
    (64, 1152, 640, 2, 40, 30, "gemv_tiles"),
    # tiles both times: 60 tokens alone take the 2-row-block K loops (paired
    # weight loads), all 400 the 6- and 7-block loops
    (4, 256, 128, 1, 400, 60, "prefill_tiles"),
])
def test_token_results_do_not_depend_on_the_call(E, H, I, k, M, m, path):
    """A token's output is a function of its own row and logits only: each
    routed row's sums run in the same order whatever items it shares, so the
    first m tokens alone give the same bits as inside the M-token call."""
    import torch
    layer, w = make_layer(synth.LayerShape(E=E, H=H, I=I, top_k=k), 5, M)
    xs, ls = dev_bf16(synth.hidden(6, M, H)), dev(synth.logits(7, M, E))
    say(f"call invariance E={E} M={M} first {m} ({path})")
    full = layer.forward(xs, ls).clone()
    part = layer.forward(xs[:m].contiguous(), ls[:m].contiguous()).clone()
    s = layer.stats()
    assert s[path] == 2  # both calls took the regime named
    # the GEMV's m tokens alone read the codes non-temporal (gate+up and
    # down), all M with the default policy; the tiles never do
    assert s["gemv_nt_launches"] == (2 if path == "gemv_tiles" else 0)
    assert s["splitk_launches"] == 0
    assert torch.equal(full[:m].view(torch.int16), part.view(torch.int16))


@pytest.mark.parametrize("M", [9, 130])  # one routing block; three meeting at a ticket
def test_uninitialised_workspace(M):
    """A workspace full of stale bytes, never initialised, gives the same
    output as the layer's own (initialised) workspace: calls depend on no
    workspace state from before."""
    import ctypes
    import torch
    shape = synth.LayerShape(E=64, H=256, I=128, top_k=4)
    layer, _ = make_layer(shape, 3, M)
    x, lg = dev_bf16(synth.hidden(4, M, shape.H)), dev(synth.logits(4, M, shape.E))
    want = layer.forward(x, lg).clone()
    ws = torch.full((layer.workspace_bytes(M),), 0xA5, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(want)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = layer.lib.qmoe_forward(layer.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(lg.data_ptr()), M,
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(), st)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


# GEMV items, one routing block; a mixed call (2.5 rows per expert: tiles and
# the dot-product GEMV over the experts of 1-2 rows); tiles, three routing
# blocks meeting at a ticket
@pytest.mark.parametrize("M", [9, 40, 130])
def test_graph_capture_replays_match_eager(M):
    """The whole forward captured into a HIP graph (fixed M; workspace,
    inputs and output allocated before the capture) replays to the eager
    result, bit for bit, four times, with eager calls on other inputs
    through the same workspace and synchronisations between the replays."""
    import torch
    shape = synth.LayerShape(E=64, H=256, I=128, top_k=4)
    layer, _ = make_layer(shape, 3, M)
    x, lg = dev_bf16(synth.hidden(4, M, shape.H)), dev(synth.logits(4, M, shape.E))
    x2, lg2 = dev_bf16(synth.hidden(5, M, shape.H)), dev(synth.logits(5, M, shape.E))
    want = layer.forward(x, lg).clone()
    want2 = layer.forward(x2, lg2).clone()
    assert not torch.equal(want.view(torch.int16), want2.view(torch.int16))
    # the eager result the replays must match is itself checked against the oracle
    xn, ln = synth.hidden(4, M, shape.H), synth.logits(4, M, shape.E)
    w = synth.all_experts(3, shape)
    ref = oracle_moe.forward(xn, ln, shape.top_k, expert_getter(w), shape.I)
    err = rel_err(want.float().cpu().numpy(), ref["out"])
    say(f"graph M={M}: eager vs oracle rel err {err:.3e}")
    assert err <= REL_TOL
    out = torch.empty_like(want)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, lg, out=out)
    for rep in range(4):
        say(f"graph M={M} replay {rep}")
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
        got2 = layer.forward(x2, lg2)  # eager work in between, same workspace
        torch.cuda.synchronize()
        assert torch.equal(got2.view(torch.int16), want2.view(torch.int16))


def _heavy_tailed(seed, M, H, frac=0.01, lo=100.0, hi=2000.0):
    """N(0,1) hidden states with a fraction of entries replaced by
    +-U(lo, hi) outliers, rounded to bf16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, H)).astype(np.float32)
    mask = rng.random((M, H)) < frac
    x[mask] = (rng.uniform(lo, hi, int(mask.sum())) * rng.choice([-1.0, 1.0], int(mask.sum()))).astype(np.float32)
    return synth.f32_to_bf16_bits(x)


def _per_token_rel_err(got, ref):
    scale = np.max(np.abs(ref), axis=1)
    scale = np.where(scale > 0, scale, 1.0)
    return float(np.max(np.max(np.abs(got.astype(np.float64) - ref), axis=1) / scale))


# (E, H, I, k, M, shared): dot-product GEMV items and 128-row tiles
RANGE_CASES = [(16, 1024, 512, 2, 4, False), (16, 1024, 512, 2, 96, True)]


@pytest.mark.parametrize("case", RANGE_CASES)
@pytest.mark.parametrize("kind", ["outliers", "x1e3", "x1e-4", "mixed"])
def test_activation_range(case, kind):
    """Hidden states outside N(0,1): 1% outliers of 100..2000 (the gate and
    up products then reach ~1e6, past fp16), the whole input scaled by 1e3 or
    1e-4, and rows of very different magnitudes in one call.  Each token's
    row is scaled by its own power of two on the GPU, so every token must
    match the oracle relative to its own largest output."""
    E, H, I, k, M, shared = case
    shape = synth.LayerShape(E=E, H=H, I=I, top_k=k, shared=shared)
    layer, w = make_layer(shape, 11, M)
    if kind == "outliers":
        x = _heavy_tailed(12, M, H)
    else:
        xf = oracle_moe.decode_bf16(synth.hidden(12, M, H))
        if kind == "x1e3":
            xf = xf * 1e3
        elif kind == "x1e-4":
            xf = xf * 1e-4
        else:  # token t scaled by 10^(t mod 9 - 4)
            xf = xf * (10.0 ** (np.arange(M) % 9 - 4))[:, None]
        x = synth.f32_to_bf16_bits(xf.astype(np.float32))
    lg = synth.logits(13, M, E)
    ref = oracle_moe.forward(x, lg, k, expert_getter(w), I, shared=shared_of(w))
    out = layer.forward(dev_bf16(x), dev(lg)).float().cpu().numpy()
    check_routing(layer, M, ref, E)
    assert np.all(np.isfinite(out))
    err, tok_err = rel_err(out, ref["out"]), _per_token_rel_err(out, ref["out"])
    say(f"range {kind} case {case}: max|oracle| {np.max(np.abs(ref['out'])):.3e}, rel err {err:.3e}, "
        f"worst per-token rel err {tok_err:.3e}")
    assert err <= REL_TOL and tok_err <= REL_TOL


def test_side_stream():
    """The layer enqueues only on the stream it is given."""
    import torch
    layer, w, x, lg, ref = _run_case(32, 2048, 1536, 4, 8, True)
    xs, ls = dev_bf16(x), dev(lg)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = layer.forward(xs, ls, stream=side)
    side.synchronize()
    assert rel_err(out.float().cpu().numpy(), ref["out"]) <= REL_TOL


def test_zero_tokens_is_a_noop():
    import torch
    shape = synth.TINY
    layer, _ = make_layer(shape, 0, 4)
    x = torch.empty((0, shape.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, shape.E), dtype=torch.float32, device="cuda")
    out = layer.forward(x, lg)
    assert out.shape == (0, shape.H)


def test_counters_and_workspace_accounting():
    shape = synth.TINY
    layer, _ = make_layer(shape, 0, 16)
    x, lg = dev_bf16(synth.hidden(0, 16, shape.H)), dev(synth.logits(0, 16, shape.E))
    layer.forward(x, lg)  # workspace allocated and initialised here
    layer.reset_stats()
    layer.forward(x, lg)
    s = layer.stats()
    # 16 tokens x top-2 over 8 experts: tiles, 4 rows per expert on average,
    # so a mixed call (each product also runs the dot-product GEMV)
    assert layer.receipt()["regime"] == "mixed"
    assert s["forward_calls"] == 1 and s["route_calls"] == 1
    assert s["gemm_launches"] == 4 and s["launches"] == 6
    assert s["workspace_inits"] == 0
    assert s["workspace_bytes_last"] == s["workspace_bytes_peak"] == layer.workspace_bytes(16) > 0
    assert s["prefill_tiles"] == 1 and s["gemv_tiles"] == 1
    assert s["gemv_nt_launches"] == 0  # 16 tokens x top-2 > 8 experts


def test_errors_from_the_library():
    import torch
    from quantized_mixture_experts_top_amd import QmoeError
    from quantized_mixture_experts_top_amd._binding import QMOE_ERR_ARG, QMOE_ERR_WORKSPACE, check
    import ctypes
    shape = synth.TINY
    layer, _ = make_layer(shape, 0, 8)
    x, lg = dev_bf16(synth.hidden(0, 9, shape.H)), dev(synth.logits(0, 9, shape.E))
    with pytest.raises(QmoeError) as ei:
        layer.forward(x, lg)  # M = 9 > max_rows = 8
    assert ei.value.code == QMOE_ERR_ARG and "max_rows" in ei.value.message
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    out = torch.empty((8, shape.H), dtype=torch.bfloat16, device="cuda")
    rc = layer.lib.qmoe_forward(layer.handle, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(lg.data_ptr()), 8,
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(small.data_ptr()), 1024,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == QMOE_ERR_WORKSPACE
    assert "needs" in layer.lib.qmoe_last_error().decode()
    with pytest.raises(QmoeError):
        check(layer.lib.qmoe_dequant_debug(layer.handle, shape.E, 0, None, None))


@pytest.mark.parametrize("E,H,I,k,M,shared", [
    (64, 1024, 512, 4, 9, False),    # GEMV, codes non-temporal (M*k <= E, no shared expert)
    (64, 1024, 512, 4, 20, True),    # GEMV with a shared expert (default cache policy)
    (64, 1024, 512, 4, 130, True),   # tiles; routing in two kernels (more than 64 tokens)
    (8, 256, 128, 2, 16, False),     # mixed (4 rows per expert); one routing kernel
    (64, 1024, 512, 4, 40, True),    # mixed with a shared expert (always on tiles)
])
def test_receipt_exact_counts(E, H, I, k, M, shared):
    """The per-call receipt names the regime, cache policy, launches, grid
    sizes and workspace bytes the call used, and the device's work-item count
    equals the count the oracle's routing implies exactly."""
    import math
    shape = synth.LayerShape(E=E, H=H, I=I, top_k=k, shared=shared)
    layer, w = make_layer(shape, 41, M)
    x, lg = synth.hidden(42, M, H), synth.logits(43, M, E)
    layer.forward(dev_bf16(x), dev(lg))
    layer.forward(dev_bf16(x), dev(lg))
    r = layer.receipt()
    counts = oracle_moe.route(lg, k)["counts"]
    gemv = 4 * M * k <= 7 * E
    mixed = not gemv and M * k <= 4 * E  # experts of 1-2 rows then leave the tile list
    rpi = 2 if gemv else 128
    items = sum(math.ceil(int(c) / rpi) for c in counts if not (mixed and 1 <= c <= 2)) + \
        (math.ceil(M / rpi) if shared else 0)
    T = M * k
    max_items = T // rpi + min(E, T) + (math.ceil(M / rpi) if shared else 0)
    say(f"receipt E={E} M={M} shared={shared}: {r}; device items {layer.item_count(M)} (expected {items})")
    assert layer.item_count(M) == items
    assert r["seq"] == 2 and r["M"] == M
    assert r["regime"] == ("gemv" if gemv else "mixed" if mixed else "tiles") and r["rows_per_item"] == rpi
    assert r["nt_codes"] == int(gemv and T <= E and not shared)
    assert r["shared_expert"] == int(shared) and r["static_scratch"] == 0
    assert r["route_kernels"] == (1 if M <= 64 else 2)
    assert r["launches"] == 3 + r["route_kernels"] + (2 if mixed else 0)
    assert r["max_items"] == max_items >= items
    if gemv:
        # a launch of fewer than 128 blocks splits K (about 512 blocks in all,
        # up to one split per 512 inputs)
        def splits(tiles, K):
            return 1 if tiles >= 128 or K // 512 < 2 else min(K // 512, math.ceil(512 / tiles))
        sg, sd = splits(max_items * math.ceil(I / 64), H), splits(max_items * math.ceil(H / 128), I)
        assert (r["splits_gate_up"], r["splits_down"]) == (sg, sd)
        assert r["gate_up_blocks"] == max_items * math.ceil(I / 64) * sg
        assert r["down_blocks"] == max_items * math.ceil(H / 128) * sd
    else:
        assert r["splits_gate_up"] == r["splits_down"] == 1
        assert r["gate_up_blocks"] == 8 * math.ceil(I / 128) * math.ceil(max_items / 8)
        assert r["down_blocks"] == 8 * math.ceil(H / 128) * math.ceil(max_items / 8)
    assert r["combine_blocks"] == math.ceil(M * H / 4 / 256)
    assert r["workspace_bytes"] == layer.workspace_bytes(M)


# ------------------------------------------------------------ router GEMM


def _router_only_layer(E, H, max_rows):
    """A layer handle for router calls only.  Creation copies the weight
    codes and scales into the layer's tile order, so all four arrays have
    their full shapes (zeros, I = 128), although the router kernels read
    none of them."""
    import torch
    from quantized_mixture_experts_top_amd import Layer
    I = 128
    w13 = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    w2 = torch.zeros((E, H, I // 2), dtype=torch.uint8, device="cuda")
    s13 = torch.zeros((E, 2 * I, H // 32), dtype=torch.int16, device="cuda")
    s2 = torch.zeros((E, H, I // 32), dtype=torch.int16, device="cuda")
    return Layer(E=E, H=H, I=I, top_k=min(8, E), max_rows=max_rows, w13=w13, s13=s13, w2=w2, s2=s2)


@pytest.mark.parametrize("E,H,M", [
    (384, 7168, 1), (384, 7168, 9), (384, 7168, 16),   # GEMV (one wave per expert and 4 tokens)
    (384, 7168, 17), (384, 7168, 300),                 # 32x64 MFMA tiles, ragged token tile
    (384, 7168, 1024), (384, 7168, 4096),              # the layer's sizes
    (100, 1024, 70), (8, 256, 16), (1000, 128, 65),    # experts not a multiple of 64; K of 2 chunks
    (64, 384, 100),                                    # 6 chunks: two K groups take 2, two take 1
])
def test_router_logits_parity(E, H, M):
    """logits = x @ W_r^T (bf16 inputs, fp32 accumulation) against the
    float64 oracle: each entry within 4e-5 of sum_k |x_k w_k| (fp32 rounding
    of a K-term sum), plus the routing the GPU logits give bit-exact."""
    x, wr = synth.hidden(51, M, H), synth.router_weights(52, E, H)
    layer = _router_only_layer(E, H, M)
    got = layer.router_logits(dev_bf16(x), dev_bf16(wr)).cpu().numpy().astype(np.float64)
    ref = oracle_moe.router_logits(x, wr)
    bound = 4e-5 * (np.abs(oracle_moe.decode_bf16(x)) @ np.abs(oracle_moe.decode_bf16(wr)).T) + 1e-30
    worst = float(np.max(np.abs(got - ref) / bound))
    say(f"router E={E} H={H} M={M}: worst |gpu-oracle| / bound = {worst:.3f}; max|logit| {np.max(np.abs(ref)):.3f}")
    assert worst <= 1.0


@pytest.mark.parametrize("M", [9, 130])
def test_forward_router(M):
    """The router and the layer in one call: bit-equal to the two-step path
    (router logits, then forward), routing bit-exact against the oracle on
    those logits, output within the bar of the oracle's."""
    import torch
    shape = synth.LayerShape(E=64, H=1024, I=512, top_k=4, shared=True)
    layer, w = make_layer(shape, 61, M)
    x, wr = synth.hidden(62, M, shape.H), synth.router_weights(63, shape.E, shape.H)
    xd, wrd = dev_bf16(x), dev_bf16(wr)
    lg = layer.router_logits(xd, wrd)
    two_step = layer.forward(xd, lg).clone()
    base_launches = layer.receipt()["launches"]
    fused = layer.forward_router(xd, wrd)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), two_step.view(torch.int16))
    r = layer.receipt()
    assert r["router"] == 1 and r["launches"] == base_launches + 1
    lgn = lg.cpu().numpy()
    ref = oracle_moe.forward(x, lgn, shape.top_k, expert_getter(w), shape.I, shared=shared_of(w))
    check_routing(layer, M, ref, shape.E)
    err = rel_err(fused.float().cpu().numpy(), ref["out"])
    say(f"forward_router M={M}: rel err {err:.3e}")
    assert err <= REL_TOL


# ------------------------------------------------------------ GEMV split-K

SPLITK_CASES = [
    # E, H, I, k, M, shared: GEMV launches of fewer than 128 blocks split K
    (8, 4096, 256, 2, 1, False),     # gate+up in 8 splits; down K=256 unsplit
    (16, 2048, 1024, 2, 2, False),   # gate+up in 4 splits, down in 2
    (4, 2048, 1536, 1, 1, True),     # shared expert: gate+up 4 splits, down 3
    (4, 4352, 640, 2, 3, False),     # 8 whole super-steps over 8 splits, a partial one in the last
]


@pytest.mark.parametrize("E,H,I,k,M,shared", SPLITK_CASES)
def test_gemv_split_k(E, H, I, k, M, shared):
    """K split over blocks, partial sums added by the last block to arrive
    in split order: parity with the oracle, bit-identical repeats (the sum
    does not depend on which block arrives last), the receipt and counter
    name the split, and a captured graph replays to the eager result."""
    import torch
    layer, w, x, lg, ref = _run_case(E, H, I, k, M, shared)
    xs, ls = dev_bf16(x), dev(lg)
    layer.reset_stats()
    out = layer.forward(xs, ls).clone()
    r = layer.receipt()
    say(f"split-K E={E} H={H} I={I} M={M} shared={shared}: splits gate+up {r['splits_gate_up']}, "
        f"down {r['splits_down']}, blocks {r['gate_up_blocks']}/{r['down_blocks']}")
    assert r["regime"] == "gemv" and r["splits_gate_up"] > 1
    assert layer.stats()["splitk_launches"] == (r["splits_gate_up"] > 1) + (r["splits_down"] > 1)
    check_routing(layer, M, ref, E)
    err = rel_err(out.float().cpu().numpy(), ref["out"])
    say(f"  rel err out {err:.3e}")
    assert err <= REL_TOL
    for _ in range(3):
        again = layer.forward(xs, ls)
        assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    g_out = torch.empty_like(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xs, ls, out=g_out)
    for rep in range(3):
        g_out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_out.view(torch.int16), out.view(torch.int16)), f"replay {rep}"


# ------------------------------------------------------ expert-parallel shard


@pytest.mark.parametrize("M", [3, 24, 130])  # GEMV items; tiles; tiles with two routing kernels
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
def test_expert_parallel_shards(M, shared, scoring):
    """Four shards of four experts each route over all 16 experts and compute
    their own: each shard's output, counts and offsets against the oracle's
    shard, and the four outputs against the whole layer (the shared expert,
    when there is one, held by shard 0 only, as it would be computed once).
    Under the sigmoid scoring every shard gets the bias of all 16 experts."""
    import torch
    E, H, I, k = 16, 512, 256, 4
    shape = synth.LayerShape(E=E, H=H, I=I, top_k=k, shared=shared)
    w = synth.all_experts(71, shape)
    x, lg = synth.hidden(72, M, H), synth.logits(73, M, E)
    get, sh = expert_getter(w), shared_of(w)
    sc_kw, sc_ref = {}, None
    if scoring == "sigmoid":
        bias = _expert_bias(74, E)
        sc_kw = {"scoring": "sigmoid", "expert_bias": bias, "routed_scale": SIG_SCALE}
        sc_ref = {"kind": "sigmoid", "bias": bias, "scale": SIG_SCALE}
    full = oracle_moe.forward(x, lg, k, get, I, shared=sh, scoring=sc_ref)
    total = np.zeros_like(full["out"])
    for g in range(4):
        lo = 4 * g
        part = {key: w[key][lo:lo + 4] for key in ("w13", "s13", "w2", "s2")}
        if shared and g == 0:
            part.update({"shared_" + key: w["shared_" + key] for key in ("w13", "s13", "w2", "s2")})
        from quantized_mixture_experts_top_amd import layer_from_numpy
        layer = layer_from_numpy(part, E=E, H=H, I=I, top_k=k, max_rows=M, local_first=lo, local_count=4,
                                 **sc_kw)
        out = layer.forward(dev_bf16(x), dev(lg)).float().cpu().numpy()
        ref = oracle_moe.forward(x, lg, k, get, I, shared=sh if g == 0 else None, local=(lo, 4),
                                 scoring=sc_ref)
        rt = layer.read_routing(M)
        assert np.array_equal(rt["ids"].cpu().numpy(), full["ids"])
        assert np.array_equal(rt["counts"].cpu().numpy(), full["counts"][lo:lo + 4])
        assert np.array_equal(rt["offsets"].cpu().numpy(), full["offsets"][lo:lo + 5] - full["offsets"][lo])
        n_loc = int(full["counts"][lo:lo + 4].sum())
        assert np.array_equal(rt["perm"].cpu().numpy()[:n_loc], full["perm"][full["offsets"][lo]:full["offsets"][lo + 4]])
        err = rel_err(out, ref["out"])
        say(f"shard [{lo}, {lo + 4}) M={M} shared={shared}: {n_loc} local slots, rel err {err:.3e}")
        assert err <= REL_TOL
        total += out
        layer.close()
    err = rel_err(total, full["out"])
    say(f"  shards summed vs the whole layer: rel err {err:.3e}")
    assert err <= REL_TOL


# ----------------------------------------------------- sigmoid router scoring

SIG_SCALE = 2.5


def _expert_bias(seed, E):
    """A per-expert selection bias of the size a load-balancing bias takes
    (a few hundredths), float32."""
    return (np.random.default_rng(seed).standard_normal(E) * 0.05).astype(np.float32)


def _check_sigmoid_routing(layer, M, lg, k, E, bias, scale):
    """ids against the oracle's float32 selection keys: equal, or, for a
    token whose keys the two sides round a few ulp apart (the GPU's expf is
    not correctly rounded), a valid top-k of those keys within that margin;
    weights, counts, offsets and perm from the GPU's own ids to the oracle's
    rules (weights to W_REL_TOL, the rest bit-exact)."""
    from helpers import W_REL_TOL
    r = {key: v.cpu().numpy() for key, v in layer.read_routing(M).items()}
    ids = r["ids"]
    ref = oracle_moe.route(lg, k, {"kind": "sigmoid", "bias": bias, "scale": scale})
    keys = oracle_moe.sigmoid_selection_keys(lg, bias).astype(np.float64)
    near = np.nonzero(np.any(ids != ref["ids"], axis=1))[0]
    for t in near:
        sel = ids[t].astype(np.int64)
        assert np.unique(sel).size == k and sel.min() >= 0 and sel.max() < E, f"token {t}: ids {sel}"
        tol = 4.0 * float(np.spacing(np.float32(max(1.0, np.max(np.abs(keys[t]))))))
        ks = keys[t, sel]
        assert np.all(ks[:-1] >= ks[1:] - tol), f"token {t}: selection order {ks}"
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            assert np.max(keys[t, rest]) <= ks.min() + tol, f"token {t}: an unselected key beats a selected one"
    assert near.size <= 2 + M // 1000, f"{near.size} tokens off the oracle's selection"
    if M:
        wref = oracle_moe.sigmoid_weights(lg, ids, scale)
        werr = np.max(np.abs(r["w"].astype(np.float64) - wref) / wref)
        assert werr <= W_REL_TOL, f"sigmoid routing weight rel err {werr:.2e}"
        assert np.allclose(r["w"].astype(np.float64).sum(axis=1), scale, rtol=1e-5)
    counts, offsets = oracle_moe.count_and_scan(ids, E)
    perm, _ = oracle_moe.sort_slots(ids, E)
    assert np.array_equal(r["counts"], counts) and np.array_equal(r["offsets"], offsets)
    assert np.array_equal(r["perm"], perm)
    return near.size


@pytest.mark.parametrize("E,k,M,kind,biased", [
    (384, 8, 1, "normal", True),
    (384, 8, 9, "normal", True),
    (384, 8, 100, "normal", False),
    (384, 8, 1024, "normal", True),
    (384, 8, 4096, "normal", True),
    (64, 4, 300, "ties", True),        # equal logits: equal scores, the bias or the index decides
    (384, 8, 256, "saturated", False), # logits x30: scores of exactly 1.0 in float32, ties to the index
    (16, 16, 130, "normal", True),     # every expert selected, in key order
    (1000, 32, 70, "normal", True),    # experts not a multiple of 64
])
def test_sigmoid_routing(E, k, M, kind, biased):
    say(f"sigmoid route E={E} k={k} M={M} {kind} bias={biased}")
    shape = synth.LayerShape(E=E, H=128, I=128, top_k=k)
    bias = _expert_bias(7, E) if biased else None
    layer, _ = make_layer(shape, 1, M, scoring="sigmoid", expert_bias=bias, routed_scale=SIG_SCALE)
    lg = synth.logits(3, M, E) * np.float32(30.0) if kind == "saturated" else _logits(kind, 3, M, E)
    layer.route(dev_bf16(synth.hidden(2, M, 128)), dev(lg))
    n = _check_sigmoid_routing(layer, M, lg, k, E, bias, SIG_SCALE)
    say(f"  {n} near-tie tokens checked for validity")
    layer.close()


@pytest.mark.parametrize("E,H,I,k,M,shared", [
    (64, 512, 256, 4, 3, False),    # GEMV items
    (16, 512, 256, 4, 130, True),   # 128-row tiles, shared expert
])
def test_sigmoid_forward_parity(E, H, I, k, M, shared):
    """The whole layer under the sigmoid router against the oracle's, and the
    fused router + layer call bit-equal to the two-step path."""
    import torch
    say(f"sigmoid forward E={E} H={H} I={I} k={k} M={M} shared={shared}")
    shape = synth.LayerShape(E=E, H=H, I=I, top_k=k, shared=shared)
    bias = _expert_bias(11, E)
    layer, w = make_layer(shape, 5, M, scoring="sigmoid", expert_bias=bias, routed_scale=SIG_SCALE)
    x, wr = synth.hidden(6, M, H), synth.router_weights(8, E, H)
    xd, wrd = dev_bf16(x), dev_bf16(wr)
    lg = layer.router_logits(xd, wrd)
    out = layer.forward(xd, lg).clone()
    fused = layer.forward_router(xd, wrd)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), out.view(torch.int16))
    lgn = lg.cpu().numpy()
    scoring = {"kind": "sigmoid", "bias": bias, "scale": SIG_SCALE}
    ref = oracle_moe.forward(x, lgn, k, expert_getter(w), I, shared=shared_of(w), scoring=scoring)
    assert _check_sigmoid_routing(layer, M, lgn, k, E, bias, SIG_SCALE) == 0
    err = rel_err(out.float().cpu().numpy(), ref["out"])
    say(f"  rel err {err:.3e}")
    assert err <= REL_TOL
    layer.close()

"""Parity at the full layer size (E=384, H=7168, I=2048, top-8, int4
group-32), in the launch configuration the benchmark times: routing for
every token bit-exact, the output checked on a seeded sample of tokens
(each output row depends only on its own token and logits).

The oracle's expert MLPs are computed once per expert for the sampled rows
of every case together (each expert's weights are decoded once), in a
thread pool; each case then combines its tokens' rows in slot order."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from helpers import REL_TOL, check_routing, dev, dev_bf16, rel_err, say, upload_full
from oracle import moe as oracle_moe

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

SEED = 0
TILE_ROWS = 128  # rows of one MFMA work item
CASES = [
    # workload, M, number of sampled tokens besides the first and last (None = all)
    ("decode", 1, None),
    ("decode", 9, None),
    ("transition", 90, 64),
    ("transition", 256, 64),
    ("plateau", 1024, 64),
    ("plateau", 4096, 256),
    ("skew", 512, 64),
]
TP8_CASES = [(1, None), (9, None), (256, 64), (4096, 256)]


def _sample(M, n, salt):
    if n is None or n + 2 >= M:
        return np.arange(M)
    rng = np.random.default_rng(salt + M)
    inner = rng.choice(np.arange(1, M - 1), n, replace=False)
    return np.unique(np.concatenate([[0, M - 1], inner]))


def _coverage(route, tokens, k, E, M):
    """Where the sampled rows sit in the MFMA work items: per sampled routed
    row, its row block (0..7) inside its 128-row item, and the number of row
    blocks of that item (the K-loop instantiation it ran through)."""
    if 4 * M * k <= 7 * E:
        return "dot-product GEMV items (<= 2 rows)"
    counts, offsets, inv = route["counts"], route["offsets"], route["inv_perm"]
    rbs, loops = set(), set()
    for t in tokens:
        for j in range(k):
            e = int(route["ids"][t, j])
            r = int(inv[t * k + j]) - int(offsets[e])
            item = r // TILE_ROWS
            rows = min(TILE_ROWS, int(counts[e]) - item * TILE_ROWS)
            rbs.add((r % TILE_ROWS) // 16)
            loops.add((rows + 15) // 16)
    return f"row blocks {sorted(rbs)}, items of {sorted(loops)} row blocks"


class _Reference:
    """Oracle outputs of the sampled tokens of several cases on one layer's
    weights: routing per case, each expert's MLP once for all rows routed to
    it, then each token's slots combined in order."""

    def __init__(self, shape, cases, salt, threads=16):
        self.shape, self.cases = shape, {}
        local = set(shape.local_experts())  # an expert-parallel shard sums its own slots only
        self.local = local
        k, I = shape.top_k, shape.I
        rows = {}  # expert -> list of (case key, token)
        for key, (wl_name, M, n) in cases.items():
            wl = synth.WORKLOADS[wl_name]
            inp = synth.inputs(SEED, wl.shape, M, skew=wl.skew)
            r = oracle_moe.route(inp["logits"], k)
            tokens = _sample(M, n, salt)
            self.cases[key] = {"inp": inp, "route": r, "tokens": tokens, "shared": wl.shape.shared,
                               "xf": oracle_moe.decode_bf16(inp["x"])}
            for t in tokens:
                for j in range(k):
                    if int(r["ids"][t, j]) in local:
                        rows.setdefault(int(r["ids"][t, j]), []).append((key, int(t)))
                if wl.shape.shared:
                    rows.setdefault("shared", []).append((key, int(t)))
        say(f"oracle: {len(rows)} expert MLPs over {sum(len(v) for v in rows.values())} sampled rows")
        self.y = {}

        def work(e):
            X = np.stack([self.cases[c]["xf"][t] for c, t in rows[e]])
            return e, oracle_moe.expert_mlp(X, synth.expert(SEED, shape, e), I)

        done = 0
        with ThreadPoolExecutor(min(threads, os.cpu_count() or 1)) as ex:
            for e, Y in ex.map(work, sorted(rows, key=str)):
                for (c, t), y in zip(rows[e], Y):
                    self.y[(c, t, e)] = y
                done += 1
                if done % 64 == 0:
                    say(f"  oracle experts done: {done}/{len(rows)}")

    def out(self, key):
        c = self.cases[key]
        r, k = c["route"], self.shape.top_k
        res = []
        for t in c["tokens"]:
            js = [j for j in range(k) if int(r["ids"][t, j]) in self.local]
            ys = [self.y[(key, int(t), int(r["ids"][t, j]))] for j in js]
            sh = self.y[(key, int(t), "shared")] if c["shared"] else None
            if js:
                res.append(oracle_moe.combine(r["w"][t][js], ys, sh))
            else:
                res.append(sh if sh is not None else np.zeros(self.shape.H))
        return np.stack(res)


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


@pytest.fixture(scope="module")
def full_ref():
    say("oracle for the sampled tokens of every full-size case")
    return _Reference(synth.FULL_SHARED, {f"{w}:{M}": (w, M, n) for w, M, n in CASES}, salt=1000)


@pytest.mark.parametrize("workload,M,nsample", CASES)
def test_full_size_parity(full, full_ref, workload, M, nsample):
    wl = synth.WORKLOADS[workload]
    shape = wl.shape
    key = f"{workload}:{M}"
    c = full_ref.cases[key]
    say(f"full size {workload} M={M}")
    layer = full["shared"] if shape.shared else full["routed"]
    inp = c["inp"]
    out = layer.forward(dev_bf16(inp["x"]), dev(inp["logits"])).float().cpu().numpy()
    check_routing(layer, M, c["route"], shape.E)
    tokens = c["tokens"]
    err = rel_err(out[tokens], full_ref.out(key))
    shown = tokens.tolist() if tokens.size <= 12 else tokens[:6].tolist() + ["..."] + tokens[-3:].tolist()
    say(f"  {tokens.size} tokens {shown}; {_coverage(c['route'], tokens, shape.top_k, shape.E, M)}; "
        f"rel err {err:.3e}")
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


@pytest.fixture(scope="module")
def tp8_ref():
    return _Reference(synth.TP8_SLICE, {f"tp8:{M}": ("tp8", M, n) for M, n in TP8_CASES}, salt=2000)


@pytest.mark.parametrize("M,nsample", TP8_CASES)
def test_tp8_slice_parity(tp8, tp8_ref, M, nsample):
    shape = synth.TP8_SLICE
    key = f"tp8:{M}"
    c = tp8_ref.cases[key]
    say(f"tp8 slice M={M}")
    out = tp8.forward(dev_bf16(c["inp"]["x"]), dev(c["inp"]["logits"])).float().cpu().numpy()
    check_routing(tp8, M, c["route"], shape.E)
    tokens = c["tokens"]
    err = rel_err(out[tokens], tp8_ref.out(key))
    say(f"  {tokens.size} tokens; {_coverage(c['route'], tokens, shape.top_k, shape.E, M)}; rel err {err:.3e}")
    assert err <= REL_TOL


EP48_CASES = [(1, None), (9, None), (256, 64), (4096, 256)]


@pytest.fixture(scope="module")
def ep48():
    """One GPU's share under 8-way expert parallelism: experts 0..47 of the
    384 the layer routes over (synthetic weights, the same as the whole
    layer's experts 0..47)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_mixture_experts_top_amd import Layer
    shape = synth.EP48_SLICE
    say("uploading the expert-parallel shard (experts 0..47 of 384, seed 0)")
    r = upload_full(SEED, shape)["routed"]
    layer = Layer(E=shape.E, H=shape.H, I=shape.I, top_k=shape.top_k, max_rows=4096, w13=r["w13"], s13=r["s13"],
                  w2=r["w2"], s2=r["s2"], local_first=shape.local_first, local_count=shape.local_count)
    yield layer
    layer.close()


@pytest.fixture(scope="module")
def ep48_ref():
    return _Reference(synth.EP48_SLICE, {f"ep48:{M}": ("ep48", M, n) for M, n in EP48_CASES}, salt=3000)


@pytest.mark.parametrize("M,nsample", EP48_CASES)
def test_ep48_shard_parity(ep48, ep48_ref, M, nsample):
    shape = synth.EP48_SLICE
    key = f"ep48:{M}"
    c = ep48_ref.cases[key]
    say(f"ep48 shard M={M}")
    out = ep48.forward(dev_bf16(c["inp"]["x"]), dev(c["inp"]["logits"])).float().cpu().numpy()
    r = c["route"]
    rt = ep48.read_routing(M)
    assert np.array_equal(rt["ids"].cpu().numpy(), r["ids"])
    assert np.array_equal(rt["counts"].cpu().numpy(), r["counts"][:48])
    n_loc = int(r["counts"][:48].sum())
    assert np.array_equal(rt["perm"].cpu().numpy()[:n_loc], r["perm"][:n_loc])
    tokens = c["tokens"]
    err = rel_err(out[tokens], ep48_ref.out(key))
    say(f"  {tokens.size} tokens, {n_loc} of {M * 8} routed slots local; rel err {err:.3e}")
    assert err <= REL_TOL

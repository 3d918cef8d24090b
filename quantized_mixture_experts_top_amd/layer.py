"""Python face of the fused int4 MoE layer: a thin wrapper over the C ABI.

Tensors are torch device tensors (PyTorch supplies device memory and the
stream); all computation happens in libqmoe.so's HIP kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from ._binding import SCORING_SIGMOID, SCORING_SOFTMAX, LayerDesc, Receipt, Stats, check, load_library

GROUP = 32


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Layer:
    """One MoE layer over packed int4 weights.

    w13 uint8 [E,2I,H/2], s13 fp16-bits (int16/uint16/float16) [E,2I,H/32],
    w2 uint8 [E,H,I/2], s2 [E,H,I/32]; `shared` an optional dict with the
    same four keys for one always-selected shared expert.  An expert-parallel
    shard routes over E experts but holds and computes only experts
    local_first .. local_first + local_count - 1 (the weight tensors then
    have local_count experts) and returns its partial sum.  The layer keeps
    references to the tensors (the library borrows their memory) and a copy
    of them in the MFMA tiles' order made at construction, so the weights
    must not change while the layer lives: build a new Layer instead."""

    def __init__(self, *, E, H, I, top_k, max_rows, w13, s13, w2, s2, shared=None, local_first=0,
                 local_count=0, scoring="softmax", expert_bias=None, routed_scale=0.0):
        self.lib = load_library()
        self.E, self.H, self.I, self.top_k, self.max_rows = E, H, I, top_k, max_rows
        # creation copies all four arrays into the tile order, so each must
        # hold its full size (a short one would be read past its end)
        n_loc = local_count or E
        need = {"w13": n_loc * 2 * I * (H // 2), "s13": n_loc * 2 * I * (H // 32) * 2,
                "w2": n_loc * H * (I // 2), "s2": n_loc * H * (I // 32) * 2}
        arrays = {"w13": w13, "s13": s13, "w2": w2, "s2": s2}
        for key, nbytes in need.items():
            t = arrays[key]
            if t is not None and t.numel() * t.element_size() < nbytes:
                raise ValueError(f"{key} holds {t.numel() * t.element_size()} bytes, {nbytes} needed")
            if shared and shared[key].numel() * shared[key].element_size() < nbytes // n_loc:
                raise ValueError(f"shared {key} holds fewer than {nbytes // n_loc} bytes")
        self._keep = [w13, s13, w2, s2]
        sh = shared or {}
        if shared:
            self._keep += [sh["w13"], sh["s13"], sh["w2"], sh["s2"]]
        self.has_shared = bool(shared)
        # router scoring: "softmax" (default) or "sigmoid" (expert_bias: fp32 [E]
        # device tensor or None; routed_scale: 0 means 1)
        if scoring not in ("softmax", "sigmoid"):
            raise ValueError(f"scoring must be 'softmax' or 'sigmoid', not {scoring!r}")
        if expert_bias is not None:
            if (expert_bias.dtype != torch.float32 or tuple(expert_bias.shape) != (E,)
                    or expert_bias.device != w13.device):
                raise ValueError("expert_bias must be a float32 [E] tensor on the weights' device")
            self._keep.append(expert_bias)
        sc = SCORING_SIGMOID if scoring == "sigmoid" else SCORING_SOFTMAX
        desc = LayerDesc(E, H, I, top_k, GROUP, max_rows, _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2),
                         _ptr(sh.get("w13")), _ptr(sh.get("s13")), _ptr(sh.get("w2")), _ptr(sh.get("s2")),
                         local_first, local_count, sc, float(routed_scale), _ptr(expert_bias))
        self.local_first, self.local_count = local_first, (local_count or E)
        handle = ctypes.c_void_p()
        check(self.lib.qmoe_layer_create(ctypes.byref(desc), ctypes.byref(handle)))
        self.handle = handle
        self.device = w13.device
        self._ws = {}  # stream handle -> workspace used by calls on that stream

    def close(self):
        if getattr(self, "handle", None):
            self.lib.qmoe_layer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ workspace

    def workspace_bytes(self, M: int) -> int:
        n = ctypes.c_size_t()
        check(self.lib.qmoe_workspace_size(self.handle, M, ctypes.byref(n)))
        return n.value

    def workspace(self, M: int, stream=None) -> torch.Tensor:
        """The workspace of calls on `stream` (default: the current stream),
        large enough for M tokens, kept and grown as needed.  Each stream has
        its own (calls that overlap must not share one), allocated while that
        stream is current, so the caching allocator does not hand its memory
        to anyone else before the stream's queued kernels are done with it.
        A new allocation is initialised explicitly (its memory may have held
        other tensors)."""
        s = torch.cuda.current_stream() if stream is None else stream
        need = self.workspace_bytes(M)
        ws = self._ws.get(s.cuda_stream)
        if ws is None or ws.numel() < need:
            self._ws.pop(s.cuda_stream, None)
            del ws
            with torch.cuda.stream(s):
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            check(self.lib.qmoe_workspace_init(self.handle, _ptr(ws), ws.numel(), _stream(s)))
            self._ws[s.cuda_stream] = ws
        return ws

    def _args(self, M, stream):
        ws = self.workspace(M, stream)
        return _ptr(ws), ws.numel(), _stream(stream)

    # -------------------------------------------------------------- calls

    def _check_inputs(self, x, logits):
        M = x.shape[0]
        if x.dtype != torch.bfloat16 or tuple(x.shape) != (M, self.H):
            raise ValueError(f"x must be bf16 [M, {self.H}]")
        if logits.dtype != torch.float32 or tuple(logits.shape) != (M, self.E):
            raise ValueError(f"logits must be float32 [M, {self.E}]")
        return M

    def forward(self, x, logits, out=None, stream=None):
        M = self._check_inputs(x, logits)
        if out is None:
            out = torch.empty((M, self.H), dtype=torch.bfloat16, device=self.device)
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_forward(self.handle, _ptr(x), _ptr(logits), M, _ptr(out), ws, nb, st))
        return out

    __call__ = forward

    def router_logits(self, x, w_router, stream=None):
        """fp32 [M, E] logits of bf16 x [M, H] through bf16 router weights [E, H]."""
        M = x.shape[0]
        if x.dtype != torch.bfloat16 or tuple(x.shape) != (M, self.H):
            raise ValueError(f"x must be bf16 [M, {self.H}]")
        if w_router.dtype != torch.bfloat16 or tuple(w_router.shape) != (self.E, self.H):
            raise ValueError(f"w_router must be bf16 [{self.E}, {self.H}]")
        out = torch.empty((M, self.E), dtype=torch.float32, device=self.device)
        check(self.lib.qmoe_router_logits(self.handle, _ptr(x), _ptr(w_router), M, _ptr(out), _stream(stream)))
        return out

    def forward_router(self, x, w_router, out=None, stream=None):
        """The router and the whole layer in one call."""
        M = x.shape[0]
        if x.dtype != torch.bfloat16 or tuple(x.shape) != (M, self.H):
            raise ValueError(f"x must be bf16 [M, {self.H}]")
        if w_router.dtype != torch.bfloat16 or tuple(w_router.shape) != (self.E, self.H):
            raise ValueError(f"w_router must be bf16 [{self.E}, {self.H}]")
        if out is None:
            out = torch.empty((M, self.H), dtype=torch.bfloat16, device=self.device)
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_forward_router(self.handle, _ptr(x), _ptr(w_router), M, _ptr(out), ws, nb, st))
        return out

    def route(self, x, logits, stream=None):
        M = self._check_inputs(x, logits)
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_route(self.handle, _ptr(x), _ptr(logits), M, ws, nb, st))

    def gate_up(self, M, stream=None):
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_gate_up(self.handle, M, ws, nb, st))

    def down(self, M, stream=None):
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_down(self.handle, M, ws, nb, st))

    def combine(self, M, out=None, stream=None):
        if out is None:
            out = torch.empty((M, self.H), dtype=torch.bfloat16, device=self.device)
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_combine(self.handle, M, _ptr(out), ws, nb, st))
        return out

    def read_routing(self, M, stream=None) -> dict:
        dev, k, E = self.device, self.top_k, self.E
        r = {
            "ids": torch.empty((M, k), dtype=torch.int32, device=dev),
            "w": torch.empty((M, k), dtype=torch.float32, device=dev),
            "counts": torch.empty((self.local_count,), dtype=torch.int32, device=dev),
            "offsets": torch.empty((self.local_count + 1,), dtype=torch.int32, device=dev),
            "perm": torch.empty((M * k,), dtype=torch.int32, device=dev),
        }
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_read_routing(self.handle, M, ws, nb, _ptr(r["ids"]), _ptr(r["w"]),
                                         _ptr(r["counts"]), _ptr(r["offsets"]), _ptr(r["perm"]), st))
        return r

    def read_intermediate(self, M, which, stream=None) -> torch.Tensor:
        rows = M * self.top_k + (M if self.has_shared else 0)
        cols = self.I if which == 0 else self.H
        out = torch.empty((rows, cols), dtype=torch.float32, device=self.device)
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_read_intermediate(self.handle, M, ws, nb, which, _ptr(out), st))
        return out

    def dequant_debug(self, expert, which, stream=None) -> torch.Tensor:
        shape = (2 * self.I, self.H) if which == 0 else (self.H, self.I)
        out = torch.empty(shape, dtype=torch.int16, device=self.device)
        check(self.lib.qmoe_dequant_debug(self.handle, expert, which, _ptr(out), _stream(stream)))
        return out

    def stats(self) -> dict:
        s = Stats()
        check(self.lib.qmoe_get_stats(self.handle, ctypes.byref(s)))
        return s.as_dict()

    def receipt(self) -> dict:
        """The engagement receipt of the last completed forward call."""
        r = Receipt()
        check(self.lib.qmoe_last_receipt(self.handle, ctypes.byref(r)))
        return r.as_dict()

    def item_count(self, M, stream=None) -> int:
        """Work items the last routing on this stream's workspace built (read back from the device)."""
        n = torch.zeros(1, dtype=torch.int32, device=self.device)
        ws, nb, st = self._args(M, stream)
        check(self.lib.qmoe_read_item_count(self.handle, M, ws, nb, _ptr(n), st))
        return int(n.item())

    def reset_stats(self):
        check(self.lib.qmoe_reset_stats(self.handle))


def layer_from_numpy(weights: dict, *, E, H, I, top_k, max_rows, device="cuda", local_first=0,
                     local_count=0, scoring="softmax", expert_bias=None, routed_scale=0.0) -> Layer:
    """Copy numpy weights (as produced by the seeded generators) to the GPU
    and create a Layer over them (expert_bias: float32 [E] numpy array or
    None, copied too)."""
    def dev(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    shared = None
    if "shared_w13" in weights:
        shared = {k: dev(weights["shared_" + k]) for k in ("w13", "s13", "w2", "s2")}
    return Layer(E=E, H=H, I=I, top_k=top_k, max_rows=max_rows,
                 w13=dev(weights["w13"]), s13=dev(weights["s13"]),
                 w2=dev(weights["w2"]), s2=dev(weights["s2"]), shared=shared, local_first=local_first,
                 local_count=local_count, scoring=scoring, routed_scale=routed_scale,
                 expert_bias=None if expert_bias is None else dev(np.asarray(expert_bias, dtype=np.float32)))

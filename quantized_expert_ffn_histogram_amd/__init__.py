"""Routed mixture-of-experts FFN layer for AMD Instinct MI355X (gfx950).

Python binding of ``libstrata_moe.so``: argument marshalling only.  Every step
of the layer runs in the library's HIP kernels; PyTorch supplies device memory
and the current stream.  The names follow the C ABI in ``include/strata_moe.h``:

    ids, w = route(logits, k)
    counts, offsets, perm, inv_perm = permute(ids, E)
    out = ffn(x, experts, offsets, perm, k, topk_w=w)      # fused combine
    y = ffn(x, experts, offsets, perm, k)                  # grouped rows
    out = combine(y, inv_perm, w, k)                       # deterministic combine
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass, replace

import numpy as np
import torch

from ._abi import LIB_PATH, StrataError, StrataMoeWeights, check, load  # noqa: F401

__all__ = [
    "QuantizedExperts",
    "tile_weights",
    "StrataError",
    "route",
    "permute",
    "ffn",
    "combine",
    "moe_layer",
    "layer",
    "layer_noalloc",
    "LayerRunner",
    "workspace_size",
    "permute_workspace_size",
    "router",
    "kv_quantize",
    "kv_quantize_pair",
    "sparse_attention",
    "timing_enable",
    "timing_query",
    "timing_kernels",
    "load",
    "LIB_PATH",
]


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _p(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


@dataclass
class QuantizedExperts:
    """Group-quantized expert weights resident on the GPU.

    gate, up: uint8 [E, I, H/2]; down: uint8 [E, H, I/2]; *_scale: float16
    [E, N, K/g].  Nibble u (the code's low 4 bits), even K in the low nibble.
    ``fmt`` (``strata_weight_format``): "int4" (q = u - 8), "int4_asym"
    (q = u - z, zero points ``*_zero`` uint8 [E, N, K/g/2], two per byte) or
    "int5" (q = u + 16 b - 16, fifth-bit words ``*_hi`` int32 [E, N, K/32]).
    ``layout`` (``strata_weight_layout``) of the bytes of gate, up and down:
    "rows" (row-major) or "tiled" (32-row x 128-K tiles, see
    ``tile_weights``; the same tensor shapes).
    """

    gate: torch.Tensor
    gate_scale: torch.Tensor
    up: torch.Tensor
    up_scale: torch.Tensor
    down: torch.Tensor
    down_scale: torch.Tensor
    group: int
    fmt: str = "int4"
    gate_zero: torch.Tensor | None = None
    up_zero: torch.Tensor | None = None
    down_zero: torch.Tensor | None = None
    gate_hi: torch.Tensor | None = None
    up_hi: torch.Tensor | None = None
    down_hi: torch.Tensor | None = None
    layout: str = "rows"

    FORMATS = {"int4": 0, "int4_asym": 1, "int5": 2}
    LAYOUTS = {"rows": 0, "tiled": 1}

    @property
    def num_experts(self) -> int:
        return int(self.gate.shape[0])

    @property
    def inter(self) -> int:
        return int(self.gate.shape[1])

    @property
    def hidden(self) -> int:
        return int(self.gate.shape[2] * 2)

    def to_tiled(self) -> "QuantizedExperts":
        """A copy whose gate, up and down codes are in the tiled layout
        (``strata_moe_tile_weights``; scales and side data are shared)."""
        if self.layout == "tiled":
            return self
        return replace(self, gate=tile_weights(self.gate), up=tile_weights(self.up),
                       down=tile_weights(self.down), layout="tiled")

    @classmethod
    def from_numpy(cls, w: dict, group: int, device="cuda", layout: str = "rows") -> "QuantizedExperts":
        """From host arrays by name: gate, gate_scale, ... and, for the other
        formats, gate_zero, ... (uint8) or gate_hi, ... (uint32 words); the
        codes are row-major and converted on the GPU for layout="tiled"."""
        if layout not in cls.LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(cls.LAYOUTS)}, got {layout!r}")

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint32:
                a = a.view(np.int32)
            return torch.from_numpy(a).to(device)

        fmt = "int4_asym" if "gate_zero" in w else "int5" if "gate_hi" in w else "int4"
        side = {name + sfx: dev(w[name + sfx]) for name in ("gate", "up", "down")
                for sfx in ("_zero", "_hi") if name + sfx in w}
        ex = cls(dev(w["gate"]), dev(w["gate_scale"]), dev(w["up"]), dev(w["up_scale"]),
                 dev(w["down"]), dev(w["down_scale"]), group, fmt=fmt, **side)
        return ex.to_tiled() if layout == "tiled" else ex

    def descriptor(self) -> StrataMoeWeights:
        for name, dt in (("gate", torch.uint8), ("up", torch.uint8), ("down", torch.uint8),
                         ("gate_scale", torch.float16), ("up_scale", torch.float16),
                         ("down_scale", torch.float16)):
            _need(getattr(self, name), dt, name)
        if self.fmt not in self.FORMATS:
            raise ValueError(f"fmt must be one of {sorted(self.FORMATS)}, got {self.fmt!r}")
        if self.layout not in self.LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(self.LAYOUTS)}, got {self.layout!r}")
        side = {}
        for name in ("gate", "up", "down"):
            for sfx, dt in (("_zero", torch.uint8), ("_hi", torch.int32)):
                t = getattr(self, name + sfx)
                if t is not None:
                    _need(t, dt, name + sfx)
                side[name + sfx] = 0 if t is None else t.data_ptr()
        return StrataMoeWeights(
            self.gate.data_ptr(), self.gate_scale.data_ptr(), self.up.data_ptr(),
            self.up_scale.data_ptr(), self.down.data_ptr(), self.down_scale.data_ptr(),
            self.num_experts, self.hidden, self.inter, self.group, self.FORMATS[self.fmt],
            side["gate_zero"], side["up_zero"], side["down_zero"],
            side["gate_hi"], side["up_hi"], side["down_hi"], self.LAYOUTS[self.layout],
        )


def tile_weights(packed: torch.Tensor) -> torch.Tensor:
    """``strata_moe_tile_weights``: packed codes uint8 [E, N, K/2] (row-major)
    -> a new tensor of the same shape holding them in the tiled layout."""
    _need(packed, torch.uint8, "packed")
    if packed.dim() != 3:
        raise ValueError(f"packed must be [E, N, K/2], got shape {tuple(packed.shape)}")
    E, N, KB = packed.shape
    out = torch.empty_like(packed)
    check(load().strata_moe_tile_weights(_p(packed), _p(out), E * N, 2 * KB, _stream(packed)))
    return out


def workspace_size(T: int, E: int, k: int, H: int, I: int, g: int) -> int:
    return int(load().strata_moe_workspace_size(T, E, k, H, I, g))


def permute_workspace_size(T: int, E: int, k: int) -> int:
    return int(load().strata_moe_permute_workspace_size(T, E, k))


def _workspace(device, nbytes: int, workspace: torch.Tensor | None) -> torch.Tensor:
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def route(logits: torch.Tensor, k: int):
    """``strata_moe_route``: returns (topk_ids int32 [T, k], topk_w float32 [T, k])."""
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    check(load().strata_moe_route(_p(logits), T, E, k, _p(ids), _p(w), _stream(logits)))
    return ids, w


def router(x: torch.Tensor, w_router: torch.Tensor, k: int):
    """``strata_moe_router``: router projection then top-k.  x bf16 [T, H],
    w_router bf16 [E, H]; returns (logits float32 [T, E], topk_ids int32
    [T, k], topk_w float32 [T, k])."""
    _need(x, torch.bfloat16, "x")
    _need(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError(f"w_router has {w_router.shape[1]} columns, x has {H}")
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    check(load().strata_moe_router(_p(x), T, H, _p(w_router), E, k, _p(logits), _p(ids), _p(w), _stream(x)))
    return logits, ids, w


def permute(topk_ids: torch.Tensor, E: int, workspace: torch.Tensor | None = None):
    """``strata_moe_permute``: returns (counts [E], offsets [E+1], perm [T*k], inv_perm [T*k])."""
    _need(topk_ids, torch.int32, "topk_ids")
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    need = load().strata_moe_permute_workspace_size(T, E, k)
    if need == ctypes.c_size_t(-1).value:
        check(load().strata_moe_permute(None, T, E, k, None, None, None, None, None, 0, None))
    ws = _workspace(dev, need, workspace)
    check(load().strata_moe_permute(_p(topk_ids), T, E, k, _p(counts), _p(offsets), _p(perm), _p(inv),
                                    _p(ws), ws.numel(), _stream(topk_ids)))
    return counts, offsets, perm, inv


def ffn(x: torch.Tensor, experts: QuantizedExperts, offsets: torch.Tensor, perm: torch.Tensor, k: int,
        topk_w: torch.Tensor | None = None, out: torch.Tensor | None = None,
        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``strata_moe_ffn``: out [T, H] float32 when ``topk_w`` is given (fused combine),
    otherwise y [T*k, H] float32 in grouped order."""
    _need(x, torch.bfloat16, "x")
    _need(offsets, torch.int32, "offsets")
    _need(perm, torch.int32, "perm")
    if topk_w is not None:
        _need(topk_w, torch.float32, "topk_w")
    T, H = x.shape
    rows = T if topk_w is not None else T * k
    if out is None:
        out = torch.empty((rows, H), dtype=torch.float32, device=x.device)
    desc = experts.descriptor()
    need = load().strata_moe_workspace_size(T, experts.num_experts, k, experts.hidden, experts.inter,
                                            experts.group)
    ws = _workspace(x.device, need, workspace)
    check(load().strata_moe_ffn(_p(x), T, k, ctypes.byref(desc), _p(offsets), _p(perm), _p(topk_w), _p(out),
                                _p(ws), ws.numel(), _stream(x)))
    return out


def combine(y: torch.Tensor, inv_perm: torch.Tensor, topk_w: torch.Tensor, k: int) -> torch.Tensor:
    """``strata_moe_combine``: out [T, H] float32, summed in slot order."""
    _need(y, torch.float32, "y")
    _need(inv_perm, torch.int32, "inv_perm")
    _need(topk_w, torch.float32, "topk_w")
    P, H = y.shape
    T = P // k
    out = torch.empty((T, H), dtype=torch.float32, device=y.device)
    check(load().strata_moe_combine(_p(y), _p(inv_perm), _p(topk_w), T, k, H, _p(out), _stream(y)))
    return out


def moe_layer(logits: torch.Tensor, x: torch.Tensor, experts: QuantizedExperts, k: int, fused: bool = True,
              workspace: torch.Tensor | None = None) -> dict:
    """All four calls for one layer invocation on the current stream."""
    E = experts.num_experts
    T = x.shape[0]
    if workspace is None:
        workspace = _workspace(x.device, workspace_size(T, E, k, experts.hidden, experts.inter, experts.group), None)
    ids, w = route(logits, k)
    counts, offsets, perm, inv = permute(ids, E, workspace)
    res = dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv_perm=inv)
    if fused:
        res["out"] = ffn(x, experts, offsets, perm, k, topk_w=w, workspace=workspace)
    else:
        y = ffn(x, experts, offsets, perm, k, workspace=workspace)
        res["y"] = y
        res["out"] = combine(y, inv, w, k)
    return res


def layer(logits: torch.Tensor, x: torch.Tensor, experts: QuantizedExperts, k: int,
          workspace: torch.Tensor | None = None) -> dict:
    """The whole layer in one C-ABI call (strata_moe_layer) on the current stream."""
    E = experts.num_experts
    T = x.shape[0]
    dev = x.device
    if workspace is None:
        workspace = _workspace(dev, workspace_size(T, E, k, experts.hidden, experts.inter, experts.group), None)
    res = _layer_outputs(T, E, k, experts.hidden, dev)
    desc = experts.descriptor()
    check(load().strata_moe_layer(_p(logits), _p(x), T, k, ctypes.byref(desc), _p(res["ids"]), _p(res["w"]),
                                  _p(res["counts"]), _p(res["offsets"]), _p(res["perm"]), _p(res["inv_perm"]),
                                  _p(res["out"]), _p(workspace), workspace.numel(), _stream(x)))
    return res


def _layer_outputs(T: int, E: int, k: int, H: int, dev) -> dict:
    return dict(ids=torch.empty((T, k), dtype=torch.int32, device=dev),
                w=torch.empty((T, k), dtype=torch.float32, device=dev),
                counts=torch.empty(E, dtype=torch.int32, device=dev),
                offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                inv_perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                out=torch.empty((T, H), dtype=torch.float32, device=dev))


def layer_noalloc(logits: torch.Tensor, x: torch.Tensor, experts: QuantizedExperts, k: int,
                  outputs: dict | None = None) -> dict:
    """``strata_moe_layer_noalloc``: the layer call on the library's static
    device scratch (no workspace).  ``outputs`` (the dict this returns) may be
    passed back in to reuse the output tensors."""
    T = x.shape[0]
    res = outputs if outputs is not None else _layer_outputs(T, experts.num_experts, k, experts.hidden, x.device)
    desc = experts.descriptor()
    check(load().strata_moe_layer_noalloc(_p(logits), _p(x), T, k, ctypes.byref(desc), _p(res["ids"]),
                                          _p(res["w"]), _p(res["counts"]), _p(res["offsets"]), _p(res["perm"]),
                                          _p(res["inv_perm"]), _p(res["out"]), _stream(x)))
    return res


def kv_quantize(x: torch.Tensor, slots: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor) -> None:
    """``strata_kv_quantize``: quantize x (bf16 [T, Hkv, D]) into cache rows
    ``slots`` (int32 [T]) of ``codes`` (uint8 [L, Hkv, D/2]) and ``scales``
    (float16 [L, Hkv])."""
    _need(x, torch.bfloat16, "x")
    _need(slots, torch.int32, "slots")
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float16, "scales")
    T, Hkv, D = x.shape
    L = codes.shape[0]
    check(load().strata_kv_quantize(_p(x), T, Hkv, D, _p(slots), _p(codes), _p(scales), L, _stream(x)))


def kv_quantize_pair(k: torch.Tensor, v: torch.Tensor, slots: torch.Tensor, k_codes: torch.Tensor,
                     k_scales: torch.Tensor, v_codes: torch.Tensor, v_scales: torch.Tensor) -> None:
    """``strata_kv_quantize_pair``: the keys k and values v (bf16 [T, Hkv, D]
    each) of the same tokens into cache rows ``slots`` of the key and value
    caches, in one launch."""
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    _need(slots, torch.int32, "slots")
    for name, t, dt in (("k_codes", k_codes, torch.uint8), ("v_codes", v_codes, torch.uint8),
                        ("k_scales", k_scales, torch.float16), ("v_scales", v_scales, torch.float16)):
        _need(t, dt, name)
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ in shape")
    T, Hkv, D = k.shape
    L = k_codes.shape[0]
    check(load().strata_kv_quantize_pair(_p(k), _p(v), T, Hkv, D, _p(slots), _p(k_codes), _p(k_scales),
                                         _p(v_codes), _p(v_scales), L, _stream(k)))


def sparse_attention(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                     v_scales: torch.Tensor, sel: torch.Tensor | None, sm_scale: float, n_sel: int | None = None,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """``strata_sparse_attention``: q bf16 [Tq, Hq, D] over the selected rows
    (``sel`` int32 [Tq, n_sel], or None with ``n_sel``: the first n_sel
    positions) of a 4-bit cache; returns float32 [Tq, Hq, D]."""
    _need(q, torch.bfloat16, "q")
    for name, t, dt in (("k_codes", k_codes, torch.uint8), ("v_codes", v_codes, torch.uint8),
                        ("k_scales", k_scales, torch.float16), ("v_scales", v_scales, torch.float16)):
        _need(t, dt, name)
    Tq, Hq, D = q.shape
    L, Hkv = k_codes.shape[0], k_codes.shape[1]
    if sel is not None:
        _need(sel, torch.int32, "sel")
        n_sel = sel.shape[1]
    if out is None:
        out = torch.empty((Tq, Hq, D), dtype=torch.float32, device=q.device)
    lib = load()
    ws = _workspace(q.device, lib.strata_sparse_attention_workspace_size(Tq, Hq, n_sel), workspace)
    check(lib.strata_sparse_attention(_p(q), Tq, Hq, _p(k_codes), _p(k_scales), _p(v_codes), _p(v_scales), L, Hkv,
                                      D, _p(sel), n_sel, float(sm_scale), _p(out), _p(ws), ws.numel(), _stream(q)))
    return out


def timing_enable(on: bool = True) -> None:
    """Start (or stop) per-kernel event timing inside the library; clears old records."""
    check(load().strata_moe_timing_enable(1 if on else 0))


def timing_query(kernel: str | None = None) -> tuple[int, float]:
    """(launches, total device ms) of ``kernel`` (None: all) since timing_enable."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    check(load().strata_moe_timing_query(kernel.encode() if kernel else None, ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def timing_kernels() -> list[str]:
    lib = load()
    n = lib.strata_moe_timing_kernels(None, 0)
    arr = (ctypes.c_char_p * max(n, 1))()
    lib.strata_moe_timing_kernels(arr, n)
    return [arr[i].decode() for i in range(n)]


class LayerRunner:
    """One layer invocation with preallocated outputs and workspace, for
    timing loops.  Marshalling only: ``single_call`` runs strata_moe_layer,
    otherwise the same three or four C-ABI calls as ``moe_layer``."""

    def __init__(self, experts: QuantizedExperts, T: int, E: int, k: int, fused: bool = True, device="cuda",
                 single_call: bool = False):
        self.experts, self.T, self.E, self.k, self.fused = experts, T, E, k, fused
        self.single_call = single_call and fused
        H = experts.hidden
        dev = torch.device(device)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        self.inv = torch.empty(T * k, dtype=torch.int32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.float32, device=dev)
        self.y = None if fused else torch.empty((T * k, H), dtype=torch.float32, device=dev)
        nbytes = workspace_size(T, E, k, H, experts.inter, experts.group)
        self.ws = _workspace(dev, nbytes, None)
        self.desc = experts.descriptor()
        self.lib = load()

    def __call__(self, logits: torch.Tensor, x: torch.Tensor) -> torch.Tensor:
        lib, T, E, k = self.lib, self.T, self.E, self.k
        s = _stream(x)
        if self.single_call:
            check(lib.strata_moe_layer(_p(logits), _p(x), T, k, ctypes.byref(self.desc), _p(self.ids), _p(self.w),
                                       _p(self.counts), _p(self.offsets), _p(self.perm), _p(self.inv), _p(self.out),
                                       _p(self.ws), self.ws.numel(), s))
            return self.out
        check(lib.strata_moe_route(_p(logits), T, E, k, _p(self.ids), _p(self.w), s))
        check(lib.strata_moe_permute(_p(self.ids), T, E, k, _p(self.counts), _p(self.offsets), _p(self.perm),
                                     _p(self.inv), _p(self.ws), self.ws.numel(), s))
        if self.fused:
            check(lib.strata_moe_ffn(_p(x), T, k, ctypes.byref(self.desc), _p(self.offsets), _p(self.perm),
                                     _p(self.w), _p(self.out), _p(self.ws), self.ws.numel(), s))
        else:
            check(lib.strata_moe_ffn(_p(x), T, k, ctypes.byref(self.desc), _p(self.offsets), _p(self.perm),
                                     None, _p(self.y), _p(self.ws), self.ws.numel(), s))
            check(lib.strata_moe_combine(_p(self.y), _p(self.inv), _p(self.w), T, k, self.experts.hidden,
                                         _p(self.out), s))
        return self.out

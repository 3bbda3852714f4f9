"""Python binding of the MoE layer library: argument marshalling only.

Every function maps torch tensors (device memory) and the current HIP stream
to the C ABI of include/moe.h and returns.  No arithmetic of the layer runs in
Python; torch provides allocation and streams.
"""

from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import (DTYPE_BF16, DTYPE_F32, LAYOUT_GATE_UP, LAYOUT_PLAIN, ROUTER_AUTO,
                   ROUTER_CANONICAL, ROUTER_MFMA, TIER_BF16, TIER_INT4, TIER_INT8, ExpertHandle,
                   LayerDesc, MoeError, check)

__all__ = [
    "TIER_BF16", "TIER_INT8", "TIER_INT4", "LAYOUT_PLAIN", "LAYOUT_GATE_UP", "MoeError",
    "ROUTER_AUTO", "ROUTER_CANONICAL", "ROUTER_MFMA",
    "packed_size", "quantize_pack", "pack_expert", "Layer",
]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _require_cuda(t: torch.Tensor, name: str, dtypes: Sequence[torch.dtype]) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def packed_size(tier: int, n_out: int, k_in: int) -> int:
    return int(_lib.load().moe_packed_size(int(tier), int(n_out), int(k_in)))


def quantize_pack(w: torch.Tensor, tier: int, layout: int = LAYOUT_PLAIN,
                  out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Quantize and pack one [n_out, k_in] bf16 matrix on the GPU -> uint8 blob."""
    _require_cuda(w, "w", _BF16)
    n, k = w.shape
    size = packed_size(tier, n, k)
    if size == 0:
        raise MoeError(_lib.MOE_ESHAPE, "quantize_pack", f"unsupported shape {tuple(w.shape)}")
    if out is None:
        out = torch.empty(size, dtype=torch.uint8, device=w.device)
    check(_lib.load().moe_quantize_pack(int(tier), int(layout), w.data_ptr(), n, k,
                                        out.data_ptr(), out.numel(), _stream(stream)),
          "moe_quantize_pack")
    return out


def quantize_pack_async(w: torch.Tensor, tier: int, layout: int, out: torch.Tensor,
                        status: torch.Tensor, stream=None) -> torch.Tensor:
    """Enqueue quantize+pack on `stream` without synchronizing; status (device
    int32 [1]) is nonzero after completion if the weights were out of range."""
    _require_cuda(w, "w", _BF16)
    _require_cuda(status, "status", (torch.int32,))
    n, k = w.shape
    check(_lib.load().moe_quantize_pack_async(tier, layout, w.data_ptr(), n, k, out.data_ptr(),
                                              out.numel(), status.data_ptr(), _stream(stream)),
          "moe_quantize_pack_async")
    return out


def plan_tiers(hot: Sequence[float], bytes_per_tier: Sequence[int], budget_bytes: int,
               hi_tier: int, lo_tier: int) -> Tuple[List[int], int]:
    """Budget-feasible top-n plan (host): (tier per expert, n promoted)."""
    E = len(hot)
    h = (ctypes.c_float * E)(*[float(v) for v in hot])
    b = (ctypes.c_size_t * 3)(*[int(v) for v in bytes_per_tier])
    out = (ctypes.c_int32 * E)()
    n = ctypes.c_int32()
    check(_lib.load().moe_plan_tiers(h, E, b, int(budget_bytes), hi_tier, lo_tier, out,
                                     ctypes.byref(n)), "moe_plan_tiers")
    return list(out), n.value


def pack_expert(w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, tier: int,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(w13 blob, w2 blob) of one expert from its bf16 [I,H], [I,H], [H,I] weights."""
    w13 = torch.cat([w_gate, w_up], dim=0).contiguous()
    return (quantize_pack(w13, tier, LAYOUT_GATE_UP, stream=stream),
            quantize_pack(w_down.contiguous(), tier, LAYOUT_PLAIN, stream=stream))


class Layer:
    """A quantized MoE layer: geometry plus the device table of expert handles.

    handles: per expert (tier, w13_blob, w2_blob) with blobs from pack_expert.
    The Layer keeps references to the blobs so they outlive its use.
    """

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int,
                 handles: Sequence[Tuple[int, torch.Tensor, torch.Tensor]], stream=None):
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k
        self._lib = _lib.load()
        self._blobs: List[Tuple[torch.Tensor, torch.Tensor]] = [(h[1], h[2]) for h in handles]
        self.handles: List[Tuple[int, torch.Tensor, torch.Tensor]] = [tuple(h) for h in handles]
        arr = self._handle_array(handles)
        desc = LayerDesc(hidden, inter, n_experts, top_k)
        out = ctypes.c_void_p()
        check(self._lib.moe_layer_create(ctypes.byref(desc), arr, _stream(stream),
                                         ctypes.byref(out)), "moe_layer_create")
        self._h = out
        self._events = None
        self._ws: Dict[Tuple[int, int], torch.Tensor] = {}
        # waves keep their own workspaces (an accumulating wave reads the
        # routing its layer call's first wave left there) and remember which
        # of them hold such a first wave
        self._wave_ws: Dict[Tuple[int, int], torch.Tensor] = {}
        self._wave_routed: set = set()

    @staticmethod
    def _handle_array(handles):
        arr = (ExpertHandle * max(1, len(handles)))()
        for i, (tier, w13, w2) in enumerate(handles):
            arr[i] = ExpertHandle(int(tier), 0, w13.data_ptr(), w2.data_ptr())
        return arr

    def set_experts(self, first: int, handles, stream=None) -> None:
        """Stream-ordered replacement of handles [first, first+len(handles))."""
        arr = self._handle_array(handles)
        check(self._lib.moe_layer_set_experts(self._h, int(first), len(handles), arr,
                                              _stream(stream)), "moe_layer_set_experts")
        for i, h in enumerate(handles):
            self._blobs[first + i] = (h[1], h[2])
            self.handles[first + i] = tuple(h)

    def workspace_size(self, T: int) -> int:
        return int(self._lib.moe_workspace_size(self._h, int(T)))

    def plan_gemms(self, T: int) -> Tuple[Tuple[int, int], Tuple[int, int]]:
        """((path, tile_rows) of the gate/up GEMM, (path, tile_rows) of the down
        GEMM) for a forward of T tokens: path 1 = few routes per expert (weight
        streaming), 2 = many (fp16 MFMA); routes per M-tile."""
        p13, r13, p2, r2 = (ctypes.c_int32() for _ in range(4))
        check(self._lib.moe_layer_plan(self._h, int(T), ctypes.byref(p13), ctypes.byref(r13),
                                       ctypes.byref(p2), ctypes.byref(r2)), "moe_layer_plan")
        return (p13.value, r13.value), (p2.value, r2.value)

    def plan(self, T: int) -> Tuple[int, int]:
        """(path, tile_rows) of the gate/up GEMM (plan_gemms has both GEMMs)."""
        return self.plan_gemms(T)[0]

    def workspace(self, T: int, device) -> torch.Tensor:
        """A cached workspace tensor large enough for T tokens (allocated by torch)."""
        dev = torch.device(device)
        key = (dev.index or 0, int(T))
        ws = self._ws.get(key)
        if ws is None:
            ws = torch.empty(max(256, self.workspace_size(T)), dtype=torch.uint8, device=dev)
            self._ws[key] = ws
        return ws

    def route(self, x: torch.Tensor, wr: torch.Tensor, bias: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None,
              want_logits: bool = True) -> Dict[str, torch.Tensor]:
        """Routing only.  want_logits=False lets many-token calls use the
        certified MFMA router (same ids, weights and permutation)."""
        _require_cuda(x, "x", _BF16)
        _require_cuda(wr, "wr", _BF16)
        if bias is not None:
            _require_cuda(bias, "bias", (torch.float32,))
        T = x.shape[0]
        dev = x.device
        k, E = self.top_k, self.n_experts
        out = dict(
            ids=torch.empty((T, k), dtype=torch.int32, device=dev),
            weights=torch.empty((T, k), dtype=torch.float32, device=dev),
            logits=torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None,
            offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
            sorted_routes=torch.empty(T * k, dtype=torch.int32, device=dev),
            route_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
        )
        ws = self.workspace(T, dev) if workspace is None else workspace
        check(self._lib.moe_route(self._h, x.data_ptr(), wr.data_ptr(), _ptr(bias), T,
                                  out["ids"].data_ptr(), out["weights"].data_ptr(),
                                  _ptr(out["logits"]), out["offsets"].data_ptr(),
                                  out["sorted_routes"].data_ptr(), out["route_pos"].data_ptr(),
                                  ws.data_ptr(), ws.numel(), _stream(stream)), "moe_route")
        if not want_logits:
            del out["logits"]
        return out

    def forward(self, x: torch.Tensor, wr: torch.Tensor, bias: Optional[torch.Tensor] = None,
                out_dtype: torch.dtype = torch.float32, y: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        _require_cuda(x, "x", _BF16)
        _require_cuda(wr, "wr", _BF16)
        if bias is not None:
            _require_cuda(bias, "bias", (torch.float32,))
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.hidden), dtype=out_dtype, device=x.device)
        _require_cuda(y, "y", (torch.float32, torch.bfloat16))
        yd = DTYPE_F32 if y.dtype == torch.float32 else DTYPE_BF16
        ws = self.workspace(T, x.device) if workspace is None else workspace
        check(self._lib.moe_layer_forward(self._h, x.data_ptr(), wr.data_ptr(), _ptr(bias), T,
                                          y.data_ptr(), yd, ws.data_ptr(), ws.numel(),
                                          _stream(stream)), "moe_layer_forward")
        return y

    def forward_noalloc(self, x: torch.Tensor, wr: torch.Tensor, y: torch.Tensor,
                        bias: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """moe_layer_forward_noalloc: the same forward with the library's fixed
        per-device scratch as workspace; y must be given (nothing is allocated)."""
        _require_cuda(x, "x", _BF16)
        _require_cuda(wr, "wr", _BF16)
        _require_cuda(y, "y", (torch.float32, torch.bfloat16))
        if bias is not None:
            _require_cuda(bias, "bias", (torch.float32,))
        check(self._lib.moe_layer_forward_noalloc(self._h, x.data_ptr(), wr.data_ptr(), _ptr(bias),
                                                  x.shape[0], y.data_ptr(),
                                                  DTYPE_F32 if y.dtype == torch.float32 else DTYPE_BF16,
                                                  _stream(stream)), "moe_layer_forward_noalloc")
        return y

    def bind_forward(self, x: torch.Tensor, wr: torch.Tensor, bias: Optional[torch.Tensor],
                     y: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None):
        """A zero-argument callable that enqueues one forward with these fixed
        buffers (arguments marshalled once; used for timing loops)."""
        _require_cuda(x, "x", _BF16)
        _require_cuda(wr, "wr", _BF16)
        _require_cuda(y, "y", (torch.float32, torch.bfloat16))
        ws = self.workspace(x.shape[0], x.device) if workspace is None else workspace
        fn = self._lib.moe_layer_forward
        args = (self._h, x.data_ptr(), wr.data_ptr(), _ptr(bias), x.shape[0], y.data_ptr(),
                DTYPE_F32 if y.dtype == torch.float32 else DTYPE_BF16, ws.data_ptr(), ws.numel(),
                _stream(stream))
        keep = (x, wr, bias, y, ws)

        def run():
            rc = fn(*args)
            if rc:
                check(rc, "moe_layer_forward")
            return keep
        return run

    def set_hotness(self, hot: Optional[torch.Tensor], decay: float = 1.0) -> None:
        """Route-count trace of later forwards: hot[e] = decay*hot[e] + routes to e."""
        if hot is not None:
            _require_cuda(hot, "hot", (torch.float32,))
            if hot.numel() != self.n_experts:
                raise ValueError("hot needs one entry per expert")
        check(self._lib.moe_layer_set_hotness(self._h, _ptr(hot), float(decay)), "moe_layer_set_hotness")
        self._hot = hot

    def set_slots(self, first: int, handles, stream=None) -> None:
        """Resident slots [first, first+len) for wave execution; handles as for
        the constructor: (tier, w13 blob, w2 blob)."""
        arr = self._handle_array(handles)
        check(self._lib.moe_layer_set_slots(self._h, first, len(handles), arr, _stream(stream)),
              "moe_layer_set_slots")
        self._keep_slots = getattr(self, "_keep_slots", {})
        for i, h in enumerate(handles):
            self._keep_slots[first + i] = h

    def set_slot_map(self, expert_to_slot: Sequence[int], stream=None) -> None:
        """Global expert -> resident slot map of the next waves (-1 = inactive)."""
        if len(expert_to_slot) != self.n_experts:
            raise ValueError(f"slot map needs {self.n_experts} entries")
        arr = (ctypes.c_int32 * self.n_experts)(*[int(v) for v in expert_to_slot])
        check(self._lib.moe_layer_set_slot_map(self._h, arr, _stream(stream)), "moe_layer_set_slot_map")

    def forward_wave(self, x: torch.Tensor, wr: torch.Tensor, bias: Optional[torch.Tensor] = None,
                     y: Optional[torch.Tensor] = None, accumulate: bool = False,
                     out_dtype: torch.dtype = torch.float32,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """One wave over the experts the current slot map sends to slots
        (y = or y += the wave's output; accumulating needs an fp32 y and reuses
        the routing the previous wave left in the workspace).  Without an
        explicit workspace the layer keeps one per token count for its waves,
        apart from the one forward() and route() use, and refuses an
        accumulating wave that no first wave (accumulate=False) of the same
        token count has routed since the last set_router_mode.  With an
        explicit workspace that ordering is the caller's to keep."""
        _require_cuda(x, "x", _BF16)
        _require_cuda(wr, "wr", _BF16)
        if bias is not None:
            _require_cuda(bias, "bias", (torch.float32,))
        T = x.shape[0]
        if y is None:
            y = torch.empty((T, self.hidden), dtype=out_dtype, device=x.device)
        _require_cuda(y, "y", (torch.float32, torch.bfloat16))
        yd = DTYPE_F32 if y.dtype == torch.float32 else DTYPE_BF16
        if workspace is None:
            key = (x.device.index or 0, int(T))
            if accumulate and key not in self._wave_routed:
                raise ValueError("an accumulating wave needs a first wave (accumulate=False) of the "
                                 "same token count, after the last set_router_mode")
            ws = self._wave_ws.get(key)
            if ws is None:
                ws = torch.empty(max(256, self.workspace_size(T)), dtype=torch.uint8, device=x.device)
                self._wave_ws[key] = ws
        else:
            ws = workspace
        check(self._lib.moe_layer_forward_wave(self._h, x.data_ptr(), wr.data_ptr(), _ptr(bias), T,
                                               y.data_ptr(), yd, int(bool(accumulate)), ws.data_ptr(),
                                               ws.numel(), _stream(stream)), "moe_layer_forward_wave")
        if workspace is None and not accumulate:
            self._wave_routed.add((x.device.index or 0, int(T)))
        return y

    def set_stage_events(self, events: Optional[Sequence["torch.cuda.Event"]]) -> None:
        """Per-stage timing events (7 torch.cuda.Event with timing, or 9: the
        last two get the gate/up GEMM kernel's own start and end), or None."""
        if not events:
            check(self._lib.moe_layer_set_stage_events(self._h, None, 0), "set_stage_events")
            self._events = None
            return
        for ev in events:
            if ev.cuda_event == 0:      # torch creates the event lazily
                ev.record()
        arr = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
        check(self._lib.moe_layer_set_stage_events(self._h, arr, len(events)), "set_stage_events")
        self._events = list(events)

    def set_router_mode(self, mode: int) -> None:
        """ROUTER_AUTO, ROUTER_CANONICAL or ROUTER_MFMA for later calls (same
        routing bit for bit; the workspace size may change, so the cached
        workspaces are dropped)."""
        check(self._lib.moe_layer_set_router_mode(self._h, int(mode)), "set_router_mode")
        self._ws.clear()
        self._wave_ws.clear()
        self._wave_routed.clear()

    def close(self) -> None:
        if getattr(self, "_h", None):
            check(self._lib.moe_layer_destroy(self._h), "moe_layer_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

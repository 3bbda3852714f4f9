"""Online precision allocation for one layer ("Dynamic Expert Quantization for
Scalable Mixture-of-Experts Inference", abstract).  Each expert's usage is
counted from the layer's own routing, with an optional decay; the n most used
experts that fit a memory budget are held at the high precision tier and the
rest at the low one; version changes are repacked off the forward stream and
swapped in through the layer's stable expert handles, so a forward never sees
a half-written expert.

Every step is a library call: the grouping kernel keeps the decayed route
counts on the device (moe_layer_set_hotness), moe_plan_tiers makes the plan,
moe_quantize_pack_async repacks on a side stream, moe_layer_set_experts swaps
the handles on the forward stream.  This class only sequences the calls and
keeps blobs alive until no enqueued forward can still read them.
"""

from __future__ import annotations

from typing import Callable, Dict, List, Optional, Sequence, Tuple

import torch

from .api import (LAYOUT_GATE_UP, LAYOUT_PLAIN, Layer, packed_size, plan_tiers,
                  quantize_pack_async)


class DynaExq:
    """master(e) -> (w_gate [I,H], w_up [I,H], w_down [H,I]) device bf16
    tensors; blobs: the layer's current (tier, w13, w2) per expert."""

    def __init__(self, layer: Layer, master: Callable[[int], Tuple[torch.Tensor, ...]],
                 blobs: Sequence[Tuple[int, torch.Tensor, torch.Tensor]], budget_bytes: int,
                 hi_tier: int = 0, lo_tier: int = 2, decay: float = 1.0, device="cuda"):
        self.layer, self.master = layer, master
        self.E, self.H, self.I = layer.n_experts, layer.hidden, layer.inter
        self.blobs: List[Tuple[int, torch.Tensor, torch.Tensor]] = list(blobs)
        self.budget, self.hi, self.lo = int(budget_bytes), hi_tier, lo_tier
        self.hot = torch.zeros(self.E, dtype=torch.float32, device=device)
        layer.set_hotness(self.hot, decay)
        self.pack_stream = torch.cuda.Stream(device=device)      # default priority
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self._pending: Optional[Tuple[torch.cuda.Event, Dict[int, tuple]]] = None
        self._retired: List[Tuple[torch.cuda.Event, list]] = []

    def bytes_per_tier(self) -> List[int]:
        return [packed_size(t, 2 * self.I, self.H) + packed_size(t, self.H, self.I) for t in range(3)]

    def plan(self, stream=None) -> Tuple[List[int], int]:
        """Top-n plan from the current hotness (reads it after the forwards
        already enqueued on `stream`)."""
        s = torch.cuda.current_stream() if stream is None else stream
        with torch.cuda.stream(s):
            hot = self.hot.to("cpu", non_blocking=False)
        return plan_tiers(hot.tolist(), self.bytes_per_tier(), self.budget, self.hi, self.lo)

    def replan(self, stream=None) -> List[int]:
        """Plan, and repack every expert whose tier changes on the side stream.
        Returns the experts that change; apply() swaps them in later."""
        tiers, _ = self.plan(stream)
        changed = [e for e in range(self.E) if tiers[e] != self.blobs[e][0]]
        fresh: Dict[int, tuple] = {}
        with torch.cuda.stream(self.pack_stream):
            self.status.zero_()
            for e in changed:
                wg, wu, wd = self.master(e)
                w13 = torch.cat([wg, wu], dim=0).contiguous()
                t = tiers[e]
                b13 = torch.empty(packed_size(t, 2 * self.I, self.H), dtype=torch.uint8, device=wg.device)
                b2 = torch.empty(packed_size(t, self.H, self.I), dtype=torch.uint8, device=wg.device)
                quantize_pack_async(w13, t, LAYOUT_GATE_UP, b13, self.status, self.pack_stream)
                quantize_pack_async(wd.contiguous(), t, LAYOUT_PLAIN, b2, self.status, self.pack_stream)
                fresh[e] = (t, b13, b2, w13)
            ev = torch.cuda.Event()
            ev.record(self.pack_stream)
        self._pending = (ev, fresh)
        return changed

    def apply(self, stream=None, wait: bool = False) -> bool:
        """Swap in the repacked experts once their packs are done (or wait for
        them).  Forwards enqueued on `stream` after this call use the new
        versions; earlier ones keep the old ones, which stay alive until the
        stream has passed the swap."""
        if self._pending is None:
            return True
        ev, fresh = self._pending
        if not wait and not ev.query():
            return False
        ev.synchronize()
        if int(self.status.item()) != 0:
            raise RuntimeError("repack failed: weights out of range")
        s = torch.cuda.current_stream() if stream is None else stream
        old = []
        for e, (t, b13, b2, _) in sorted(fresh.items()):
            old.append(self.blobs[e])
            self.blobs[e] = (t, b13, b2)
            self.layer.set_experts(e, [(t, b13, b2)], stream=s)
        done = torch.cuda.Event()
        done.record(s)
        self._retired.append((done, old))
        self._retired = [(d, b) for d, b in self._retired if not d.query()]
        self._pending = None
        return True

    def tiers(self) -> List[int]:
        return [b[0] for b in self.blobs]

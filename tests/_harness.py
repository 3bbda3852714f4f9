"""Shared helpers of the GPU parity tests: build the same layer on both sides.

GPU side: master weights from the seeded generator, uploaded, quantized and
packed by the HIP library, run through the C ABI.  Oracle side: the same master
weights through the numpy oracle.  Nothing crosses from the GPU side into the
oracle's inputs.
"""

from __future__ import annotations

import functools
import sys
from typing import Callable, Dict, Optional

import numpy as np

import inputs
import oracle


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


# Parity margins of the session's layer comparisons: (case, path, error / RMS,
# tolerance).  tests/conftest.py prints them after the run, so a quiet
# (-q) log still records each case's margin.
MARGINS = []


def record_margin(case: str, path: int, err: float, tol: float) -> None:
    MARGINS.append((case, int(path), float(err), float(tol)))


def to_dev(a: np.ndarray, dev="cuda:0"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev_to_np(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def tile_boundary_tokens(routing, n_experts: int, tile_rows: int) -> np.ndarray:
    """Tokens owning the first and the last row of every M-tile of the grouped
    GEMMs: each expert's routes, in the oracle's grouped order, cut into tiles
    of tile_rows (the library's M-tiling, reported by moe_layer_plan).  Every
    (M-tile, column block) of both GEMMs then writes into a compared row."""
    off, srt = routing["offsets"], routing["sorted_routes"]
    k = routing["ids"].shape[1]
    pos = []
    for e in range(n_experts):
        for a in range(int(off[e]), int(off[e + 1]), tile_rows):
            pos += [a, min(a + tile_rows, int(off[e + 1])) - 1]
    return np.unique(srt[np.asarray(pos, dtype=np.int64)] // k)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return float(np.max(np.abs(y.astype(np.float64) - ref))) / rms


@functools.lru_cache(maxsize=None)
def _cached_expert(cfg, e):
    """Master weights of one expert, drawn once per test session."""
    return inputs.gen_expert(cfg, e)


class Setup:
    """A synthetic layer: inputs, tier table and an expert source."""

    def __init__(self, cid: int, T: Optional[int] = None, tiers: Optional[np.ndarray] = None,
                 source: Optional[Callable] = None, bias="config", cfg=None):
        self.cfg = inputs.get_config(cid) if cfg is None else cfg
        c = self.cfg
        self.T = c.default_tokens if T is None else T
        self.x = inputs.gen_tokens(c, self.T)
        self.wr = inputs.gen_router(c)
        self.bias = inputs.gen_bias(c) if isinstance(bias, str) else bias
        self.tiers = inputs.gen_tiers(c) if tiers is None else np.asarray(tiers, np.int32)
        self.source = source or functools.partial(_cached_expert, c)
        self.H, self.I, self.E, self.k = c.hidden, c.inter, c.n_experts, c.top_k

    def oracle_layer(self) -> oracle.OracleLayer:
        return oracle.OracleLayer(self.H, self.I, self.E, self.k, self.tiers, self.source)

    def gpu_layer(self, experts=None):
        """Pack every expert (or the given subset; the rest get expert 0's blobs)."""
        import torch
        from mixed_precision_moe_amd import Layer, pack_expert
        blobs: Dict[int, tuple] = {}
        todo = range(self.E) if experts is None else sorted(set(experts))
        for e in todo:
            wg, wu, wd = self.source(e)
            blobs[e] = pack_expert(to_dev(wg), to_dev(wu), to_dev(wd), int(self.tiers[e]))
        first = next(iter(blobs))
        handles = []
        for e in range(self.E):
            if e in blobs:
                handles.append((int(self.tiers[e]), *blobs[e]))
            else:
                handles.append((int(self.tiers[first]), *blobs[first]))
        torch.cuda.synchronize()
        return Layer(self.H, self.I, self.E, self.k, handles)

    def dev_inputs(self):
        x = to_dev(self.x)
        wr = to_dev(self.wr)
        b = None if self.bias is None else to_dev(self.bias)
        return x, wr, b

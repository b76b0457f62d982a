"""Verify-latency cost table: measured step latency over (batch, context, nodes).

"EAGLE-4 Technical Deepdive" (blog.fal.ai), "EAGLE-4 verification trees and
harness": before serving, a cost-aware tree harness calibrates once on the target
GPU a table of verification latency against batch size, context length and number
of candidates.  While drafting it compares, level by level, the gain in cumulative
acceptance probability with the measured marginal cost per token, and keeps
widening or deepening the tree only while that ratio stays above a threshold.

``bench.py --cost-table PREFIX`` measures the table for this library's step and
writes ``PREFIX.json``; this module reads it and answers the two questions the
harness asks: the latency of verifying N candidates, and the marginal cost of
adding more.  Between grid points the latency is piecewise linear in each axis
(attention grows linearly with context and nodes, sampling with nodes and batch);
outside the grid it extends the nearest segment linearly.
"""
from __future__ import annotations

import json

import numpy as np


def _segment(axis: np.ndarray, x: float):
    """(lower index, weight of the upper point) for linear interpolation along a sorted
    axis, extending the first or last segment beyond the ends."""
    if axis.size == 1:
        return 0, 0.0
    i = int(np.clip(np.searchsorted(axis, x, side="right") - 1, 0, axis.size - 2))
    return i, (x - axis[i]) / (axis[i + 1] - axis[i])


class CostTable:
    """Latency (microseconds) on a full grid of (batch, ctx, n_nodes) points."""

    def __init__(self, batch, ctx, n_nodes, latency_us, meta=None):
        self.axes = [np.asarray(a, np.float64) for a in (batch, ctx, n_nodes)]
        for a in self.axes:
            if a.size < 1 or np.any(np.diff(a) <= 0):
                raise ValueError("each axis must be strictly increasing")
        self.lat = np.asarray(latency_us, np.float64)
        if self.lat.shape != tuple(a.size for a in self.axes):
            raise ValueError("latency grid does not match the axes")
        self.meta = meta or {}

    @classmethod
    def from_rows(cls, rows, key="step_us", meta=None):
        """Build from measured rows ({"batch", "ctx", "n_nodes", key}); every grid point
        must be present exactly once."""
        axes = [sorted({int(r[k]) for r in rows}) for k in ("batch", "ctx", "n_nodes")]
        lat = np.full([len(a) for a in axes], np.nan)
        for r in rows:
            idx = tuple(a.index(int(r[k])) for a, k in zip(axes, ("batch", "ctx", "n_nodes")))
            if not np.isnan(lat[idx]):
                raise ValueError(f"duplicate grid point {idx}")
            lat[idx] = float(r[key])
        if np.isnan(lat).any():
            raise ValueError("the rows do not cover the full grid")
        return cls(*axes, lat, meta)

    @classmethod
    def load(cls, path, key="step_us"):
        with open(path) as f:
            doc = json.load(f)
        return cls.from_rows(doc["rows"], key=key, meta=doc.get("meta"))

    def latency_us(self, batch: float, ctx: float, n_nodes: float) -> float:
        """Multilinear interpolation (linear extension outside the grid)."""
        segs = [_segment(a, float(x)) for a, x in zip(self.axes, (batch, ctx, n_nodes))]
        out = 0.0
        for corner in range(8):
            w, idx = 1.0, []
            for dim, (i, t) in enumerate(segs):
                up = (corner >> dim) & 1
                if self.axes[dim].size == 1:
                    if up:
                        w = 0.0
                    idx.append(0)
                    continue
                w *= t if up else 1.0 - t
                idx.append(i + up)
            if w != 0.0:
                out += w * self.lat[tuple(idx)]
        return float(out)

    def marginal_us(self, batch: float, ctx: float, n_nodes: float, extra: int = 1) -> float:
        """Extra verify latency per added candidate when the tree grows from n_nodes to
        n_nodes + extra."""
        if extra <= 0:
            raise ValueError("extra must be positive")
        return (self.latency_us(batch, ctx, n_nodes + extra) - self.latency_us(batch, ctx, n_nodes)) / extra

    def worth_expanding(self, gain: float, batch: float, ctx: float, n_nodes: float, extra: int,
                        threshold: float) -> bool:
        """The harness's stopping rule for one proposed expansion of ``extra`` candidates
        that raises the expected number of accepted tokens by ``gain``: expand while
        gain per microsecond of marginal verify cost stays at or above ``threshold``.
        A non-positive marginal cost (flat latency at this size) always expands."""
        m = self.marginal_us(batch, ctx, n_nodes, extra) * extra
        if m <= 0.0:
            return True
        return gain / m >= threshold

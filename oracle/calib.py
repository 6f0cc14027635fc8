"""Static per-tensor activation scale by clipping-percentile search (test infrastructure only).

Passage followed: Q-ARVD page (aitrends.kr), Technical details: activations are
quantized per tensor, and the clipping percentile and the scaling factor are learned
during reconstruction.

Readings where the page is silent:

* the reconstruction objective is that of the activation quantizer alone, the mean
  squared error between the calibration tensor and its static quantize-dequantize
  (the page's frame-weighted layer-output loss needs a model and its frame
  sensitivities, which this layer does not have);
* the clip of percentile p is the order statistic of |x| at rank ceil(p/100 * N)
  (1-based, ascending), so p = 100 is the absolute maximum;
* candidate scale s = fl32(clip / Q); the static quantizer then uses r = fl32(1 / s),
  q = clamp(rne(fl32(x * r)), -Q, Q), deq = fl32(q * s) (as in ``quantizer``);
* MSE = sum over all elements of (x - deq)^2 / N, in float64;
* the search picks the candidate of smallest MSE; a tie keeps the earlier candidate in
  the caller's order; the default grid is ``GRID``.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import to_f32
from .quantizer import qmax, quantize_static

GRID = (100.0, 99.999, 99.99, 99.9, 99.8, 99.5, 99.0, 98.0, 97.0, 95.0, 90.0)


def rank_of(p: float, n: int) -> int:
    """1-based rank of the p-th percentile among n values."""
    return max(1, min(n, math.ceil(p / 100.0 * n)))


def percentile_clip(x_f32: np.ndarray, p: float) -> np.float32:
    a = np.sort(np.abs(np.asarray(x_f32, dtype=np.float32)).reshape(-1))
    return np.float32(a[rank_of(p, a.size) - 1])


def static_mse(x_f32: np.ndarray, s: np.float32, bits: int) -> float:
    x = np.asarray(x_f32, dtype=np.float32)
    q, s = quantize_static(x, qmax(bits), s)
    deq = (q.astype(np.float32) * np.float32(s)).astype(np.float32)
    err = x.astype(np.float64) - deq.astype(np.float64)
    return float(np.sum(err * err) / err.size)


def search(x_store: np.ndarray, dtype: str, bits: int, grid=GRID):
    """Returns dict(clips, scales, mse, best, scale) over the candidate percentiles."""
    x = to_f32(x_store, dtype)
    Q = np.float32(qmax(bits))
    clips = np.array([percentile_clip(x, p) for p in grid], dtype=np.float32)
    scales = (clips / Q).astype(np.float32)
    mse = np.array([static_mse(x, s, bits) for s in scales], dtype=np.float64)
    best = int(np.argmin(mse))  # first minimum
    return {"clips": clips, "scales": scales, "mse": mse, "best": best, "scale": np.float32(scales[best])}

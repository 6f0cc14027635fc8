"""DMPQ routing statistic of the oracle (test infrastructure only).

Follows the 6Bit-Diffusion page: Key Insights 1 (the previous timestep's relative
L1 distance between a transformer block's input and output, Gamma_{t-1}, tracks the
current quantization error linearly) and Methodology B.1, DMPQ (a block whose
Gamma_{t-1} exceeds a threshold routes its activations to INT8, otherwise to the
4-bit format).

Readings: Gamma = sum|y - x| / sum|x| in float64; the page's pre-learned linear model
is taken as the identity, so Gamma itself is compared with the threshold; "exceeds"
is strict, so Gamma equal to the threshold routes to the 4-bit side.
"""
from __future__ import annotations

import numpy as np


def relative_l1(x_f32: np.ndarray, y_f32: np.ndarray) -> float:
    x = np.asarray(x_f32, dtype=np.float64).reshape(-1)
    y = np.asarray(y_f32, dtype=np.float64).reshape(-1)
    den = np.sum(np.abs(x))
    return float(np.sum(np.abs(y - x)) / den) if den > 0 else float("inf")


def route_bits(gamma: float, threshold: float = 0.1, hi_bits: int = 8, lo_bits: int = 4) -> int:
    return hi_bits if gamma > threshold else lo_bits

"""Per-block runtime control of one denoising step (test infrastructure only).

Passages followed: 6Bit-Diffusion page (gist.science, arXiv 2603.18742):

* Key Insights 2 and Methodology B.2, TDC: the residual deltas of a transformer block
  are very similar across adjacent timesteps, so from the difference E_t between the
  deltas of the two previous timesteps a stable block skips its computation and reuses
  its cached delta; to stop drift, computation is forced once an accumulated error
  threshold is exceeded or a maximum number of consecutive skips is reached.
* Methodology B.3, PDR: a layer whose input has a high outlier ratio is computed at
  FP16/BF16; the first computed step after a skip has no routing information, so it is
  forced to INT8.
* Key Insights 1 and Methodology B.1, DMPQ: otherwise Gamma_{t-1} routes the activations
  (``route.route_bits``).

Readings where the page gives no formula:

* a block's delta is its output minus its input at a computed timestep; the caller keeps
  the last two, d1 (newer) and d2 (older);
* E = sum|d1 - d2| / sum|d2| in float64, the relative-L1 form of Gamma; E = 0 when the
  numerator is 0 (identical deltas) and +inf when only the denominator is 0;
* stable means E does not exceed the skip threshold (E <= tau_skip), mirroring the
  strict "exceeds" of the route;
* the accumulated error is the sum of E over the current run of consecutive skips; a
  skip needs that sum, including the current E, not to exceed tau_drift, and fewer than
  max_skips skips before it; without two cached deltas the block computes;
* outlier ratio = outlier channels of the block input (the flag rule of ``detect``) /
  its channel count; high means above rho (strict);
* on a computed step the precedence is: high outlier ratio -> unquantized (16), then
  first step after a skip -> 8, then the Gamma route; an unknown Gamma (no previous
  input/output pair) takes the high width;
* result codes: skip flag, and bits = 0 when skipped, 16 for unquantized, else the
  activation width; the state (consecutive skips, accumulated error) is reset on a
  computed step.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .route import route_bits


@dataclass
class Params:
    skip_threshold: float = 0.05
    drift_threshold: float = 0.15
    max_skips: int = 3
    route_threshold: float = 0.1
    bits_hi: int = 8
    bits_lo: int = 4
    outlier_ratio_max: float = 0.01


@dataclass
class State:
    skips: int = 0
    drift: float = 0.0


def stability(d1_f32: np.ndarray, d2_f32: np.ndarray) -> float:
    """E = sum|d1 - d2| / sum|d2| (float64)."""
    a = np.asarray(d1_f32, dtype=np.float64).reshape(-1)
    b = np.asarray(d2_f32, dtype=np.float64).reshape(-1)
    num = float(np.sum(np.abs(a - b)))
    den = float(np.sum(np.abs(b)))
    if num == 0.0:
        return 0.0
    return num / den if den > 0.0 else float("inf")


def step(state: State, p: Params, e: float | None = None, gamma: float | None = None,
         n_out: int | None = None, channels: int | None = None):
    """One decision.  Returns (skip, bits, new State)."""
    if e is not None and state.skips < p.max_skips and e <= p.skip_threshold \
            and state.drift + e <= p.drift_threshold:
        return True, 0, State(state.skips + 1, state.drift + e)
    if n_out is not None and channels and n_out / channels > p.outlier_ratio_max:
        bits = 16
    elif state.skips > 0:
        bits = 8
    elif gamma is None:
        bits = p.bits_hi
    else:
        bits = route_bits(gamma, p.route_threshold, p.bits_hi, p.bits_lo)
    return False, bits, State(0, 0.0)

"""Outlier input-channel detection of the oracle (test infrastructure only).

Follows the Q-ARVD page (Methodology, "Outlier-aware Adaptive Dual-scale
Quantization", and its formula paragraph): take the L2 norm v_i of every input
channel, the median v~ of those norms and their median absolute deviation MAD,
form the modified z-score M_i = (v_i - v~) / MAD, and flag channel i when M_i
exceeds the threshold tau AND v_i exceeds the minimum magnitude alpha * v~.

Readings where the page is silent or garbled:

* the garbled inequality "v_i > v~ + (tau/MAD) MAD" is read as v_i > v~ + tau * MAD,
  i.e. M_i > tau (the literal form would compare a norm with tau itself);
* both comparisons are strict;
* ``kfac`` multiplies M_i; 1.0 is the page's formula, 0.6745 the textbook
  Iglewicz-Hoaglin variant;
* an even-length median is the mean of the two middle values (NumPy's);
* MAD = 0: M_i = +inf where v_i > v~, else 0.
"""
from __future__ import annotations

import numpy as np


def channel_l2_norms(x_f32: np.ndarray) -> np.ndarray:
    """v_k = sqrt(sum_r x[r, k]^2) in float64; channels are the columns of x."""
    x64 = np.asarray(x_f32, dtype=np.float64)
    return np.sqrt(np.sum(x64 * x64, axis=0))


def modified_z(v: np.ndarray, kfac: float = 1.0):
    v = np.asarray(v, dtype=np.float64)
    med = np.median(v)
    mad = np.median(np.abs(v - med))
    if mad == 0.0:
        m = np.where(v > med, np.inf, 0.0)
    else:
        m = kfac * (v - med) / mad
    return m, med, mad


def flag_outliers(v: np.ndarray, tau: float = 3.5, alpha: float = 2.0, kfac: float = 1.0):
    """Returns (mask bool[K], outlier indices ascending, M, median, MAD)."""
    m, med, mad = modified_z(v, kfac)
    mask = (m > tau) & (np.asarray(v, dtype=np.float64) > alpha * med)
    return mask, np.flatnonzero(mask).astype(np.int32), m, med, mad


def detect_outliers(x_f32: np.ndarray, tau: float = 3.5, alpha: float = 2.0, kfac: float = 1.0):
    """Column norms of x, then the flag rule.  Returns (mask, idx, norms, M, median, MAD)."""
    v = channel_l2_norms(x_f32)
    mask, idx, m, med, mad = flag_outliers(v, tau, alpha, kfac)
    return mask, idx, v, m, med, mad


def decision_margin(v: np.ndarray, tau: float = 3.5, alpha: float = 2.0, kfac: float = 1.0) -> float:
    """Smallest relative distance of any channel from either threshold.

    A margin above the float64 summation-order error of the norms means every
    correct implementation, whatever its reduction order, flags the same set.
    """
    v = np.asarray(v, dtype=np.float64)
    m, med, mad = modified_z(v, kfac)
    d1 = np.abs(v - alpha * med) / max(alpha * med, 1e-300)
    if mad == 0.0:
        return float(np.min(d1))
    thr = med + tau * mad / kfac
    d2 = np.abs(v - thr) / max(abs(thr), 1e-300)
    return float(min(np.min(d1), np.min(d2)))

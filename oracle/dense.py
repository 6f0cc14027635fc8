"""The unquantized linear layer of the precision override (test infrastructure only).

Passage followed: 6Bit-Diffusion page (gist.science, arXiv 2603.18742), Methodology B.3
(PDR): a layer whose input has a high outlier ratio is computed in FP16/BF16 instead of
a quantized format (the step control returns precision code 16 for it).

Readings where the page is silent:

* Y = X . W^T with X [M x K] and W [N x K] in the same 16-bit storage type (fp16 or
  bf16), no bias, no activation function;
* the products of 16-bit values are exact in float32 and the sums are accumulated in
  float32 (the matrix cores' accumulator type); the reference value is the exact sum
  (float64 here: every product of two 16-bit values and every partial sum over at most
  2^20 terms of them is exact or within 2^-53 relative in float64) rounded once to
  float32 and then, round to nearest even, to the output type;
* a float32 accumulation in any order differs from the exact sum by at most
  (K + 2) * 2^-24 * sum_k |x_k w_k| (the recursive-summation bound), which is the
  tolerance the device result is held to (plus half an output ulp for 16-bit outputs).
"""
from __future__ import annotations

import numpy as np

from .numerics import from_f32, to_f32


def exact(x_store, dtype: str, w_store, wdtype: str | None = None) -> np.ndarray:
    """sum_k x[m, k] w[n, k] in float64 for the decoded 16-bit inputs."""
    x = to_f32(x_store, dtype).astype(np.float64)
    w = to_f32(w_store, wdtype or dtype).astype(np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return x @ w.T


def magnitude(x_store, dtype: str, w_store, wdtype: str | None = None) -> np.ndarray:
    """sum_k |x[m, k] w[n, k]|: the scale of the float32 summation bound."""
    x = np.abs(to_f32(x_store, dtype).astype(np.float64))
    w = np.abs(to_f32(w_store, wdtype or dtype).astype(np.float64))
    return x @ w.T


def bound(mag: np.ndarray, k: int) -> np.ndarray:
    """Largest difference between a float32 accumulation (any order) and the exact sum."""
    return (k + 2) * 2.0 ** -24 * mag


def forward(x_store, dtype: str, w_store, out_dtype: str | None = None):
    """Returns (y_exact float64, y_f32 = fl32(y_exact), y_store in out_dtype)."""
    y = exact(x_store, dtype, w_store)
    y32 = y.astype(np.float32)
    return y, y32, from_f32(y32, out_dtype or dtype)

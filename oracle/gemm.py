"""Exact integer GEMM and dequantization epilogue of the oracle (test infrastructure only).

Follows the Q-ARVD page (Technical details): activation quantization is followed by a
GEMM with dequantization; activations carry a per-tensor (here also per-token) scale
and weights a per-channel scale, so Y[m, n] = s_a[m] * s_w[n] * sum_k qa[m, k] qw[n, k].
With dual scale (Q-ARVD page, Methodology) the sum splits over the two K partitions,
each with its own pair of scales.

Readings where the page is silent (the epilogue arithmetic):

* acc_P[m, n] = sum over partition P of qa * qw, exact in int32;
* in float32, with no fused multiply-add: f = fl32(acc), t = fl32(s_a[m] * s_w[n]),
  y = fl32(f * t); with two partitions y = fl32(y_0 + y_1);
* then round-to-nearest-even to the output dtype; no bias, no activation function.
"""
from __future__ import annotations

import numpy as np

from .numerics import from_f32


def int_gemm(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc = qa @ qw^T exactly, as int32.

    Computed as a float64 matrix product: every partial sum is an integer of
    magnitude below 2^53, so the result is exact whatever order or FMA the BLAS uses.
    """
    qa = np.asarray(qa, dtype=np.int8)
    qw = np.asarray(qw, dtype=np.int8)
    k = qa.shape[1]
    if qw.shape[1] != k:
        raise ValueError("K mismatch")
    bound = k * int(np.max(np.abs(qa), initial=0)) * int(np.max(np.abs(qw), initial=0))
    if bound >= 2 ** 53:
        raise ValueError("partial sums may not be exact in float64")
    acc = qa.astype(np.float64) @ qw.astype(np.float64).T
    if acc.size and np.max(np.abs(acc)) >= 2 ** 31:
        raise OverflowError("accumulator exceeds int32")
    return acc.astype(np.int64).astype(np.int32)


def partition_bounds(kp: int, k0: int):
    """[(0, k0), (k0, kp)] for two partitions, [(0, kp)] for one (k0 == kp)."""
    return [(0, kp)] if k0 >= kp else [(0, k0), (k0, kp)]


def accumulators(qa: np.ndarray, qw: np.ndarray, k0: int):
    """Exact int32 accumulators per partition, list of [M x N]."""
    kp = qa.shape[1]
    return [int_gemm(qa[:, a:b], qw[:, a:b]) for a, b in partition_bounds(kp, k0)]


def _scale_col(s: np.ndarray, p: int, n_parts: int) -> np.ndarray:
    s = np.asarray(s, dtype=np.float32)
    if n_parts == 1:
        return s.reshape(-1)
    return s.reshape(-1, n_parts)[:, p]


def epilogue(accs, sa: np.ndarray, sb: np.ndarray, sa_per_token: bool, out_dtype: str):
    """Dequantize the partition accumulators: returns (y_f32, y_store)."""
    n_parts = len(accs)
    y = None
    for p, acc in enumerate(accs):
        m, n = acc.shape
        sa_p = _scale_col(sa, p, n_parts)
        if not sa_per_token:
            sa_p = np.full(m, sa_p[0], dtype=np.float32)
        sb_p = _scale_col(sb, p, n_parts)
        f = acc.astype(np.float32)
        t = (sa_p[:, None] * sb_p[None, :]).astype(np.float32)
        yp = (f * t).astype(np.float32)
        y = yp if y is None else (y + yp).astype(np.float32)
    return y, from_f32(y, out_dtype)


def qgemm_dequant(qa, sa, sa_per_token, qw, sb, k0, out_dtype):
    """Accumulators and dequantized output: returns (accs, y_f32, y_store)."""
    accs = accumulators(qa, qw, k0)
    y, ys = epilogue(accs, sa, sb, sa_per_token, out_dtype)
    return accs, y, ys

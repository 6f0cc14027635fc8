"""Activation decomposition: residual re-quantization of selected tokens (test infrastructure only).

Passage followed: SemanticDialect page (gist.science, arXiv 2603.02883), Methodology
2.2, activation decomposition.  In quantization-sensitive layers the activation is
quantized, the quantization error left over (the residual) is quantized once more, and
its contribution is added back to the layer output; to keep the bit budget, only
selected (salient) tokens are decomposed.

Readings where the page is silent:

* the first quantizer is the path's per-token quantizer (``quantizer.quant_act`` with
  gran="token", no rotation, no dual scale), bit width b1;
* the dequantized value is deq = fl32(q1 * s1) and the residual r = fl32(x - deq), both
  in float32;
* the residual is quantized by the same per-token absmax quantizer with its own bit
  width b2 and its own scale s2 (r2 = fl32(Q2 / max|r|), s2 = fl32(max|r| / Q2));
* the salient tokens are given by the caller as distinct row indices (the page picks
  them from attention scores, which this layer does not have);
* output: a decomposed row m has two accumulators, acc1 = q1 . qw and acc2 = q2 . qw,
  and y = fl32(fl32(acc1 * fl32(s1 * sw)) + fl32(acc2 * fl32(s2 * sw))), rounded once to
  the output type (the two-partition epilogue of ``gemm.epilogue``); other rows are
  exactly those of the layer without decomposition.
"""
from __future__ import annotations

import numpy as np

from .gemm import epilogue, int_gemm
from .numerics import from_f32, to_f32
from .quantizer import qmax, quant_act, quantize_groups


def residual_quant(x_store: np.ndarray, dtype: str, bits1: int, bits2: int, rows):
    """Residual codes of the listed rows: returns (q2 int8 [R x K], s2 float32 [R])."""
    rows = np.asarray(rows, dtype=np.int64)
    x = to_f32(x_store, dtype)[rows]
    q1, s1 = quantize_groups(x, qmax(bits1), axis=1)
    deq = (q1.astype(np.float32) * s1.astype(np.float32)[:, None]).astype(np.float32)
    r = (x - deq).astype(np.float32)
    return quantize_groups(r, qmax(bits2), axis=1)


def forward(x_store, dtype: str, bits1: int, bits2: int, rows, w_codes, w_scales, out_dtype: str):
    """The layer with decomposition of ``rows``: returns dict of intermediates and outputs."""
    rows = np.asarray(rows, dtype=np.int64)
    q1, s1 = quant_act(x_store, dtype, bits1, "token")
    q2, s2 = residual_quant(x_store, dtype, bits1, bits2, rows)
    acc1 = int_gemm(q1, w_codes)
    y, _ = epilogue([acc1], s1, w_scales, True, "fp32")
    if len(rows):
        acc2 = int_gemm(q2, w_codes)
        sa = np.stack([s1[rows], s2], axis=1).astype(np.float32)
        sb = np.stack([w_scales, w_scales], axis=1).astype(np.float32)
        y_rows, _ = epilogue([acc1[rows], acc2], sa, sb, True, "fp32")
        y = np.array(y, copy=True)
        y[rows] = y_rows
    else:
        acc2 = np.zeros((0, w_codes.shape[0]), dtype=np.int32)
    return {"q1": q1, "s1": s1, "q2": q2, "s2": s2, "acc1": acc1, "acc2": acc2,
            "y": y, "y_store": from_f32(y, out_dtype)}

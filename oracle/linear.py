"""The whole quantized linear layer, chaining the oracle's steps (test infrastructure only).

Order of operations (Q-ARVD page, Methodology and Technical details; 6Bit-Diffusion
page, Methodology B.1):

1. offline: optional outlier detection on a calibration tensor, then per-channel
   weight packing (optionally pre-rotated by the block Hadamard transform);
2. online: activation quantization (per tensor or per token, optionally rotated, or
   split into normal/outlier partitions);
3. integer GEMM over each K partition and the dequantization epilogue.
"""
from __future__ import annotations

import numpy as np

from . import detect as _detect
from . import gemm as _gemm
from . import quantizer as _q
from .numerics import to_f32


def prepare_weights(w_store, dtype, w_bits, had_block=0, out_idx=None):
    return _q.pack_weights(w_store, dtype, w_bits, had_block, out_idx)


def forward(x_store, dtype, a_bits, gran, w_codes, w_scales, had_block=0, out_idx=None,
            out_dtype=None, static_scale=None):
    """Returns a dict with codes, scales, accumulators and the output (float32 and stored)."""
    out_dtype = out_dtype or dtype
    qa, sa = _q.quant_act(x_store, dtype, a_bits, gran, had_block, out_idx, static_scale)
    k = np.asarray(x_store).shape[1]
    k0 = k if out_idx is not None and len(out_idx) else qa.shape[1]
    accs, y, ys = _gemm.qgemm_dequant(qa, sa, gran == "token", w_codes, w_scales, k0, out_dtype)
    return dict(qa=qa, sa=sa, accs=accs, y=y, y_store=ys, k0=k0)


def detect_on(t_store, dtype, tau=3.5, alpha=2.0, kfac=1.0):
    mask, idx, v, m, med, mad = _detect.detect_outliers(to_f32(t_store, dtype), tau, alpha, kfac)
    return dict(mask=mask, idx=idx, norms=v, z=m, median=med, mad=mad)

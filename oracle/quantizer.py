"""Symmetric absmax quantizer, dual-scale split and packing (test infrastructure only).

Passages followed:

* Q-ARVD page, Methodology and Technical details: activations are quantized per
  tensor, weights per (output) channel, and outlier input channels get their own
  quantizer: Q_dual(W) = [Q_outlier(W_outliers) | Q_normal(W_normal)].
* 6Bit-Diffusion page, Methodology B.1 (DMPQ): weights are quantized offline to a
  4-bit format; activations are routed to INT8 or 4-bit per block.
* S2Q-VDiT page: the W4A6 setting (6-bit activations).

Readings where the pages are silent:

* quantizer: symmetric, no zero-point, restricted range [-Q, Q] with Q = 2^(b-1) - 1;
  scale from the group's absolute maximum a; r = fl32(Q / a), s = fl32(a / Q),
  q = clamp(rne(fl32(x * r)), -Q, Q); a = 0 (or a non-finite r) gives s = 0 and q = 0;
* a static per-tensor scale s gives r = fl32(1 / s);
* groups: per tensor = the whole tensor, per token = one row of X, per channel = one
  row of W (each taken separately in each partition);
* dual scale splits the input channels (K) of both operands into two partitions:
  partition 0 holds the normal channels in place (outlier positions hold code 0),
  partition 1 holds the outlier channels gathered in ascending order and zero-padded
  to a multiple of 64; codes are [rows x (K + pad64(n_out))], scales [rows x 2];
* 6-bit and 4-bit activation codes are stored one per int8; 4-bit weights are packed
  two per byte, low nibble = even k: byte j = (q[2j] & 0xF) | ((q[2j+1] & 0xF) << 4);
* with the block Hadamard rotation both operands are rotated unnormalized (z = H x);
  the weight scale carries the exact factor 1/block (2^-7 for 128-point blocks), so
  the product equals that of the normalized rotation with no irrational constant.
"""
from __future__ import annotations

import numpy as np

from .fwht import fwht_blocks
from .numerics import to_f32

K_ALIGN = 64


def qmax(bits: int) -> int:
    if bits not in (4, 6, 8):
        raise ValueError("bits must be 4, 6 or 8")
    return (1 << (bits - 1)) - 1


def part_len(n_out: int) -> int:
    """Length of the outlier partition: n_out rounded up to a multiple of 64."""
    return ((n_out + K_ALIGN - 1) // K_ALIGN) * K_ALIGN


def packed_k(k: int, n_out: int) -> int:
    return k + part_len(n_out) if n_out > 0 else k


def _codes_from(x: np.ndarray, r: np.ndarray, Q: int) -> np.ndarray:
    t = (x * r).astype(np.float32)
    return np.clip(np.rint(t), -Q, Q).astype(np.int8)


def quantize_groups(x: np.ndarray, Q: int, axis=None):
    """Dynamic absmax quantization of float32 ``x``.

    ``axis=None``: one group (the whole array), else one group per index of the
    remaining axis (axis=1 on a 2-D array: one group per row).  Returns (codes int8, s float32).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=axis, keepdims=True).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = (np.float32(Q) / a).astype(np.float32)
        s = (a / np.float32(Q)).astype(np.float32)
    bad = (a == 0) | ~np.isfinite(r)
    r = np.where(bad, np.float32(0), r).astype(np.float32)
    s = np.where(bad, np.float32(0), s).astype(np.float32)
    codes = _codes_from(x, r, Q)
    return codes, (s.reshape(()) if axis is None else np.squeeze(s, axis=axis))


def quantize_static(x: np.ndarray, Q: int, s: float):
    """Static-scale quantization: r = fl32(1 / s)."""
    s = np.float32(s)
    with np.errstate(divide="ignore"):
        r = np.float32(np.float32(1.0) / s)
    if s == 0 or not np.isfinite(r):
        return np.zeros(np.shape(x), dtype=np.int8), np.float32(0)
    return _codes_from(np.asarray(x, dtype=np.float32), r, Q), s


def split_dual(x: np.ndarray, out_idx: np.ndarray):
    """Partition 0: x with outlier columns set to 0; partition 1: outlier columns, zero-padded."""
    out_idx = np.asarray(out_idx, dtype=np.int64)
    normal = np.array(x, dtype=np.float32, copy=True)
    normal[:, out_idx] = 0.0
    outl = np.zeros((x.shape[0], part_len(len(out_idx))), dtype=np.float32)
    outl[:, : len(out_idx)] = x[:, out_idx]
    return normal, outl


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, low nibble = even k."""
    c = np.asarray(codes, dtype=np.int8)
    if c.shape[-1] % 2:
        raise ValueError("even number of codes required")
    lo = (c[..., 0::2].astype(np.int16) & 0xF).astype(np.uint8)
    hi = (c[..., 1::2].astype(np.int16) & 0xF).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def quant_act(x_store: np.ndarray, dtype: str, bits: int, gran: str = "token", had_block: int = 0,
              out_idx=None, static_scale=None):
    """Online activation quantization.

    gran: "token" (one scale per row), "tensor" (dynamic, one scale per partition) or
    "static" (``static_scale`` per partition).  Returns (codes int8 [M x kp], scales).
    Scales: token -> [M] or [M, 2]; tensor/static -> [1] or [2].
    """
    Q = qmax(bits)
    x = to_f32(x_store, dtype)
    if had_block:
        if out_idx is not None and len(out_idx):
            raise ValueError("Hadamard rotation and dual scale are not combined")
        x = fwht_blocks(x, had_block)
    parts = [x] if out_idx is None or len(out_idx) == 0 else list(split_dual(x, out_idx))
    codes, scales = [], []
    for p_i, p in enumerate(parts):
        if gran == "token":
            c, s = quantize_groups(p, Q, axis=1)
        elif gran == "tensor":
            c, s = quantize_groups(p, Q, axis=None)
            s = np.array([s], dtype=np.float32)
        elif gran == "static":
            c, s = quantize_static(p, Q, np.asarray(static_scale, dtype=np.float32).reshape(-1)[p_i])
            s = np.array([s], dtype=np.float32)
        else:
            raise ValueError(gran)
        codes.append(c)
        scales.append(np.asarray(s, dtype=np.float32))
    codes = np.concatenate(codes, axis=1)
    if len(parts) == 1:
        return codes, scales[0]
    if gran == "token":
        return codes, np.stack(scales, axis=1).astype(np.float32)
    return codes, np.concatenate(scales).astype(np.float32)


def pack_weights(w_store: np.ndarray, dtype: str, bits: int, had_block: int = 0, out_idx=None):
    """Offline per-output-channel weight quantization.

    Returns (codes, packed, scales): ``codes`` int8 [N x kp] (always), ``packed`` the
    stored form (int8 codes for 8 bits, uint8 [N x kp/2] nibbles for 4 bits) and
    ``scales`` float32 [N] or [N, 2].
    """
    if bits not in (4, 8):
        raise ValueError("weights are 4 or 8 bits")
    Q = qmax(bits)
    w = to_f32(w_store, dtype)
    fold = np.float32(1.0)
    if had_block:
        if out_idx is not None and len(out_idx):
            raise ValueError("Hadamard rotation and dual scale are not combined")
        w = fwht_blocks(w, had_block)
        fold = np.float32(1.0 / had_block)  # exact power of two
    parts = [w] if out_idx is None or len(out_idx) == 0 else list(split_dual(w, out_idx))
    codes, scales = [], []
    for p in parts:
        c, s = quantize_groups(p, Q, axis=1)
        codes.append(c)
        scales.append((np.asarray(s, dtype=np.float32) * fold).astype(np.float32))
    codes = np.concatenate(codes, axis=1)
    scales = scales[0] if len(parts) == 1 else np.stack(scales, axis=1).astype(np.float32)
    packed = pack_int4(codes) if bits == 4 else codes
    return codes, packed, scales

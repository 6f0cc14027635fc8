"""MX (microscaling) block formats and their GEMM (test infrastructure only).

Passages followed: 6Bit-Diffusion page (gist.science, arXiv 2603.18742), Introduction
(hardware compatibility) and Methodology B.1: recent GPUs dropped INT4 in favour of a
4-bit floating-point block format, and DMPQ routes activations between INT8 and that
format, with weights in it offline.  On gfx950 the corresponding hardware format is the
OCP Microscaling (MX) family, consumed by the scaled MFMA with E8M0 block scales; this
module states that family's conversion as published in the OCP MX v1.0 specification:

* a block is 32 consecutive elements of a row along K, with one shared scale
  X = 2^e stored as an E8M0 byte (code = e + 127, e in [-127, 127]);
* e = floor(log2(max |v|)) - emax_elem, where emax_elem is the exponent of the element
  format's largest normal value (2 for FP4 E2M1 and FP6 E2M3);
* each element is v / X rounded to the nearest element value, ties to even, and
  clamped to the largest magnitude (6 for E2M1, 7.5 for E2M3);
* element formats: E2M1 = sign, 2 exponent bits (bias 1), 1 mantissa bit, values
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}; E2M3 = sign, 2 exponent bits (bias 1), 3 mantissa bits,
  values k/8 for k < 8 and (1 + m/8) * 2^(e-1) up to 7.5; no infinities or NaNs.

Readings where the specification leaves a choice:

* a block whose maximum is 0 gets e = -127 (code 0) and zero elements;
* e is clamped to [-127, 127]; a negative value that rounds to zero keeps its sign
  (code with the sign bit set);
* packing along K: element p of a row occupies bits [w*p, w*p + w) of the row's
  little-endian bit string (w = 4 or 6), so FP4 puts element 2j in the low nibble of
  byte j; the scales of a row are its K/32 E8M0 bytes in order;
* the GEMM result is the exact sum over K of the decoded products (float64 here; every
  product and block sum of these formats is exactly representable), rounded once to
  float32 and then to the output type; the hardware accumulates in float32, so the
  device result is compared within a derived tolerance, the codes bit for bit.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32

# name -> (exponent bits, mantissa bits, bias, emax_elem, largest magnitude)
FORMATS = {
    "fp4": (2, 1, 1, 2, 6.0),   # E2M1
    "fp6": (2, 3, 1, 2, 7.5),   # E2M3
}


def bits_of(fmt: str) -> int:
    e, m, _, _, _ = FORMATS[fmt]
    return 1 + e + m


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exactly (from the float64 exponent)."""
    _, ex = np.frexp(a)
    return ex.astype(np.int64) - 1


def block_scales(x: np.ndarray, fmt: str) -> np.ndarray:
    """E8M0 exponents e (int64 [rows x K/32]) of float32 x [rows x K]."""
    _, _, _, emax, _ = FORMATS[fmt]
    rows, k = x.shape
    amax = np.abs(x.astype(np.float64)).reshape(rows, k // BLOCK, BLOCK).max(axis=2)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = _floor_log2(amax[nz]) - emax
    return np.clip(e, -127, 127)


def encode(t: np.ndarray, fmt: str) -> np.ndarray:
    """Element codes of scaled values t (round to nearest even, saturate)."""
    E, M, bias, _, vmax = FORMATS[fmt]
    t = np.asarray(t, dtype=np.float64)
    sign = np.signbit(t).astype(np.int64)
    a = np.minimum(np.abs(t), vmax)
    # exponent of the binade (the subnormal binade shares the smallest normal exponent)
    e = np.zeros(a.shape, dtype=np.int64)
    big = a >= 2.0 ** (1 - bias)
    e[big] = _floor_log2(a[big])
    e = np.maximum(e, 1 - bias)
    step = np.ldexp(1.0, e - M)
    n = np.rint(a / step).astype(np.int64)  # rint: ties to even
    mag = (e - (1 - bias)) * (1 << M) + n     # codes grow monotonically with the value
    return (sign << (E + M)) | mag


def decode(code: np.ndarray, fmt: str) -> np.ndarray:
    """Values of element codes (float64)."""
    E, M, bias, _, _ = FORMATS[fmt]
    code = np.asarray(code, dtype=np.int64)
    s = np.where((code >> (E + M)) & 1, -1.0, 1.0)
    ef = (code >> M) & ((1 << E) - 1)
    m = code & ((1 << M) - 1)
    sub = np.ldexp(m / 2.0 ** M, 1 - bias)
    nrm = np.ldexp(1.0 + m / 2.0 ** M, ef - bias)
    return s * np.where(ef == 0, sub, nrm)


def quantize(x: np.ndarray, fmt: str):
    """MX quantization of float32 x [rows x K]: returns (element codes int64, E8M0 bytes uint8)."""
    x = np.asarray(x, dtype=np.float32)
    rows, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    e = block_scales(x, fmt)
    t = x.astype(np.float64) * np.ldexp(1.0, -np.repeat(e, BLOCK, axis=1))
    return encode(t, fmt), (e + 127).astype(np.uint8)


def quantize_rotated(x: np.ndarray, fmt: str, exp_offset: int = 0, block: int = 128):
    """MX quantization of the rows of float32 x rotated by the online block Hadamard
    transform (6Bit-Diffusion page, Methodology B.1: the 4-bit floating-point route
    rotates the activations by 128-point Hadamard blocks before quantizing them).

    z = the unnormalized block FWHT of each row (fwht.fwht_blocks: float32 butterflies,
    ascending distances); t = fl32(z * 2^exp_offset); then quantize(t).  Activations take
    exp_offset = 0.  Weights pre-rotated offline take exp_offset = -7: their decoded values
    approximate z_w / 128, so that products with unnormalized rotated activations give
    sum_k z_x z_w / 128 = sum_k x w (H H^T = 128 I), with no irrational 1/sqrt(128) and no
    extra operation in the GEMM.  Scaling by a power of two leaves the element codes
    unchanged and moves the block exponents by exp_offset, unless it leaves the float32
    normal range.
    """
    from .fwht import fwht_blocks
    z = fwht_blocks(np.asarray(x, dtype=np.float32), block)
    t = (z * np.float32(2.0 ** exp_offset)).astype(np.float32)
    return quantize(t, fmt)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    e = scales.astype(np.int64) - 127
    return decode(codes, fmt) * np.ldexp(1.0, np.repeat(e, BLOCK, axis=1))


def pack(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Bit-pack element codes along K: [rows x K] -> uint8 [rows x K*w/8]."""
    w = bits_of(fmt)
    codes = np.asarray(codes, dtype=np.uint64) & np.uint64((1 << w) - 1)
    rows, k = codes.shape
    out = np.zeros((rows, k * w // 8), dtype=np.uint8)
    for p in range(k):
        bit = w * p
        for b in range(w):
            byte, off = divmod(bit + b, 8)
            out[:, byte] |= (((codes[:, p] >> np.uint64(b)) & np.uint64(1)).astype(np.uint8) << np.uint8(off))
    return out


def unpack(packed: np.ndarray, k: int, fmt: str) -> np.ndarray:
    w = bits_of(fmt)
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.zeros((packed.shape[0], k), dtype=np.int64)
    for p in range(k):
        for b in range(w):
            byte, off = divmod(w * p + b, 8)
            codes[:, p] |= ((packed[:, byte] >> off) & 1).astype(np.int64) << b
    return codes


def gemm(a_codes, a_scales, fa: str, b_codes, b_scales, fb: str) -> np.ndarray:
    """Exact Y = deq(A) . deq(B)^T in float64 ([M x K] and [N x K] codes, [rows x K/32] scales)."""
    return dequantize(a_codes, a_scales, fa) @ dequantize(b_codes, b_scales, fb).T


def forward(x_store, dtype: str, fa: str, w_store, wdtype: str, fb: str, out_dtype: str):
    """The MX linear layer: quantize X and W, exact GEMM, one rounding to float32, then to out_dtype."""
    from .numerics import from_f32, to_f32
    ac, asc = quantize(to_f32(x_store, dtype), fa)
    bc, bsc = quantize(to_f32(w_store, wdtype), fb)
    y = gemm(ac, asc, fa, bc, bsc, fb).astype(np.float32)
    return {"a_codes": ac, "a_scales": asc, "b_codes": bc, "b_scales": bsc, "y": y, "y_store": from_f32(y, out_dtype)}

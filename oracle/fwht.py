"""Block Hadamard rotation of the oracle (test infrastructure only).

Follows the 6Bit-Diffusion page (Methodology, B.1 DMPQ), which applies an online
block Hadamard transform to activations to spread outliers before quantizing.  The
page gives neither block size, ordering nor normalization; the readings used here:

* blocks of ``block`` (128) contiguous elements along each row;
* the Sylvester (natural-order) Hadamard matrix H[i][j] = (-1)^popcount(i & j),
  applied by in-place butterflies in float32, stages in ascending distance
  h = 1, 2, 4, ..., block/2, each pair (i, i + h) with bit h of i clear becoming
  (z[i] + z[i+h], z[i] - z[i+h]);
* the unnormalized result z = H x is what the fused quantizer sees; the standalone
  transform can also return z * fl32(1/sqrt(block)).
"""
from __future__ import annotations

import numpy as np


def fwht_blocks(x: np.ndarray, block: int = 128) -> np.ndarray:
    """Unnormalized block FWHT along the last axis, float32 butterflies."""
    z = np.array(x, dtype=np.float32, copy=True)
    n = z.shape[-1]
    if block < 1 or block & (block - 1) or n % block:
        raise ValueError("block must be a power of two dividing the row length")
    lead = z.shape[:-1]
    z = z.reshape(lead + (n // block, block))
    h = 1
    while h < block:
        v = z.reshape(lead + (n // block, block // (2 * h), 2, h))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return z.reshape(lead + (n,))


def inv_sqrt_f32(block: int) -> np.float32:
    """fl32(1/sqrt(block)): the normalization constant of the standalone transform."""
    return np.float32(1.0 / np.sqrt(np.float64(block)))


def hadamard_block(x: np.ndarray, block: int = 128, normalize: bool = True) -> np.ndarray:
    """Standalone transform: z, or fl32(z * fl32(1/sqrt(block))) when normalized."""
    z = fwht_blocks(x, block)
    if normalize:
        z = (z * inv_sqrt_f32(block)).astype(np.float32)
    return z

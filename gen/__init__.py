"""Seeded synthetic inputs for the quantized video-DiT linear layer.

This module only draws random numbers and casts them to the storage dtype.
It holds none of the quantization arithmetic: both the CPU oracle (through the
tests) and the GPU path receive exactly the tensors produced here.

Workloads (shapes from the five DiT-shaped linear configurations):

  c1  tiny W8A8:        X fp16 [256 x 512] N(0,1), 8 channels x20; W fp16 [512 x 512] N(0,0.02^2)
  c2  W8A8 fused QKV:   X bf16 [17776 x 1920] N(0,1), 19 channels x30; W bf16 [5760 x 1920]
  c3  W4A8 FFN-up dual: X bf16 [17776 x 3072] N(0,1); W bf16 [12288 x 3072], 30 input channels x25
  c4  W4A6 FFN-down:    X bf16 [17776 x 12288] Laplace(0,1), Bernoulli(1e-3) elements x50;
                        W bf16 [3072 x 12288]
  c5  DMPQ routed:      X bf16 [35552 x 3072] = two independent N(0,1) halves of 17776 rows
                        (classifier-free-guidance cond/uncond); 42 layers W_l bf16 [3072 x 3072];
                        routing pairs (x_l, y_l), 65536 elements, y_l = x_l + g_l * eps, g_l ~ U(0, 0.2)

Seeding: every draw uses numpy's PCG64 through
``np.random.default_rng(np.random.SeedSequence([1000 * cfg + role, index]))``
with role 0 = X, 1 = W, 2 = outlier-channel choice, 3 = spikes, 4 = routing pairs,
10 = per-layer weights; ``index`` separates halves / layers.  Values are drawn in
float32, scaled in float32, and cast once to fp16/bf16 by torch's round-to-nearest-even
cast.  "1% of channels" is floor(0.01 * K) distinct channels chosen without replacement.
"""
from __future__ import annotations

import numpy as np
import torch

ROLE_X, ROLE_W, ROLE_CHANNELS, ROLE_SPIKES, ROLE_ROUTE, ROLE_LAYER_W = 0, 1, 2, 3, 4, 10

CONFIGS = {
    1: dict(name="c1_tiny_w8a8_per_tensor", M=256, K=512, N=512, dtype="fp16",
            w_bits=8, a_bits=8, gran="tensor", had=0, dual=False,
            x_dist="normal", x_chan_count=8, x_chan_mult=20.0, w_std=0.02),
    2: dict(name="c2_qkv_w8a8_per_token", M=17776, K=1920, N=5760, dtype="bf16",
            w_bits=8, a_bits=8, gran="token", had=0, dual=False,
            x_dist="normal", x_chan_count=19, x_chan_mult=30.0, w_std=0.02),
    3: dict(name="c3_ffn_up_w4a8_dual_scale", M=17776, K=3072, N=12288, dtype="bf16",
            w_bits=4, a_bits=8, gran="token", had=0, dual=True,
            x_dist="normal", w_chan_count=30, w_chan_mult=25.0, w_std=0.02),
    4: dict(name="c4_ffn_down_w4a6_hadamard128", M=17776, K=12288, N=3072, dtype="bf16",
            w_bits=4, a_bits=6, gran="token", had=128, dual=False,
            x_dist="laplace", spike_p=1e-3, spike_mult=50.0, w_std=0.02),
    5: dict(name="c5_dmpq_routed_42_layers", M=35552, K=3072, N=3072, dtype="bf16",
            w_bits=4, a_bits=None, gran="token", had=0, dual=False, layers=42,
            x_dist="normal_halves", w_std=0.02, route_n=65536, route_gmax=0.2,
            route_threshold=0.1, route_hi_bits=8, route_lo_bits=4),
}

TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}


def rng_for(cfg: int, role: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([1000 * cfg + role, index]))


def to_storage(a32: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> CPU torch tensor of the storage dtype (RNE cast by torch)."""
    assert a32.dtype == np.float32
    return torch.from_numpy(np.ascontiguousarray(a32)).to(TORCH_DTYPE[dtype])


def channel_choice(cfg: int, k: int, count: int) -> np.ndarray:
    rng = rng_for(cfg, ROLE_CHANNELS)
    return np.sort(rng.choice(k, size=count, replace=False)).astype(np.int64)


def _laplace(rng: np.random.Generator, shape) -> np.ndarray:
    # Laplace(0, 1) as a random sign times an Exp(1) magnitude.
    mag = rng.standard_exponential(size=shape, dtype=np.float32)
    sign = rng.random(size=shape, dtype=np.float32) < 0.5
    return np.where(sign, -mag, mag).astype(np.float32)


def make_x(cfg: int, m: int | None = None, k: int | None = None) -> torch.Tensor:
    """Activation tensor X [m x k] of configuration ``cfg`` (defaults: the full shape)."""
    c = CONFIGS[cfg]
    m = c["M"] if m is None else m
    k = c["K"] if k is None else k
    dist = c["x_dist"]
    if dist == "normal":
        x = rng_for(cfg, ROLE_X).standard_normal(size=(m, k), dtype=np.float32)
    elif dist == "normal_halves":
        half = (m + 1) // 2
        a = rng_for(cfg, ROLE_X, 0).standard_normal(size=(half, k), dtype=np.float32)
        b = rng_for(cfg, ROLE_X, 1).standard_normal(size=(m - half, k), dtype=np.float32)
        x = np.concatenate([a, b], axis=0)
    elif dist == "laplace":
        x = _laplace(rng_for(cfg, ROLE_X), (m, k))
        spikes = rng_for(cfg, ROLE_SPIKES).random(size=(m, k), dtype=np.float32) < c["spike_p"]
        x = np.where(spikes, x * np.float32(c["spike_mult"]), x).astype(np.float32)
    else:
        raise ValueError(dist)
    if c.get("x_chan_count"):
        cnt = c["x_chan_count"] if k == c["K"] else max(1, (c["x_chan_count"] * k) // c["K"])
        idx = channel_choice(cfg, k, cnt)
        x[:, idx] *= np.float32(c["x_chan_mult"])
    return to_storage(x, c["dtype"])


def x_outlier_channels(cfg: int, k: int | None = None) -> np.ndarray:
    c = CONFIGS[cfg]
    k = c["K"] if k is None else k
    cnt = c["x_chan_count"] if k == c["K"] else max(1, (c["x_chan_count"] * k) // c["K"])
    return channel_choice(cfg, k, cnt)


def w_outlier_channels(cfg: int, k: int | None = None) -> np.ndarray:
    c = CONFIGS[cfg]
    k = c["K"] if k is None else k
    cnt = c["w_chan_count"] if k == c["K"] else max(1, (c["w_chan_count"] * k) // c["K"])
    return channel_choice(cfg, k, cnt)


def make_w(cfg: int, n: int | None = None, k: int | None = None, layer: int | None = None) -> torch.Tensor:
    """Weight tensor W [n x k] (rows = output channels) of configuration ``cfg``."""
    c = CONFIGS[cfg]
    n = c["N"] if n is None else n
    k = c["K"] if k is None else k
    rng = rng_for(cfg, ROLE_W) if layer is None else rng_for(cfg, ROLE_LAYER_W, layer)
    w = rng.standard_normal(size=(n, k), dtype=np.float32) * np.float32(c["w_std"])
    if c.get("w_chan_count"):
        w[:, w_outlier_channels(cfg, k)] *= np.float32(c["w_chan_mult"])
    return to_storage(w.astype(np.float32), c["dtype"])


def make_route_pair(cfg: int, layer: int, n: int | None = None):
    """Previous-step block input/output pair (x_l, y_l) for the routing statistic."""
    c = CONFIGS[cfg]
    n = c["route_n"] if n is None else n
    rng = rng_for(cfg, ROLE_ROUTE, layer)
    g = np.float32(rng.uniform(0.0, c["route_gmax"]))
    x = rng.standard_normal(size=n, dtype=np.float32)
    eps = rng.standard_normal(size=n, dtype=np.float32)
    y = (x + g * eps).astype(np.float32)
    return to_storage(x, c["dtype"]), to_storage(y, c["dtype"]), float(g)


def as_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Storage view handed to the oracle: fp16 -> np.float16, bf16 -> raw uint16 bits."""
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)

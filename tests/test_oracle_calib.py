"""Pins of the clipping-percentile search oracle (Q-ARVD page, Technical details: per-tensor
activations with a learned clipping percentile and scale).

Checked against closed forms and brute force: the 100th percentile is the maximum and
gives the dynamic per-tensor scale; percentile ranks on a tiny hand-made set; the MSE of
a tensor its quantizer represents exactly is zero; the MSE equals a direct element sum
written out independently; clipping a lone outlier wins over the full range.
"""
import numpy as np
import pytest

from oracle import calib, numerics
from oracle import quantizer as oq


def test_percentile_ranks_hand_set():
    x = np.array([-5.0, 1.0, 2.0, -3.0, 4.0, 0.5, 0.0, 7.0, -6.0, 8.0], np.float32)  # |x| sorted: 0 .5 1 2 3 4 5 6 7 8
    assert calib.percentile_clip(x, 100.0) == 8.0
    assert calib.percentile_clip(x, 90.0) == 7.0     # rank 9
    assert calib.percentile_clip(x, 85.0) == 7.0     # ceil(8.5) = 9
    assert calib.percentile_clip(x, 80.0) == 6.0     # rank 8
    assert calib.percentile_clip(x, 0.001) == 0.0    # rank 1
    assert calib.rank_of(99.999, 10) == 10


def test_full_range_equals_dynamic_per_tensor_scale():
    rng = np.random.default_rng(1)
    x = numerics.from_f32(rng.standard_normal((64, 96)).astype(np.float32), "bf16")
    r = calib.search(x, "bf16", 8, grid=(100.0,))
    _, s_dyn = oq.quant_act(x, "bf16", 8, "tensor")
    assert r["scales"][0] == s_dyn[0]


def test_exactly_representable_tensor_has_zero_error():
    q = np.random.default_rng(2).integers(-127, 128, size=(16, 64))
    q[0, 0] = 127
    x = (q * 2.0 ** -5).astype(np.float32)
    assert calib.static_mse(x, np.float32(127 * 2.0 ** -5 / 127), 8) == 0.0


def test_mse_is_the_element_sum():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(500).astype(np.float32)
    s = np.float32(0.03125)
    want = 0.0
    for v in x:  # written out element by element
        t = np.float32(v * np.float32(1.0 / s))
        q = min(127.0, max(-127.0, float(np.rint(t))))
        d = float(np.float32(np.float32(q) * s))
        want += (float(v) - d) ** 2
    assert calib.static_mse(x, s, 8) == pytest.approx(want / x.size, rel=1e-12)


def test_lone_outlier_is_clipped():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((128, 256)).astype(np.float32)
    # One large value.  Full range (s = 20/31): MSE about s^2/12 = 0.035.  Clipping near the
    # 99.99th percentile (about 3.9): about (3.9/31)^2/12 + (20 - 3.9)^2/N = 0.0013 + 0.0079.
    x[5, 7] = 20.0
    r = calib.search(numerics.from_f32(x, "bf16"), "bf16", 6)
    assert r["best"] != 0
    assert r["mse"][r["best"]] < r["mse"][0]
    assert r["scale"] < r["scales"][0]

"""GPU parity of the static-scale calibration (Q-ARVD page, Technical details: learned
clipping percentile and scale; oracle/calib.py).

The device histogram of |x| is compared with a bincount of the magnitude patterns (exact),
the clips and candidate scales bit for bit with the oracle, the reconstruction errors
within float64 summation-order rounding, and the chosen scale end to end through the
static quantizer.
"""
import numpy as np
import pytest
import torch

import gen
from oracle import calib, numerics
from oracle import quantizer as oq

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def bits16(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def check(vq, x, dtype, bits):
    r = vq.vq_calib_static_scale(x.to(DEV), bits)
    torch.cuda.synchronize()
    hist = r["hist"].cpu().numpy().view(np.uint32)
    want_hist = np.bincount((bits16(x) & 0x7FFF).reshape(-1), minlength=32768)
    assert np.array_equal(hist, want_hist)
    store = gen.as_numpy_bits(x)
    o = calib.search(store, dtype, bits)
    assert np.array_equal(np.array(r["clips"], np.float32), o["clips"])
    assert np.array_equal(np.array(r["scales"], np.float32), o["scales"])
    np.testing.assert_allclose(np.array(r["mse"]), o["mse"], rtol=1e-9)
    m = np.sort(o["mse"])
    if m[1] - m[0] > 1e-9 * m[0]:  # a clear minimum: the same choice
        assert r["best"] == o["best"]
    assert r["scale"].item() == r["scales"][r["best"]]
    # The chosen scale drives the static quantizer.
    codes, s = vq.vq_quant_act(x.to(DEV), bits, "static", static_scale=r["scale"])
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(store, dtype, bits, "static", static_scale=np.array([r["scales"][r["best"]]], np.float32))
    assert np.array_equal(codes.cpu().numpy(), rc)
    return r


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_calibration_bf16(vq, bits):
    g = np.random.default_rng(bits)
    x = g.standard_normal((300, 640)).astype(np.float32)
    x[g.integers(0, 300, 5), g.integers(0, 640, 5)] = 30.0  # a few outliers
    check(vq, gen.to_storage(x, "bf16"), "bf16", bits)


def test_calibration_fp16_with_subnormals_and_zeros(vq):
    g = np.random.default_rng(9)
    x = (g.standard_normal((128, 256)) * 1e-3).astype(np.float32)
    x[0, :64] = 0.0
    x[1, :32] = 3e-7  # fp16 subnormals
    check(vq, gen.to_storage(x, "fp16"), "fp16", 8)


def test_calibration_fullsize_c2_activations(vq):
    """The fused-QKV input, 17776 x 1920 bf16 with its planted outlier channels."""
    r = check(vq, gen.make_x(2), "bf16", 8)
    assert 0 <= r["best"] < len(r["mse"])

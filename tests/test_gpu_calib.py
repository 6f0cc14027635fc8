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
    clips, scales, mse = r["clips"].cpu().numpy(), r["scales"].cpu().numpy(), r["mse"].cpu().numpy()
    best = int(r["best"].item())
    assert np.array_equal(clips.view(np.uint32), o["clips"].view(np.uint32))
    assert np.array_equal(scales.view(np.uint32), o["scales"].view(np.uint32))
    np.testing.assert_allclose(mse, o["mse"], rtol=1e-9)
    m = np.sort(o["mse"])
    if m[1] - m[0] > 1e-9 * m[0]:  # a clear minimum: the same choice
        assert best == o["best"]
    # The device pick is the first minimum of the device errors.
    assert best == int(np.argmin(mse))
    assert r["scale"].item() == scales[best]
    # The chosen scale drives the static quantizer.
    codes, s = vq.vq_quant_act(x.to(DEV), bits, "static", static_scale=r["scale"])
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(store, dtype, bits, "static", static_scale=np.array([scales[best]], np.float32))
    assert np.array_equal(codes.cpu().numpy(), rc)
    return r, best


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
    r, best = check(vq, gen.make_x(2), "bf16", 8)
    assert 0 <= best < r["mse"].numel()


def test_calibration_ties_and_one_candidate(vq):
    """Repeated percentiles give identical candidates: the first one is chosen."""
    g = np.random.default_rng(3)
    x = gen.to_storage(g.standard_normal((64, 128)).astype(np.float32), "bf16").to(DEV)
    r = vq.vq_calib_static_scale(x, 8, percentiles=(99.0, 99.0, 100.0, 99.0))
    torch.cuda.synchronize()
    mse = r["mse"].cpu().numpy()
    assert mse[0] == mse[1] == mse[3]
    assert int(r["best"].item()) in (0, 2)
    one = vq.vq_calib_static_scale(x, 8, percentiles=(100.0,))
    torch.cuda.synchronize()
    assert int(one["best"].item()) == 0
    assert one["scale"].item() == r["scales"][2].item()


def test_calibration_all_zero_tensor(vq):
    """|x| = 0 everywhere: every clip is 0, the scale is 0 and the error is 0."""
    x = torch.zeros((32, 64), dtype=torch.float16, device=DEV)
    r = vq.vq_calib_static_scale(x, 8)
    torch.cuda.synchronize()
    assert not r["clips"].any() and not r["scales"].any() and not r["mse"].any()
    assert int(r["best"].item()) == 0 and r["scale"].item() == 0.0


def test_calibration_strided_rows(vq):
    """A column slice of a wider tensor (row pitch 1032 > 776 columns)."""
    g = np.random.default_rng(11)
    wide = gen.to_storage(g.standard_normal((257, 1032)).astype(np.float32) * 2.0, "bf16")
    xs = wide[:, 8:784]
    r = vq.vq_calib_static_scale(wide.to(DEV)[:, 8:784], 6)
    torch.cuda.synchronize()
    o = calib.search(gen.as_numpy_bits(xs.contiguous()), "bf16", 6)
    hist = r["hist"].cpu().numpy().view(np.uint32)
    assert np.array_equal(hist, np.bincount((bits16(xs) & 0x7FFF).reshape(-1), minlength=32768))
    assert np.array_equal(r["clips"].cpu().numpy().view(np.uint32), o["clips"].view(np.uint32))
    np.testing.assert_allclose(r["mse"].cpu().numpy(), o["mse"], rtol=1e-9)

"""Pins of the unquantized FP16/BF16 layer of the oracle (oracle/dense.py; 6Bit-Diffusion
page, Methodology B.3, PDR), against values fixed by hand and by brute force."""
import numpy as np
import pytest

import gen
from oracle import dense
from oracle import numerics as onum


def store(a, dt):
    return gen.as_numpy_bits(gen.to_storage(np.asarray(a, dtype=np.float32), dt))


def test_hand_worked_product():
    """[[1, 2], [3, -4]] . [[0.5, 0.25], [-1, 2]]^T = [[1, 3], [0.5, -11]], exact in any type."""
    for dt in ("bf16", "fp16"):
        x = store([[1, 2], [3, -4]], dt)
        w = store([[0.5, 0.25], [-1, 2]], dt)
        y, y32, ys = dense.forward(x, dt, w)
        assert y.tolist() == [[1.0, 3.0], [0.5, -11.0]]
        assert onum.to_f32(ys, dt).tolist() == [[1.0, 3.0], [0.5, -11.0]]


def test_brute_force_triple_loop():
    rng = np.random.default_rng(3)
    x = store(rng.standard_normal((5, 7)), "bf16")
    w = store(rng.standard_normal((4, 7)), "bf16")
    xf, wf = onum.to_f32(x, "bf16"), onum.to_f32(w, "bf16")
    want = np.zeros((5, 4))
    for m in range(5):
        for n in range(4):
            for k in range(7):
                want[m, n] += float(xf[m, k]) * float(wf[n, k])
    y, _, _ = dense.forward(x, "bf16", w)
    assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_ones_give_k_and_rounding_of_the_output():
    """All-ones operands sum to K exactly; K = 257 is not a bf16 value (8 bits of mantissa),
    so the bf16 output is 256 (ties to even) while fp16 keeps 257."""
    x = store(np.ones((2, 257)), "bf16")
    y, y32, ys = dense.forward(x, "bf16", x)
    assert y.tolist() == [[257.0, 257.0]] * 2
    assert onum.to_f32(ys, "bf16").tolist() == [[256.0, 256.0]] * 2
    xh = store(np.ones((1, 257)), "fp16")
    assert onum.to_f32(dense.forward(xh, "fp16", xh)[2], "fp16").tolist() == [[257.0]]


def test_products_of_16_bit_values_are_exact_and_bound_covers_float32_orders():
    """A float32 accumulation in two different orders stays within the stated bound of the
    exact sum, and the bound is not vacuous (cancellation makes the float32 sum wrong in
    its last bits)."""
    rng = np.random.default_rng(5)
    k = 3000
    x = store(rng.standard_normal((3, k)) * 100, "bf16")
    w = store(rng.standard_normal((2, k)), "bf16")
    xf, wf = onum.to_f32(x, "bf16"), onum.to_f32(w, "bf16")
    y = dense.exact(x, "bf16", w)
    b = dense.bound(dense.magnitude(x, "bf16", w), k)
    for order in (slice(None), slice(None, None, -1)):
        acc = np.zeros((3, 2), dtype=np.float32)
        for kk in range(k)[order]:
            acc = (acc + (xf[:, kk:kk + 1] * wf[:, kk][None, :]).astype(np.float32)).astype(np.float32)
        assert np.all(np.abs(acc.astype(np.float64) - y) <= b)
        assert np.any(acc.astype(np.float64) != y)


def test_transposition_symmetry_and_k_mismatch():
    rng = np.random.default_rng(7)
    a = store(rng.standard_normal((3, 64)), "fp16")
    b = store(rng.standard_normal((5, 64)), "fp16")
    assert np.array_equal(dense.exact(a, "fp16", b), dense.exact(b, "fp16", a).T)
    with pytest.raises(ValueError):
        dense.exact(a, "fp16", b[:, :32])

"""Pins of the activation-decomposition oracle (SemanticDialect page, Methodology 2.2).

Each test checks the oracle against something other than itself: a hand-worked
example, closed forms (a row its quantizer represents exactly leaves no residual), the
rounding bound of the residual, the error reduction the decomposition must bring, and
the identity that undecomposed rows equal the plain layer.
"""
import json
import os

import numpy as np
import pytest

import gen
from oracle import decompose, linear, numerics
from oracle import gemm as ogemm
from oracle import quantizer as oq

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    with open(os.path.join(HERE, "golden", "decompose.json")) as f:
        return json.load(f)


def test_hand_worked_example():
    g = golden()
    x = numerics.from_f32(np.array([g["x_bf16_values"]], np.float32), "bf16")
    wc = np.array([g["w_codes"]], np.int8)
    ws = np.array([g["w_scale"]], np.float32)
    r = decompose.forward(x, "bf16", g["bits1"], g["bits2"], [0], wc, ws, "bf16")
    assert r["q1"].tolist() == [g["q1"]]
    assert r["s1"].tolist() == [g["s1"]]
    assert r["q2"].tolist() == [g["q2"]]
    assert hex(int(r["s2"].view(np.uint32)[0])) == g["s2_bits"]
    assert int(r["acc1"][0, 0]) == g["acc1"] and int(r["acc2"][0, 0]) == g["acc2"]
    assert float(r["y"][0, 0]) == g["y_with"]
    assert hex(int(r["y_store"][0, 0])) == g["y_with_bf16_bits"]
    r0 = decompose.forward(x, "bf16", g["bits1"], g["bits2"], [], wc, ws, "bf16")
    assert float(r0["y"][0, 0]) == g["y_without"]


@pytest.mark.parametrize("bits1", [4, 6, 8])
def test_exactly_representable_rows_leave_no_residual(bits1):
    # x = s * q with s a power of two and max |q| = Q: the first quantizer is exact.
    Q = oq.qmax(bits1)
    rng = np.random.default_rng(7)
    q = rng.integers(-Q, Q + 1, size=(5, 96))
    q[:, 3] = Q
    x = (q * 2.0 ** -3).astype(np.float32)
    xs = numerics.from_f32(x, "bf16")
    assert np.array_equal(numerics.to_f32(xs, "bf16"), x)
    q2, s2 = decompose.residual_quant(xs, "bf16", bits1, 8, np.arange(5))
    assert not q2.any() and not s2.any()


@pytest.mark.parametrize("bits1,bits2", [(4, 4), (4, 8), (6, 6), (8, 8)])
def test_residual_bound_and_error_reduction(bits1, bits2):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 320)).astype(np.float32)
    xs = numerics.from_f32(x, "bf16")
    xf = numerics.to_f32(xs, "bf16").astype(np.float64)
    rows = np.arange(16)
    q1, s1 = oq.quantize_groups(numerics.to_f32(xs, "bf16"), oq.qmax(bits1), axis=1)
    q2, s2 = decompose.residual_quant(xs, "bf16", bits1, bits2, rows)
    Q1 = oq.qmax(bits1)
    deq1 = q1.astype(np.float64) * s1.astype(np.float64)[:, None]
    resid = xf - deq1
    # float32 holds deq1 to 1 ulp of the row maximum Q1*s1: slack 2^-23 * 2 * Q1 * s1.
    slack = 2.0 ** -22 * Q1 * s1.astype(np.float64)
    # Rounding to nearest leaves at most half a step.
    assert np.all(np.abs(resid).max(axis=1) <= 0.5 * s1 + slack)
    # The residual's scale is its own absolute maximum over Q2.
    np.testing.assert_allclose(s2 * oq.qmax(bits2), np.abs(resid).max(axis=1), rtol=1e-6, atol=slack.max())
    # Adding the dequantized residual back shrinks the error to half a residual step.
    deq2 = q2.astype(np.float64) * s2.astype(np.float64)[:, None]
    err1 = np.abs(xf - deq1).max(axis=1)
    err2 = np.abs(xf - deq1 - deq2).max(axis=1)
    assert np.all(err2 <= 0.5 * s2 * (1 + 1e-6) + 2 * slack)
    assert np.all(err2 < err1)


def test_rows_outside_the_set_equal_the_plain_layer():
    x, w = gen.make_x(2)[:64, :256], gen.make_w(2)[:96, :256]
    xs, wsb = gen.as_numpy_bits(x), gen.as_numpy_bits(w)
    wcodes, _, wsc = linear.prepare_weights(wsb, "bf16", 8)
    rows = np.array([0, 5, 31, 63])
    r = decompose.forward(xs, "bf16", 8, 8, rows, wcodes, wsc, "bf16")
    plain = linear.forward(xs, "bf16", 8, "token", wcodes, wsc)
    keep = np.setdiff1d(np.arange(64), rows)
    assert np.array_equal(r["y_store"][keep], plain["y_store"][keep])
    assert np.array_equal(r["q1"], plain["qa"])
    assert not np.array_equal(r["y_store"][rows], plain["y_store"][rows])


def test_decomposed_rows_match_the_dequantized_product():
    # y = (deq1 + deq2) . deq(W)^T up to float32 rounding of the two-term epilogue.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 192)).astype(np.float32)
    xs = numerics.from_f32(x, "bf16")
    w = (0.02 * rng.standard_normal((40, 192))).astype(np.float32)
    wcodes, _, wsc = oq.pack_weights(numerics.from_f32(w, "bf16"), "bf16", 8)
    rows = np.arange(8)
    r = decompose.forward(xs, "bf16", 4, 8, rows, wcodes, wsc, "bf16")
    deq = r["q1"].astype(np.float64) * r["s1"][:, None] + r["q2"].astype(np.float64) * r["s2"][:, None]
    ref = deq @ (wcodes.astype(np.float64) * wsc[:, None].astype(np.float64)).T
    np.testing.assert_allclose(r["y"], ref, rtol=2e-6, atol=2e-6 * np.abs(ref).max())


def test_planted_sign_error_is_caught():
    # Subtracting the residual instead of adding it must violate the error-reduction pin.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    xs = numerics.from_f32(x, "bf16")
    xf = numerics.to_f32(xs, "bf16").astype(np.float64)
    q1, s1 = oq.quantize_groups(numerics.to_f32(xs, "bf16"), 7, axis=1)
    q2, s2 = decompose.residual_quant(xs, "bf16", 4, 8, np.arange(4))
    deq1 = q1 * s1[:, None].astype(np.float64)
    wrong = np.abs(xf - deq1 + q2 * s2[:, None].astype(np.float64)).max(axis=1)
    assert np.all(wrong > s2 * 0.5 * 1.0001)

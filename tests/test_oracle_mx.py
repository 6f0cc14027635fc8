"""Pins of the MX block-format oracle (oracle/mx.py).

The element formats, the shared-exponent rule and the rounding come from the OCP
Microscaling (MX) v1.0 definition (the gfx950 counterpart of the 4-bit floating-point
route of the 6Bit-Diffusion page, Methodology B.1).  Each test checks the oracle against
something it does not compute itself: the formats' value tables typed from their
definitions, a brute-force nearest-value search, hand-worked block scales and bit
packing, and a table-lookup dequantized matrix product.
"""
import numpy as np
import pytest

from oracle import mx

# Value tables typed from the format definitions (positive codes 0..2^(E+M)-1).
FP4_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
FP6_VALUES = ([k / 8 for k in range(8)] + [1 + m / 8 for m in range(8)] + [2 + m / 4 for m in range(8)]
              + [4 + m / 2 for m in range(8)])
TABLES = {"fp4": FP4_VALUES, "fp6": FP6_VALUES}


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
def test_value_tables(fmt):
    tab = TABLES[fmt]
    n = len(tab)
    assert mx.decode(np.arange(n), fmt).tolist() == tab
    neg = mx.decode(np.arange(n) | n, fmt)
    assert neg.tolist() == [-v for v in tab]
    assert np.signbit(neg[0])
    assert max(tab) == mx.FORMATS[fmt][4]


def brute(t, fmt):
    """Nearest table value, ties to the code with an even mantissa bit; saturating."""
    tab = np.array(TABLES[fmt])
    mag = abs(t)
    d = np.abs(tab - mag)
    best = np.flatnonzero(d == d.min())
    c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return int(c) | ((len(tab)) if np.signbit(t) else 0)


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
def test_encode_matches_brute_force(fmt):
    rng = np.random.default_rng(4)
    tab = np.array(TABLES[fmt])
    mids = (tab[1:] + tab[:-1]) / 2          # every tie
    ts = np.concatenate([rng.uniform(-9, 9, 4000), mids, -mids, tab, -tab, [0.0, -0.0, 7.0, 8.5, -100.0]])
    got = mx.encode(ts, fmt)
    want = np.array([brute(t, fmt) for t in ts])
    assert np.array_equal(got, want)


def test_hand_worked_block_scales():
    x = np.zeros((1, 128), np.float32)
    x[0, 0:32] = 1.0          # amax 1: e = 0 - 2 = -2, X = 1/4, 1/X = 4 -> FP4 code 6 (4.0)
    x[0, 32] = 7.0            # amax 7: e = 2 - 2 = 0, X = 1; 7 saturates to 6
    x[0, 33] = 2.5            # tie between 2 and 3 -> 2 (even mantissa)
    x[0, 34] = -0.2           # rounds to -0
    # block 2 all zero: e = -127
    x[0, 96] = 2.0 ** -130    # a tiny block: e clamps to -127
    codes, scales = mx.quantize(x, "fp4")
    assert scales.tolist() == [[125, 127, 0, 0]]
    assert codes[0, 0] == 6 and codes[0, 31] == 6
    assert codes[0, 32] == 7 and codes[0, 33] == 4 and codes[0, 34] == 8
    assert not codes[0, 64:96].any()
    # 2^-130 / 2^-127 = 1/8 rounds to 0 in FP4 (ties-to-even of 0.125 is below 0.25)
    assert codes[0, 96] == 0


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
def test_representable_blocks_round_trip(fmt):
    rng = np.random.default_rng(8)
    tab = np.array(TABLES[fmt])
    rows = 6
    vals = rng.choice(tab, size=(rows, 64)) * rng.choice([-1, 1], size=(rows, 64))
    vals[:, 0] = tab[-1]  # each block's maximum is the largest value, so X = 2^e exactly
    vals[:, 32] = tab[-1]
    e = rng.integers(-20, 20, size=(rows, 2))
    x = (vals * np.ldexp(1.0, np.repeat(e, 32, axis=1))).astype(np.float32)
    codes, scales = mx.quantize(x, fmt)
    np.testing.assert_array_equal(mx.dequantize(codes, scales, fmt), x.astype(np.float64))


def test_packing_hand_cases():
    assert mx.pack(np.array([[1, 2]]), "fp4").tolist() == [[0x21]]
    # 1 | 2 << 6 | 3 << 12 | 4 << 18 = 0x103081
    assert mx.pack(np.array([[1, 2, 3, 4]]), "fp6").tolist() == [[0x81, 0x30, 0x10]]
    rng = np.random.default_rng(2)
    for fmt, w in (("fp4", 4), ("fp6", 6)):
        c = rng.integers(0, 1 << w, size=(3, 64))
        assert np.array_equal(mx.unpack(mx.pack(c, fmt), 64, fmt), c)


def test_quantization_error_bound():
    # Outside saturation, rounding leaves at most half a step of the element's binade.
    rng = np.random.default_rng(9)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    for fmt in ("fp4", "fp6"):
        codes, scales = mx.quantize(x, fmt)
        deq = mx.dequantize(codes, scales, fmt)
        X = np.ldexp(1.0, np.repeat(scales.astype(np.int64) - 127, 32, axis=1))
        t = x / X
        M = mx.FORMATS[fmt][1]
        sat = np.abs(t) > mx.FORMATS[fmt][4]
        binade = np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 1e-30))), 0)
        half_step = np.ldexp(0.5, (binade - M).astype(np.int64)) * X
        assert np.all(np.abs(x - deq)[~sat] <= half_step[~sat] * (1 + 1e-12))
        assert np.all(np.abs(deq[sat]) == mx.FORMATS[fmt][4] * X[sat])


def test_gemm_equals_table_lookup_product():
    rng = np.random.default_rng(12)
    a = rng.standard_normal((5, 96)).astype(np.float32)
    b = rng.standard_normal((7, 96)).astype(np.float32)
    ac, asc = mx.quantize(a, "fp6")
    bc, bsc = mx.quantize(b, "fp4")
    lut6 = np.array(FP6_VALUES + [-v for v in FP6_VALUES])
    lut4 = np.array(FP4_VALUES + [-v for v in FP4_VALUES])
    da = lut6[ac] * np.ldexp(1.0, np.repeat(asc.astype(int) - 127, 32, axis=1))
    db = lut4[bc] * np.ldexp(1.0, np.repeat(bsc.astype(int) - 127, 32, axis=1))
    np.testing.assert_array_equal(mx.gemm(ac, asc, "fp6", bc, bsc, "fp4"), da @ db.T)


# ---------------------------------------------------------------- rotated route (online block Hadamard)

def test_rotated_hand_worked_blocks():
    """x = e_0 rotates to a row of ones (column 0 of the Sylvester matrix): every 32-block
    has amax 1, e = 0 - 2 = -2 (byte 125) and 1 / 2^-2 = 4 -> FP4 code 6.  x = e_1 gives
    (+1, -1, +1, ...): codes alternate 6 and 14 (sign bit 8).  x = 2 e_0 + e_1 gives
    (3, 1, 3, 1, ...): amax 3, e = 1 - 2 = -1 (byte 126), 3 / 0.5 = 6 -> code 7, 1 / 0.5 =
    2 -> code 4."""
    x = np.zeros((3, 128), np.float32)
    x[0, 0] = 1.0
    x[1, 1] = 1.0
    x[2, 0], x[2, 1] = 2.0, 1.0
    codes, scales = mx.quantize_rotated(x, "fp4")
    assert codes[0].tolist() == [6] * 128
    assert codes[1].tolist() == [6, 14] * 64
    assert codes[2].tolist() == [7, 4] * 64
    assert scales.tolist() == [[125] * 4, [125] * 4, [126] * 4]
    # Weights pre-rotated with exp_offset = -7: same codes, exponents 7 lower; the decoded
    # product of the two rotated e_0 rows is 128 * 1 * 2^-7 = 1 = e_0 . e_0.
    wc, ws = mx.quantize_rotated(x[:1], "fp4", exp_offset=-7)
    assert wc[0].tolist() == [6] * 128 and ws.tolist() == [[118] * 4]
    y = mx.gemm(codes[:1], scales[:1], "fp4", wc, ws, "fp4")
    assert y.tolist() == [[1.0]]


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
def test_rotated_equals_explicit_hadamard_product(fmt):
    """On small-integer rows the float32 butterflies are exact, so the rotated codes must
    equal the codes of H x computed as a float64 product with the explicit +-1 matrix
    (scipy's Sylvester construction), for both exponent offsets."""
    from scipy.linalg import hadamard
    rng = np.random.default_rng(11)
    x = rng.integers(-9, 10, size=(16, 384)).astype(np.float32)
    h = hadamard(128).astype(np.float64)
    z = (x.astype(np.float64).reshape(16, 3, 128) @ h.T).reshape(16, 384)
    for off in (0, -7):
        got = mx.quantize_rotated(x, fmt, exp_offset=off)
        want = mx.quantize((z * 2.0 ** off).astype(np.float32), fmt)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_rotated_offset_moves_only_exponents():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    c0, s0 = mx.quantize_rotated(x, "fp6")
    c7, s7 = mx.quantize_rotated(x, "fp6", exp_offset=-7)
    assert np.array_equal(c0, c7)
    assert np.array_equal(s0.astype(int) - 7, s7.astype(int))

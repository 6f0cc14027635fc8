"""Pins of the CPU oracle against hand-worked examples, closed forms and library routines.

Each pin checks the oracle against something other than itself: values worked by
hand from the pages' definitions (tests/golden/*.json, each with its citation),
textbook constructions (the Sylvester Hadamard matrix by popcount), library
routines (scipy's Hadamard matrix and MAD, torch's bf16 cast, NumPy's float16 cast)
and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.stats
import torch

import oracle
from oracle import detect, fwht, gemm, numerics, quantizer, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- detection


@pytest.mark.parametrize("case", load("modified_zscore.json")["cases"], ids=lambda c: c["name"])
def test_modified_zscore_worked_examples(case):
    fx = load("modified_zscore.json")
    v = np.array(case["v"], dtype=np.float64)
    mask, idx, m, med, mad = detect.flag_outliers(v, fx["tau"], fx["alpha"], 1.0)
    assert med == pytest.approx(case["median"], abs=1e-12)
    assert mad == pytest.approx(case["mad"], abs=1e-12)
    want_z = np.array([np.inf if z == "inf" else z for z in case["z"]], dtype=np.float64)
    fin = np.isfinite(want_z)
    np.testing.assert_allclose(m[fin], want_z[fin], rtol=1e-9, atol=1e-9)
    assert np.all(np.isinf(m[~fin]))
    assert mask.astype(int).tolist() == case["mask"]
    assert idx.tolist() == [i for i, f in enumerate(case["mask"]) if f]


def test_median_and_mad_match_scipy():
    rng = np.random.default_rng(7)
    for n in (7, 8, 101, 3072):
        v = rng.gamma(2.0, size=n)
        _, med, mad = detect.modified_z(v)
        assert med == np.median(v)
        assert mad == pytest.approx(scipy.stats.median_abs_deviation(v, scale=1.0), rel=0, abs=0)


def test_textbook_constant_variant():
    v = np.array([1.0, 1.1, 0.9, 1.2, 0.8, 1.05, 6.0, 0.95])
    m1, _, _ = detect.modified_z(v, 1.0)
    m2, _, _ = detect.modified_z(v, 0.6745)
    np.testing.assert_allclose(m2, 0.6745 * m1, rtol=1e-15)


def test_detection_permutation_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((512, 256)).astype(np.float32)
    x[:, [5, 77, 200]] *= 25
    mask, idx, v, *_ = detect.detect_outliers(x)
    assert idx.tolist() == [5, 77, 200]
    perm = rng.permutation(256)
    mask_p, *_ = detect.detect_outliers(x[:, perm])
    assert np.array_equal(mask_p, mask[perm])
    mask_s, *_ = detect.detect_outliers(x * np.float32(4.0))
    assert np.array_equal(mask_s, mask)


def test_column_norms_brute_force():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, 5)).astype(np.float32)
    v = detect.channel_l2_norms(x)
    for k in range(5):
        s = 0.0
        for r in range(9):
            s += float(x[r, k]) ** 2
        assert v[k] == pytest.approx(math.sqrt(s), rel=1e-15)


# ---------------------------------------------------------------- quantizer


@pytest.mark.parametrize("g", load("quantizer.json")["groups"], ids=lambda g: f"bits{g['bits']}")
def test_quantizer_worked_examples(g):
    Q = quantizer.qmax(g["bits"])
    x = np.array(g["x"], dtype=np.float32)
    codes, s = quantizer.quantize_groups(x, Q)
    assert codes.tolist() == g["codes"]
    assert float(s) == g["s"]
    deq = codes.astype(np.float32) * np.float32(s)
    assert deq.tolist() == g["dequant"]


def test_qmax_values():
    assert [quantizer.qmax(b) for b in (4, 6, 8)] == [7, 31, 127]
    with pytest.raises(ValueError):
        quantizer.qmax(5)


def test_dual_per_token_worked_example():
    d = load("quantizer.json")["dual_per_token"]
    x = np.array(d["x"], dtype=np.float32)
    codes, scales = quantizer.quant_act(x, "fp32", d["bits"], "token", 0, np.array(d["outlier_channels"]))
    assert codes.shape == (2, 4 + d["partition1_length"])
    assert codes[:, :4].tolist() == d["codes_partition0"]
    assert codes[:, 4:5].tolist() == d["codes_partition1_first"]
    assert np.all(codes[:, 5:] == 0)
    want = np.array([[np.float32(a) / np.float32(b) for a, b in row] for row in d["scale_fractions"]],
                    dtype=np.float32)
    assert np.array_equal(scales, want)


def test_per_tensor_worked_example():
    d = load("quantizer.json")["per_tensor"]
    x = np.array(d["x"], dtype=np.float32)
    codes, s = quantizer.quant_act(x, "fp32", d["bits"], "tensor")
    assert codes.tolist() == d["codes"]
    assert s.tolist() == [np.float32(d["s_fraction"][0]) / np.float32(d["s_fraction"][1])]


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quantizer_invariants(bits):
    Q = quantizer.qmax(bits)
    rng = np.random.default_rng(bits)
    x = (rng.laplace(size=(64, 257)) * 3).astype(np.float32)
    codes, s = quantizer.quantize_groups(x, Q, axis=1)
    assert codes.min() >= -Q and codes.max() <= Q
    # the largest magnitude maps to +-Q
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(codes[np.arange(64), am]) == Q)
    # reconstruction error at most half a step (plus float32 slack)
    err = np.abs(x - codes.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # odd symmetry and exact power-of-two scale invariance
    cn, sn = quantizer.quantize_groups(-x, Q, axis=1)
    assert np.array_equal(cn, -codes) and np.array_equal(sn, s)
    c4, s4 = quantizer.quantize_groups(x * np.float32(4), Q, axis=1)
    assert np.array_equal(c4, codes) and np.array_equal(s4, s * np.float32(4))
    # monotone within a group
    order = np.argsort(x[0], kind="stable")
    assert np.all(np.diff(codes[0][order].astype(int)) >= 0)


def test_quantizer_brute_force_nearest_code():
    """Each code is the integer in [-Q, Q] nearest to fl32(x*r), ties to the even integer."""
    rng = np.random.default_rng(5)
    for bits in (4, 6, 8):
        Q = quantizer.qmax(bits)
        x = rng.standard_normal(40).astype(np.float32)
        codes, s = quantizer.quantize_groups(x, Q)
        r = np.float32(Q) / np.float32(np.max(np.abs(x)))
        for xi, ci in zip(x, codes):
            t = float(np.float32(xi * r))
            best = min(range(-Q, Q + 1), key=lambda q: (abs(t - q), q % 2))
            assert ci == best


def test_static_scale():
    x = np.array([[0.3, -1.0, 2.0]], dtype=np.float32)
    codes, s = quantizer.quant_act(x, "fp32", 8, "static", static_scale=np.array([0.0625], np.float32))
    # r = 16: 4.8 -> 5, -16, 32 (no clipping needed)
    assert codes.tolist() == [[5, -16, 32]] and s.tolist() == [0.0625]
    codes, _ = quantizer.quant_act(x, "fp32", 4, "static", static_scale=np.array([0.0625], np.float32))
    assert codes.tolist() == [[5, -7, 7]]  # clamped to +-7


@pytest.mark.parametrize("case", load("pack_gemm_epilogue_route.json")["int4_pack"], ids=str)
def test_int4_pack_worked_examples(case):
    got = quantizer.pack_int4(np.array(case["codes"], dtype=np.int8))
    assert [f"0x{b:02X}" for b in got] == case["bytes"]


def test_int4_pack_round_trip():
    rng = np.random.default_rng(9)
    c = rng.integers(-7, 8, size=(5, 128)).astype(np.int8)
    p = quantizer.pack_int4(c)
    # unpack written independently: sign-extend each nibble
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    u = np.empty_like(c, dtype=np.int16)
    u[:, 0::2] = lo
    u[:, 1::2] = hi
    assert np.array_equal(u.astype(np.int8), c)


def test_packed_k_layout():
    assert quantizer.part_len(0) == 0 and quantizer.part_len(1) == 64 and quantizer.part_len(64) == 64
    assert quantizer.part_len(65) == 128
    assert quantizer.packed_k(3072, 30) == 3136 and quantizer.packed_k(1920, 0) == 1920


# ---------------------------------------------------------------- Hadamard


def sylvester(n):
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


@pytest.mark.parametrize("case", load("fwht.json")["cases"], ids=lambda c: c["name"])
def test_fwht_worked_examples(case):
    x = np.array(case["x"], dtype=np.float32)
    z = fwht.fwht_blocks(x[None, :], len(x))[0]
    assert z.tolist() == case["z"]
    if "twice" in case:
        assert fwht.fwht_blocks(z[None, :], len(x))[0].tolist() == case["twice"]
    if "after_h1" in case:
        assert fwht.fwht_blocks(x[None, :], 2)[0].tolist() == case["after_h1"]
    if "z_if_descending" in case:
        assert case["z_if_descending"] != case["z"]


def test_sylvester_orthogonality_and_scipy():
    H = sylvester(128)
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, scipy.linalg.hadamard(128))


def test_fwht_unit_vectors_give_columns():
    H = sylvester(128)
    z = fwht.fwht_blocks(np.eye(128, dtype=np.float32), 128)  # row j = FWHT(e_j)
    assert np.array_equal(z.T.astype(np.int64), H)


def test_fwht_matches_matrix_product_within_fp32_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    z = fwht.fwht_blocks(x, 128).astype(np.float64)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    ref = (x.astype(np.float64).reshape(16, 4, 128) @ H.T).reshape(16, 512)
    bound = 7 * 2.0 ** -24 * (np.abs(x.astype(np.float64)).reshape(16, 4, 128).sum(-1, keepdims=True)
                              * np.ones((1, 1, 128))).reshape(16, 512) * 2
    assert np.all(np.abs(z - ref) <= bound)
    # Parseval: ||z||^2 = 128 ||x||^2 per block (float32 rounding only)
    np.testing.assert_allclose((z.reshape(16, 4, 128) ** 2).sum(-1),
                               128 * (x.astype(np.float64).reshape(16, 4, 128) ** 2).sum(-1), rtol=1e-5)


def test_fwht_involution_on_small_integers():
    rng = np.random.default_rng(4)
    x = rng.integers(-100, 100, size=(3, 256)).astype(np.float32)
    zz = fwht.fwht_blocks(fwht.fwht_blocks(x, 128), 128)
    assert np.array_equal(zz, 128 * x)


def test_inv_sqrt_constant():
    want = int(load("fwht.json")["inv_sqrt_128_f32_bits"], 16)
    assert int(np.array(fwht.inv_sqrt_f32(128), dtype=np.float32).view(np.uint32)) == want


def test_fused_rotation_scale_fold_is_the_normalized_product():
    """Unnormalized z_x . z_w with the 1/128 fold equals x . w (Hadamard is orthogonal up to 128)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    w = rng.standard_normal((3, 256)).astype(np.float32)
    zx = fwht.fwht_blocks(x, 128).astype(np.float64)
    zw = fwht.fwht_blocks(w, 128).astype(np.float64)
    np.testing.assert_allclose(zx @ zw.T / 128.0, x.astype(np.float64) @ w.astype(np.float64).T,
                               rtol=1e-4, atol=1e-4)


# ---------------------------------------------------------------- GEMM and epilogue


def test_int_gemm_worked_example():
    c = load("pack_gemm_epilogue_route.json")["int_gemm"][0]
    acc = gemm.int_gemm(np.array(c["a"], np.int8), np.array(c["b_rows_out"], np.int8))
    assert acc.tolist() == c["acc"]


def test_int_gemm_brute_force():
    rng = np.random.default_rng(8)
    for m, n, k in [(1, 1, 1), (3, 5, 7), (4, 2, 64), (7, 9, 130)]:
        a = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
        b = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
        acc = gemm.int_gemm(a, b)
        for i in range(m):
            for j in range(n):
                s = 0
                for kk in range(k):
                    s += int(a[i, kk]) * int(b[j, kk])
                assert int(acc[i, j]) == s


def test_int_gemm_extreme_magnitude_exact():
    a = np.full((2, 3072), 127, np.int8)
    b = np.full((2, 3072), -127, np.int8)
    assert np.all(gemm.int_gemm(a, b) == -3072 * 127 * 127)
    a = np.zeros((1, 1041 + 64), np.int8)
    a[0, :1041] = 127
    a[0, 1041] = 1
    acc = gemm.int_gemm(a, a)
    assert int(acc[0, 0]) == 1041 * 127 * 127 + 1


@pytest.mark.parametrize("case", load("pack_gemm_epilogue_route.json")["epilogue"], ids=lambda c: c["name"])
def test_epilogue_worked_examples(case):
    acc = [np.array([[case["acc"]]], dtype=np.int32)]
    y, yb = gemm.epilogue(acc, np.array([case["sa"]], np.float32), np.array([case["sw"]], np.float32),
                          True, "bf16")
    assert float(y[0, 0]) == case["y"]
    assert f"0x{int(yb[0, 0]):04X}" == case["bf16_bits"]
    if "fp16_bits" in case:
        _, yh = gemm.epilogue(acc, np.array([case["sa"]], np.float32), np.array([case["sw"]], np.float32),
                              True, "fp16")
        assert f"0x{int(yh.view(np.uint16)[0, 0]):04X}" == case["fp16_bits"]


def test_epilogue_dual_worked_example():
    d = load("pack_gemm_epilogue_route.json")["epilogue_dual"]
    accs = [np.array([[d["acc"][0]]], np.int32), np.array([[d["acc"][1]]], np.int32)]
    y, _ = gemm.epilogue(accs, np.array([d["sa"]], np.float32), np.array([d["sw"]], np.float32), True, "bf16")
    assert float(y[0, 0]) == d["y"]


def test_bf16_and_fp16_rounding_match_torch():
    rng = np.random.default_rng(12)
    f = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        (1 + np.arange(1024, dtype=np.float32) * 2 ** -16).astype(np.float32)])
    ours = numerics.f32_to_bf16_bits(f)
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(numerics.from_f32(f, "fp16"), torch.from_numpy(f).to(torch.float16).numpy())
    back = numerics.bf16_bits_to_f32(theirs)
    assert np.array_equal(back, torch.from_numpy(theirs.view(np.int16)).view(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------- routing


@pytest.mark.parametrize("case", load("pack_gemm_epilogue_route.json")["route"], ids=str)
def test_route_worked_examples(case):
    g = route.relative_l1(np.array(case["x"], np.float32), np.array(case["y"], np.float32))
    assert g == case["gamma"]
    assert route.route_bits(g, case["threshold"]) == case["bits"]


# ---------------------------------------------------------------- whole layer


def _ref_linear(x, w):
    return x.astype(np.float64) @ w.astype(np.float64).T


@pytest.mark.parametrize("wb,ab,had", [(8, 8, 0), (4, 8, 0), (4, 6, 128), (4, 4, 128)])
def test_whole_layer_approximates_float_product(wb, ab, had):
    rng = np.random.default_rng(wb * 10 + ab + had)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    codes, _, sw = oracle.linear.prepare_weights(w, "fp32", wb, had)
    out = oracle.linear.forward(x, "fp32", ab, "token", codes, sw, had, out_dtype="fp32")
    ref = _ref_linear(x, w)
    rel = np.linalg.norm(out["y"] - ref) / np.linalg.norm(ref)
    # expected noise: uniform rounding noise step/sqrt(12) of each operand, with
    # step = amax/Q and amax ~ 3.3 sigma over 512 Gaussian values -> 0.136 for 4 bits,
    # 0.031 for 6 bits, 0.0075 for 8 bits (relative); the bounds allow 25% over that.
    bound = {(8, 8): 0.02, (4, 8): 0.17, (4, 6): 0.18, (4, 4): 0.25}[(wb, ab)]
    assert rel < bound, rel


def test_dual_scale_reduces_error_with_outlier_channels():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    w = (rng.standard_normal((96, 512)) * 0.02).astype(np.float32)
    idx = np.array([3, 100, 300, 411, 500])
    w[:, idx] *= 25
    mask, found, *_ = detect.detect_outliers(w)
    assert found.tolist() == idx.tolist()
    ref = _ref_linear(x, w)
    errs = []
    for oi in (None, found):
        codes, _, sw = oracle.linear.prepare_weights(w, "fp32", 4, 0, oi)
        out = oracle.linear.forward(x, "fp32", 8, "token", codes, sw, 0, oi, out_dtype="fp32")
        errs.append(np.linalg.norm(out["y"] - ref) / np.linalg.norm(ref))
    assert errs[1] < 0.5 * errs[0], errs


def test_dual_split_equals_sum_of_partitions():
    rng = np.random.default_rng(22)
    qa = rng.integers(-127, 128, size=(5, 128)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(6, 128)).astype(np.int8)
    a0, a1 = gemm.accumulators(qa, qw, 64)
    assert np.array_equal(a0.astype(np.int64) + a1, gemm.int_gemm(qa, qw).astype(np.int64))

"""Property tests of the MX route, the static-scale calibration and the step control against
the oracle, over drawn inputs.

Each test draws its shape and options with hypothesis (derandomized, a bounded number of
examples, stopping at the first failure) and holds the device to the same bar as the
hand-picked cases:
- MX quantizer (6Bit-Diffusion, Methodology B.1, in the OCP MX form), plain and with the
  online 128-point block Hadamard: codes and E8M0 scales bit for bit;
- MX GEMM: within the float32 summation bound (K/32 + 2) * 2^-24 * sum|a b| of the
  oracle's exact sum, 16-bit outputs within that bound plus half a 16-bit ulp and equal to
  the float32 result rounded once; shapes with K >= 6144 take the remainder split;
- calibration (Q-ARVD, Technical details: learned clipping percentile and scale) over
  drawn percentile grids: histogram exact, clips and scales bit for bit, errors within
  float64 summation-order rounding, the pick the first minimum of the device errors;
- step control (6Bit-Diffusion, Methodology B.1-B.3) over drawn parameter sets and step
  sequences: E and Gamma within float64 summation-order rounding, the decisions and the
  state equal to the oracle's.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import gen
from oracle import calib, control, mx, numerics, route

pytestmark = pytest.mark.gpu

DEV = "cuda"
TD = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
SETTINGS = dict(deadline=None, derandomize=True, database=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def npb(t):
    return gen.as_numpy_bits(t.cpu())


def pitched(t, pitch):
    """t [rows x cols] on the device inside a zero buffer of row pitch `pitch` elements."""
    rows, cols = t.shape
    buf = torch.zeros((rows, pitch), dtype=t.dtype)
    buf[:, :cols] = t
    return buf.to(DEV)[:, :cols]


def draw_values(g, rows, cols, dist):
    """float32 values of one of the drawn distributions."""
    x = g.standard_normal((rows, cols)).astype(np.float32)
    if dist == "binades":  # 32-element blocks of very different magnitudes
        e = g.integers(-12, 13, size=(rows, (cols + 31) // 32)).repeat(32, axis=1)[:, :cols]
        x *= np.exp2(e).astype(np.float32)
    elif dist == "specials":  # zero blocks, saturating values, signed zeros, tiny values
        x[g.random((rows, cols)) < 0.05] = 0.0
        x[g.random((rows, cols)) < 0.02] = -0.0
        x[g.random((rows, cols)) < 0.02] *= 1e4
        x[g.random((rows, cols)) < 0.02] = 2.0 ** -130
        blk = g.integers(0, max(cols // 32, 1))
        x[:, 32 * blk:32 * blk + 32] = 0.0
    elif dist == "laplace":
        x = (g.laplace(size=(rows, cols)) * 3).astype(np.float32)
    return x


def step_major(scales_rows, rows):
    """Oracle scales [rows x K/32] -> the device's step-major bytes [K/64][rows8][2]."""
    k32 = scales_rows.shape[1]
    r8 = (rows + 7) // 8 * 8
    out = np.zeros((k32 // 2, r8, 2), dtype=np.uint8)
    out[:, :rows, :] = scales_rows.reshape(rows, k32 // 2, 2).transpose(1, 0, 2)
    return out


def device_scales(s, rows, k):
    r8 = (rows + 7) // 8 * 8
    return s.cpu().numpy()[: (k // 64) * r8 * 2].reshape(k // 64, r8, 2)


# ------------------------------------------------------------------ MX quantizer

@st.composite
def mx_quant_cases(draw):
    rotated = draw(st.booleans())
    unit = 128 if rotated else 64
    return dict(rows=draw(st.integers(1, 300)), k=unit * draw(st.integers(1, 30)), rotated=rotated,
                fmt=draw(st.sampled_from(["fp4", "fp6"])), dt=draw(st.sampled_from(["bf16", "fp16"])),
                off=draw(st.sampled_from([0, -7, 3])) if rotated else 0, pad=8 * draw(st.integers(0, 3)),
                dist=draw(st.sampled_from(["normal", "binades", "specials", "laplace"])),
                seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=40, **SETTINGS)
@given(case=mx_quant_cases())
def test_mx_quant_matches_oracle(vq, case):
    print(f"mx quant case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    rows, k, fmt = case["rows"], case["k"], case["fmt"]
    x32 = draw_values(g, rows, k, case["dist"])
    if case["dt"] == "fp16":
        x32 = np.clip(x32, -60000 / 128, 60000 / 128)  # finite in fp16, and after the rotation
    t = gen.to_storage(x32, case["dt"])
    xd = pitched(t, k + case["pad"])
    if case["rotated"]:
        codes, scales = vq.vq_mx_quant(xd, fmt, had_block=128, exp_offset=case["off"])
    else:
        codes, scales = vq.vq_mx_quant(xd, fmt)
    torch.cuda.synchronize()
    xf = numerics.to_f32(npb(t), case["dt"])
    if case["rotated"]:
        rc, rs = mx.quantize_rotated(xf, fmt, exp_offset=case["off"])
    else:
        rc, rs = mx.quantize(xf, fmt)
    assert np.array_equal(codes.cpu().numpy(), mx.pack(rc, fmt)), "codes"
    assert np.array_equal(device_scales(scales, rows, k)[:, :rows], step_major(rs, rows)[:, :rows]), "scales"


# ------------------------------------------------------------------ MX GEMM

@st.composite
def mx_gemm_cases(draw):
    long_k = draw(st.integers(0, 4)) == 0  # about one case in five takes the remainder split
    return dict(m=draw(st.integers(1, 160 if long_k else 520)), n=draw(st.integers(1, 160 if long_k else 520)),
                k=64 * (draw(st.integers(96, 104)) if long_k else draw(st.integers(1, 40))),
                fa=draw(st.sampled_from(["fp4", "fp6"])), rotated=draw(st.booleans()),
                out=draw(st.sampled_from(["fp32", "bf16", "fp16"])),
                dist=draw(st.sampled_from(["normal", "binades", "specials"])),
                seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=30, **SETTINGS)
@given(case=mx_gemm_cases())
def test_mx_gemm_within_float32_bound(vq, case):
    print(f"mx gemm case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    m, n, k, fa = case["m"], case["n"], case["k"], case["fa"]
    rot = case["rotated"] and k % 128 == 0
    x = gen.to_storage(draw_values(g, m, k, case["dist"]), "bf16")
    w = gen.to_storage((g.standard_normal((n, k)) * 0.05).astype(np.float32), "bf16")
    kw_a = dict(had_block=128) if rot else {}
    kw_b = dict(had_block=128, exp_offset=-7) if rot else {}
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), fa, **kw_a)
    bc_d, bs_d = vq.vq_mx_quant(w.to(DEV), "fp4", **kw_b)
    y32 = vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", torch.float32)
    y = y32 if case["out"] == "fp32" else vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", TD[case["out"]])
    torch.cuda.synchronize()
    xf, wf = numerics.to_f32(npb(x), "bf16"), numerics.to_f32(npb(w), "bf16")
    if rot:
        ac, asc = mx.quantize_rotated(xf, fa)
        bc, bsc = mx.quantize_rotated(wf, "fp4", exp_offset=-7)
    else:
        ac, asc = mx.quantize(xf, fa)
        bc, bsc = mx.quantize(wf, "fp4")
    assert np.array_equal(ac_d.cpu().numpy(), mx.pack(ac, fa)), "activation codes"
    exact = mx.gemm(ac, asc, fa, bc, bsc, "fp4")
    mag = np.abs(mx.dequantize(ac, asc, fa)) @ np.abs(mx.dequantize(bc, bsc, "fp4")).T
    bound = (k / 32 + 2) * 2.0 ** -24 * mag
    if case["out"] != "fp32":
        assert torch.equal(y, y32.to(TD[case["out"]])), "16-bit output = float32 output rounded once"
        mant, emin = (7, -126) if case["out"] == "bf16" else (10, -14)
        v = np.abs(exact) + bound
        bound = bound + 0.5 * np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** emin))) - mant)
    err = np.abs(y.float().cpu().numpy().astype(np.float64) - exact)
    assert np.all(err <= bound + 1e-300), float((err / np.maximum(bound, 1e-300)).max())


# ------------------------------------------------------------------ calibration

@st.composite
def calib_cases(draw):
    grid = draw(st.one_of(st.just(None),
                          st.lists(st.floats(50.0, 100.0, allow_nan=False), min_size=1, max_size=64)))
    return dict(rows=draw(st.integers(1, 200)), cols=8 * draw(st.integers(1, 88)),  # rows of whole 16-byte pieces
                dt=draw(st.sampled_from(["bf16", "fp16"])), bits=draw(st.sampled_from([4, 6, 8])),
                dist=draw(st.sampled_from(["normal", "laplace", "outliers", "zeros", "constant"])),
                pad=8 * draw(st.integers(0, 2)), grid=grid, seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=30, **SETTINGS)
@given(case=calib_cases())
def test_calibration_matches_oracle(vq, case):
    print(f"calibration case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    rows, cols, bits = case["rows"], case["cols"], case["bits"]
    if case["dist"] == "laplace":
        x32 = (g.laplace(size=(rows, cols)) * 2).astype(np.float32)
    elif case["dist"] == "zeros":
        x32 = np.zeros((rows, cols), np.float32)
    elif case["dist"] == "constant":
        x32 = np.full((rows, cols), -1.5, np.float32)
    else:
        x32 = g.standard_normal((rows, cols)).astype(np.float32)
        if case["dist"] == "outliers":
            x32[g.integers(0, rows, 4), g.integers(0, cols, 4)] = 200.0
    t = gen.to_storage(x32, case["dt"])
    grid = tuple(calib.GRID if case["grid"] is None else case["grid"])
    xd = pitched(t, cols + case["pad"])
    r = vq.vq_calib_static_scale(xd, bits, percentiles=grid)
    torch.cuda.synchronize()
    store = npb(t)
    hist = r["hist"].cpu().numpy().view(np.uint32)
    want_hist = np.bincount((store.view(np.uint16) & 0x7FFF).reshape(-1), minlength=hist.size)
    assert np.array_equal(hist, want_hist), "histogram"
    o = calib.search(store, case["dt"], bits, grid=grid)
    clips, scales, mse = r["clips"].cpu().numpy(), r["scales"].cpu().numpy(), r["mse"].cpu().numpy()
    assert np.array_equal(clips.view(np.uint32), o["clips"].view(np.uint32)), "clips"
    assert np.array_equal(scales.view(np.uint32), o["scales"].view(np.uint32)), "scales"
    np.testing.assert_allclose(mse, o["mse"], rtol=1e-9, atol=0)
    best = int(r["best"].item())
    assert best == int(np.argmin(mse)), "the first minimum of the device errors"
    srt = np.sort(o["mse"])
    if len(grid) > 1 and srt[1] - srt[0] > 1e-9 * srt[0]:
        assert best == o["best"], "a clear minimum: the oracle's choice"
    assert r["scale"].cpu().numpy().view(np.uint32)[0] == scales[best].view(np.uint32)


# ------------------------------------------------------------------ step control

@st.composite
def control_cases(draw):
    p = dict(skip_threshold=draw(st.sampled_from([0.02, 0.05, 0.1])),
             drift_threshold=draw(st.sampled_from([0.05, 0.12, 0.3])),
             max_skips=draw(st.integers(0, 4)), bits_hi=8, bits_lo=draw(st.sampled_from([4, 6])),
             route_threshold=draw(st.sampled_from([0.05, 0.1, 0.2])),
             outlier_ratio_max=draw(st.sampled_from([0.01, 0.05])))
    steps = draw(st.lists(st.fixed_dictionaries(dict(
        e=st.one_of(st.none(), st.sampled_from([0.0, 0.01, 0.03, 0.07, 0.15, 0.5])),
        gamma=st.one_of(st.none(), st.sampled_from([0.0, 0.03, 0.08, 0.15, 0.4])),
        n_out=st.one_of(st.none(), st.integers(0, 200)))), min_size=1, max_size=10))
    return dict(params=p, steps=steps, n=draw(st.sampled_from([1, 777, 70000])),
                dt=draw(st.sampled_from(["bf16", "fp16", "fp32"])), seed=draw(st.integers(0, 2 ** 31 - 1)))


def near(v, t):
    return abs(v - t) <= 1e-9 * max(abs(t), 1e-300)


@settings(max_examples=25, **SETTINGS)
@given(case=control_cases())
def test_step_control_matches_oracle(vq, case):
    """Each drawn step perturbs a base vector by roughly the drawn relative size; the values
    themselves come from the stored inputs (oracle sums in float64), and a step whose value
    lands within 1e-9 of a threshold keeps only the value comparison (never seen here: the
    inputs are continuous)."""
    print(f"control case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    p = control.Params(**case["params"])
    dp = vq.ControlParams(p.skip_threshold, p.drift_threshold, p.max_skips, p.bits_hi, p.bits_lo,
                          p.route_threshold, p.outlier_ratio_max)
    n, dt = case["n"], case["dt"]
    channels = 1920
    st_dev = vq.vq_control_state(DEV)
    ost = control.State()

    def pair(rel):
        a = g.standard_normal(n).astype(np.float32) + 2.0
        b = a + (rel * 1.25 * np.abs(a).mean()) * g.standard_normal(n).astype(np.float32)
        ta, tb = (torch.from_numpy(v).to(TD[dt]) for v in (a, b))
        fa, fb = ((t.numpy() if dt == "fp32" else numerics.to_f32(npb(t), dt)) for t in (ta, tb))
        return ta.to(DEV), tb.to(DEV), fa, fb

    for i, s in enumerate(case["steps"]):
        kw, oe, og, on = {}, None, None, None
        if s["e"] is not None:
            d_old, d_new, f_old, f_new = pair(s["e"])
            kw.update(delta_old=d_old, delta_new=d_new)
            oe = control.stability(f_new, f_old)
        if s["gamma"] is not None:
            x, y, fx, fy = pair(s["gamma"])
            kw.update(x_prev=x, y_prev=y)
            og = route.relative_l1(fx, fy)
        if s["n_out"] is not None:
            kw.update(n_out_dev=torch.tensor([s["n_out"]], dtype=torch.int32, device=DEV), channels=channels)
            on = s["n_out"]
        skip, bits, e, gm = vq.vq_step_control(st_dev, dp, **kw)
        torch.cuda.synchronize()
        where = f"step {i}"
        if oe is None:
            assert math.isnan(e.item()), where
        else:
            assert e.item() == pytest.approx(oe, rel=1e-12), where
        if og is None:
            assert math.isnan(gm.item()), where
        else:
            assert gm.item() == pytest.approx(og, rel=1e-12), where
        edges = []
        if oe is not None:
            edges += [(oe, p.skip_threshold), (ost.drift + oe, p.drift_threshold)]
        if og is not None:
            edges.append((og, p.route_threshold))
        if any(near(v, t) for v, t in edges):
            return
        oskip, obits, ost = control.step(ost, p, oe, og, on, channels if on is not None else None)
        assert (bool(skip.item()), bits.item()) == (oskip, obits), where
        raw = st_dev.cpu().numpy().view(np.uint8)
        assert int(raw[:4].view(np.int32)[0]) == ost.skips, where
        assert float(raw[8:16].view(np.float64)[0]) == pytest.approx(ost.drift, rel=1e-12, abs=0), where

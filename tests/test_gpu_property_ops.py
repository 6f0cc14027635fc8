"""Property tests of the path's other device operations against the oracle, over drawn inputs.

Each test draws its shape and options with hypothesis (derandomized, a bounded number of
examples, stopping at the first failure) and holds the device result to the same bar as
the hand-picked cases:
- outlier detection (Q-ARVD, Methodology): the column norms within 1e-12 of the oracle's
  float64 norms, and the mask and index list equal to the oracle's flag rule applied to the
  device norms; equal to the oracle's own decision wherever the rule is not within 1e-9 of
  a boundary;
- block Hadamard (6Bit-Diffusion, Methodology B.1): every output bit for bit;
- residual decomposition (SemanticDialect, Methodology 2.2): the stacked operand and every
  output element bit for bit;
- the unquantized layer of the precision override (6Bit-Diffusion, Methodology B.3): within
  the float32 summation bound of the exact sum.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import gen
from oracle import decompose, dense, linear
from oracle import detect as odetect
from oracle import fwht as ofwht
from oracle import numerics as onum
from oracle import quantizer as oq

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


# ------------------------------------------------------------------ outlier detection

@st.composite
def detect_cases(draw):
    return dict(rows=draw(st.integers(1, 48)), cols=draw(st.integers(1, 2500)),
                dt=draw(st.sampled_from(["bf16", "fp16"])),
                ties=draw(st.sampled_from([0.0, 0.3, 0.7])),  # share of columns with one common norm
                spikes=draw(st.integers(0, 12)), spike=draw(st.sampled_from([1.5, 3.0, 10.0])),
                kfac=draw(st.sampled_from([1.0, 0.6745])), tau=draw(st.sampled_from([2.5, 3.5])),
                alpha=draw(st.sampled_from([1.5, 2.0])), pad=draw(st.integers(0, 2)),
                seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=40, **SETTINGS)
@given(case=detect_cases())
def test_detect_matches_oracle(vq, case):
    print(f"detect case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    rows, cols = case["rows"], case["cols"]
    x = g.standard_normal((rows, cols)).astype(np.float32)
    nt = int(case["ties"] * cols)
    if nt:
        x[:, :nt] = x[:, :1]
    if case["spikes"]:
        x[:, g.integers(0, cols, case["spikes"])] *= case["spike"]
    t = gen.to_storage(x, case["dt"])
    xd = pitched(t, (cols + 7) // 8 * 8 + 8 * case["pad"])
    mask, idx, norms = vq.vq_detect_outliers(xd, case["tau"], case["alpha"], case["kfac"])
    v = norms.numpy()
    r = linear.detect_on(npb(t), case["dt"], case["tau"], case["alpha"], case["kfac"])
    np.testing.assert_allclose(v, r["norms"], rtol=1e-12, atol=0)
    fm, fidx, _, _, _ = odetect.flag_outliers(v, case["tau"], case["alpha"], case["kfac"])
    assert np.array_equal(mask.numpy().astype(bool), fm), "mask against the rule on the device norms"
    assert np.array_equal(idx.numpy(), fidx), "indices against the rule on the device norms"
    if odetect.decision_margin(r["norms"], case["tau"], case["alpha"], case["kfac"]) > 1e-9:
        assert np.array_equal(idx.numpy(), r["idx"]), "indices against the oracle"


# ------------------------------------------------------------------ block Hadamard

@st.composite
def hadamard_cases(draw):
    pair = draw(st.sampled_from([("bf16", "bf16"), ("bf16", "fp32"), ("fp16", "fp16"), ("fp16", "bf16"),
                                 ("fp32", "fp32"), ("fp32", "bf16")]))
    return dict(rows=draw(st.integers(1, 300)), blocks=draw(st.integers(1, 24)), din=pair[0], dout=pair[1],
                norm=draw(st.booleans()), pad=draw(st.integers(0, 1)),
                dist=draw(st.sampled_from(["normal", "laplace", "wide"])), seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=40, **SETTINGS)
@given(case=hadamard_cases())
def test_hadamard_matches_oracle(vq, case):
    print(f"hadamard case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    rows, cols = case["rows"], 128 * case["blocks"]
    if case["dist"] == "normal":
        x32 = g.standard_normal((rows, cols)).astype(np.float32)
    elif case["dist"] == "laplace":
        x32 = (g.laplace(size=(rows, cols)) * 3).astype(np.float32)
    else:  # magnitudes spread over many binades
        x32 = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-20, 20, (rows, cols)))).astype(np.float32)
    if case["din"] == "fp16":
        x32 = np.clip(x32, -60000 / 128, 60000 / 128)  # the unnormalized sums stay finite in fp16
    x = torch.from_numpy(x32).to(TD[case["din"]])
    xd = pitched(x, cols + 128 * case["pad"])
    y = vq.vq_hadamard_block(xd, TD[case["dout"]], case["norm"])
    torch.cuda.synchronize()
    xs = npb(x) if case["din"] != "fp32" else x.numpy()
    ref = ofwht.hadamard_block(onum.to_f32(xs, case["din"]), 128, case["norm"])
    want = onum.from_f32(ref, case["dout"])
    got = npb(y) if case["dout"] != "fp32" else y.cpu().numpy()
    assert np.array_equal(got.view(np.uint8), np.asarray(want).view(np.uint8)), "hadamard output"


# ------------------------------------------------------------------ residual decomposition

@st.composite
def residual_cases(draw):
    m = draw(st.integers(1, 600))
    n_rows = draw(st.integers(0, min(m, 40)))
    return dict(m=m, n=draw(st.integers(1, 600)), k=64 * draw(st.integers(1, 16)), n_rows=n_rows,
                bits1=draw(st.sampled_from([4, 6, 8])), bits2=draw(st.sampled_from([4, 8])),
                w_bits=draw(st.sampled_from([4, 8])), dt=draw(st.sampled_from(["bf16", "fp16"])),
                out=draw(st.sampled_from(["bf16", "fp16", "fp32"])), seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=30, **SETTINGS)
@given(case=residual_cases())
def test_residual_layer_matches_oracle(vq, case):
    print(f"residual case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    m, n, k = case["m"], case["n"], case["k"]
    x32 = g.standard_normal((m, k)).astype(np.float32)
    x32[:, g.integers(0, k, 3)] *= 25.0
    x = gen.to_storage(x32, case["dt"])
    w = gen.to_storage((g.standard_normal((n, k)) * 0.02).astype(np.float32), case["dt"])
    rows = g.choice(m, case["n_rows"], replace=False).astype(np.int32)  # distinct, any order
    xd, wd = x.to(DEV), w.to(DEV)
    rd = torch.from_numpy(rows).to(DEV)
    wc, ws = vq.vq_pack_weights(wd, case["w_bits"])
    ac, as_ = vq.vq_quant_act(xd, case["bits1"], "token")
    c2, s2 = vq.vq_quant_residual(xd, rd, case["bits1"], case["bits2"])
    y = vq.vq_qgemm_dequant_residual(ac, as_, wc, ws, case["w_bits"], c2, s2, rd, TD[case["out"]])
    torch.cuda.synchronize()
    xs = npb(x)
    if case["n_rows"]:
        q1, s1 = oq.quant_act(xs, case["dt"], case["bits1"], "token")
        q2, rs2 = decompose.residual_quant(xs, case["dt"], case["bits1"], case["bits2"], rows)
        R = len(rows)
        assert np.array_equal(c2.cpu().numpy()[:R], q1[rows]), "first codes of the listed rows"
        assert np.array_equal(c2.cpu().numpy()[R:], q2), "residual codes"
        assert np.array_equal(s2.cpu().numpy()[R:].view(np.uint32), rs2.view(np.uint32)), "residual scales"
    wcodes, _, wsc = linear.prepare_weights(npb(w), case["dt"], case["w_bits"])
    r = decompose.forward(xs, case["dt"], case["bits1"], case["bits2"], rows, wcodes, wsc, case["out"])
    want = np.asarray(r["y_store"])
    got = y.cpu().numpy() if case["out"] == "fp32" else npb(y)
    u = np.uint32 if case["out"] == "fp32" else np.uint16  # compare bit patterns (signed zeros too)
    bad = np.flatnonzero(got.reshape(-1).view(u) != want.reshape(-1).view(u))
    assert bad.size == 0, f"outputs: {bad.size} mismatches, first at {bad[:5]}"


# ------------------------------------------------------------------ unquantized layer

@st.composite
def dense_cases(draw):
    return dict(m=draw(st.integers(1, 700)), n=draw(st.integers(1, 700)), k=64 * draw(st.integers(1, 24)),
                dt=draw(st.sampled_from(["bf16", "fp16"])), out=draw(st.sampled_from(["bf16", "fp16", "fp32"])),
                scale=draw(st.sampled_from([1.0, 2.0 ** -10, 2.0 ** 6])), seed=draw(st.integers(0, 2 ** 31 - 1)))


@settings(max_examples=30, **SETTINGS)
@given(case=dense_cases())
def test_dense_within_float32_bound(vq, case):
    print(f"dense case: {case}", flush=True)
    g = np.random.default_rng(case["seed"])
    m, n, k = case["m"], case["n"], case["k"]
    x = gen.to_storage((g.standard_normal((m, k)) * case["scale"]).astype(np.float32), case["dt"])
    w = gen.to_storage((g.standard_normal((n, k)) * 0.02).astype(np.float32), case["dt"])
    y = vq.vq_gemm_dense(x.to(DEV), w.to(DEV), TD[case["out"]])
    torch.cuda.synchronize()
    xs, ws = npb(x), npb(w)
    got = y.float().cpu().numpy().astype(np.float64)
    ex = dense.exact(xs, case["dt"], ws)
    b = dense.bound(dense.magnitude(xs, case["dt"], ws), k)
    if case["out"] != "fp32":  # one more rounding: half a 16-bit ulp of the value
        mant, emin = (7, -126) if case["out"] == "bf16" else (10, -14)
        v = np.abs(ex) + b
        b = b + 0.5 * np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** emin))) - mant)
    err = np.abs(got - ex)
    assert np.all(err <= b + 1e-300), float((err / np.maximum(b, 1e-300)).max())

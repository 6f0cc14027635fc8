"""GPU parity of the unquantized FP16/BF16 layer of the precision override
(oracle/dense.py; 6Bit-Diffusion page, Methodology B.3, PDR).

The kernel accumulates in float32 on the matrix cores, so its output is compared with
the oracle's exact sum within the float32 summation bound (k + 2) * 2^-24 * sum|x w|,
plus half an output ulp for 16-bit outputs; on small-integer inputs every partial sum is
exact in float32 and the outputs must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import gen
from oracle import dense
from oracle import numerics as onum

pytestmark = pytest.mark.gpu

DEV = "cuda"
TD = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def npb(t):
    return gen.as_numpy_bits(t.cpu())


def check(y, x_st, w_st, dt, out, rows=None):
    got = y.float().cpu().numpy().astype(np.float64)
    ex = dense.exact(x_st, dt, w_st)
    b = dense.bound(dense.magnitude(x_st, dt, w_st), x_st.shape[1])
    if rows is not None:
        got = got[rows]
    if out != "fp32":
        mant, emin = (7, -126) if out == "bf16" else (10, -14)
        v = np.abs(ex) + b
        b = b + 0.5 * np.exp2(np.floor(np.log2(np.maximum(v, 2.0 ** emin))) - mant)
    err = np.abs(got - ex)
    assert np.all(err <= b + 1e-300), float((err / np.maximum(b, 1e-300)).max())


@pytest.mark.parametrize("m,n,k,dt,out", [
    (1, 1, 64, "bf16", "bf16"),
    (31, 33, 64, "fp16", "fp16"),
    (300, 520, 640, "bf16", "fp32"),
    (257, 255, 192, "fp16", "bf16"),
    (1100, 1030, 128, "bf16", "bf16"),   # 25 tiles, ragged both ways
    (600, 300, 3072, "bf16", "fp16"),
])
def test_dense_within_float32_bound(vq, m, n, k, dt, out):
    rng = np.random.default_rng(m + n + k)
    x = gen.to_storage(rng.standard_normal((m, k)).astype(np.float32), dt)
    w = gen.to_storage((rng.standard_normal((n, k)) * 0.02).astype(np.float32), dt)
    y = vq.vq_gemm_dense(x.to(DEV), w.to(DEV), TD[out])
    torch.cuda.synchronize()
    check(y, npb(x), npb(w), dt, out)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_dense_exact_on_small_integers(vq, dt):
    """Integer inputs in [-8, 8]: every product and partial sum (|sum| < 2^24) is exact in
    float32 in any order, so the stored outputs must equal the oracle's bit for bit."""
    rng = np.random.default_rng(9)
    m, n, k = 520, 300, 1024
    x = gen.to_storage(rng.integers(-8, 9, size=(m, k)).astype(np.float32), dt)
    w = gen.to_storage(rng.integers(-8, 9, size=(n, k)).astype(np.float32), dt)
    for out in ("fp32", dt):
        y = vq.vq_gemm_dense(x.to(DEV), w.to(DEV), TD[out])
        torch.cuda.synchronize()
        _, _, ys = dense.forward(npb(x), dt, npb(w), out)
        got = y.cpu().numpy() if out == "fp32" else npb(y)
        assert np.array_equal(got.reshape(-1).view(np.asarray(ys).dtype), np.asarray(ys).reshape(-1)), out


def test_dense_pitched_operands_and_output(vq):
    """Row slices with wider pitches for x, w and y."""
    rng = np.random.default_rng(11)
    m, n, k = 200, 130, 256
    xf = gen.to_storage(rng.standard_normal((m, k + 64)).astype(np.float32), "bf16")
    wf = gen.to_storage((rng.standard_normal((n, k + 128)) * 0.02).astype(np.float32), "bf16")
    big = torch.empty((m, n + 6), dtype=torch.bfloat16, device=DEV)
    y = vq.vq_gemm_dense(xf.to(DEV)[:, :k], wf.to(DEV)[:, :k], y=big[:, :n])
    torch.cuda.synchronize()
    check(y, npb(xf)[:, :k], npb(wf)[:, :k], "bf16", "bf16")
    y2 = vq.vq_gemm_dense(xf.to(DEV)[:, :k].contiguous(), wf.to(DEV)[:, :k].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(y, y2)  # the same sums, only the layouts differ


def test_dense_fullsize_c2_sampled_rows(vq):
    """The fused-QKV shape (17776 x 1920 x 5760) unquantized, sampled rows against the oracle."""
    x, w = gen.make_x(2), gen.make_w(2)
    y = vq.vq_gemm_dense(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 17775], rng.choice(17776, 20, replace=False)]))
    check(y[torch.from_numpy(rows).to(DEV)], npb(x)[rows], npb(w), "bf16", "bf16")

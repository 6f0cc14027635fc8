"""GPU parity of the MX block-format route (oracle/mx.py; 6Bit-Diffusion page, Methodology
B.1, in the OCP MX form that gfx950's scaled MFMA consumes).

Codes and E8M0 scales are compared bit for bit.  The GEMM accumulates in float32 on the
matrix cores, so its output is compared with the exact sum within the bound of float32
summation over the K/32 block terms: |y - y_exact| <= (K/32 + 2) * 2^-24 * sum_k |a_k b_k|.
"""
import numpy as np
import pytest
import torch

import gen
from oracle import mx, numerics

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def npb(t):
    return gen.as_numpy_bits(t.cpu())


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


def rand_x(m, k, dtype, seed, spread=True):
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    if spread:  # blocks of very different magnitudes
        x *= np.exp2(g.integers(-8, 9, size=(m, k // 32))).repeat(32, axis=1).astype(np.float32)
    return gen.to_storage(x, "bf16" if dtype == torch.bfloat16 else "fp16")


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_mx_quant_bit_exact(vq, fmt, dtype):
    m, k = 300, 640
    x = rand_x(m, k, dtype, 17)
    codes, scales = vq.vq_mx_quant(x.to(DEV), fmt)
    torch.cuda.synchronize()
    name = "bf16" if dtype == torch.bfloat16 else "fp16"
    rc, rs = mx.quantize(numerics.to_f32(npb(x), name), fmt)
    assert np.array_equal(codes.cpu().numpy(), mx.pack(rc, fmt))
    got = device_scales(scales, m, k)
    assert np.array_equal(got[:, :m], step_major(rs, m)[:, :m])


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
@pytest.mark.parametrize("m,k,pad", [(1, 64, 0), (3, 64, 64), (37, 192, 32), (1000, 1920, 128), (9, 12288, 0)])
def test_mx_quant_shapes_and_strides(vq, fmt, m, k, pad):
    """Block numbering over the whole matrix: rows whose block count is not a multiple of
    the 64 blocks a wave takes (waves spanning row ends), a single block pair per row, and
    rows read through a pitch wider than K (a column slice of a wider tensor)."""
    full = rand_x(m, k + pad, torch.bfloat16, m + k + pad)
    x = full.to(DEV)[:, :k]
    assert x.stride(0) == k + pad
    codes, scales = vq.vq_mx_quant(x, fmt)
    torch.cuda.synchronize()
    rc, rs = mx.quantize(numerics.to_f32(npb(full)[:, :k], "bf16"), fmt)
    assert np.array_equal(codes.cpu().numpy(), mx.pack(rc, fmt))
    got = device_scales(scales, m, k)
    assert np.array_equal(got[:, :m], step_major(rs, m)[:, :m])


def test_mx_quant_edge_values(vq):
    k = 128
    x = np.zeros((4, k), np.float32)
    x[0, :32] = 7.0                      # saturates to 6 with X = 1
    x[0, 32:64] = np.linspace(-3, 3, 32)  # ties and both signs
    x[1, 0] = -1e-3                      # lone small value: its own scale
    x[1, 32] = -0.0                      # signed zero in an all-zero block
    x[2] = 2.0 ** -125                   # tiny block (exponent clamps to -127)
    x[3, ::2] = 448.0
    x[3, 1::2] = -0.5                    # -0.5 / 2^6 rounds to -0
    xs = gen.to_storage(x, "bf16")
    for fmt in ("fp4", "fp6"):
        codes, scales = vq.vq_mx_quant(xs.to(DEV), fmt)
        torch.cuda.synchronize()
        rc, rs = mx.quantize(numerics.to_f32(npb(xs), "bf16"), fmt)
        assert np.array_equal(codes.cpu().numpy(), mx.pack(rc, fmt))
        assert np.array_equal(device_scales(scales, 4, k)[:, :4], step_major(rs, 4)[:, :4])


def check_gemm(y, ac, asc, fa, bc, bsc):
    exact = mx.gemm(ac, asc, fa, bc, bsc, "fp4")
    mag = np.abs(mx.dequantize(ac, asc, fa)) @ np.abs(mx.dequantize(bc, bsc, "fp4")).T
    k = ac.shape[1]
    bound = (k / 32 + 2) * 2.0 ** -24 * mag
    err = np.abs(y.astype(np.float64) - exact)
    assert np.all(err <= bound + 1e-300), float((err / np.maximum(bound, 1e-300)).max())
    return exact


@pytest.mark.parametrize("fa", ["fp4", "fp6"])
@pytest.mark.parametrize("m,n,k", [(300, 320, 640), (64, 96, 128), (257, 520, 192)])
def test_mx_gemm_within_float32_bound(vq, fa, m, n, k):
    x = rand_x(m, k, torch.bfloat16, 30 + m)
    w = rand_x(n, k, torch.bfloat16, 40 + n, spread=False)
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), fa)
    bc_d, bs_d = vq.vq_mx_quant(w.to(DEV), "fp4")
    y = vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", torch.float32)
    torch.cuda.synchronize()
    ac, asc = mx.quantize(numerics.to_f32(npb(x), "bf16"), fa)
    bc, bsc = mx.quantize(numerics.to_f32(npb(w), "bf16"), "fp4")
    check_gemm(y.cpu().numpy(), ac, asc, fa, bc, bsc)


def ulp16(v, out):
    """Spacing of the 16-bit output format at |v| (normal range; subnormal spacing below)."""
    mant, emin = (7, -126) if out == torch.bfloat16 else (10, -14)
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return np.exp2(e - mant)


@pytest.mark.parametrize("out", [torch.bfloat16, torch.float16])
def test_mx_gemm_16bit_outputs(vq, out):
    """16-bit outputs against the oracle's exact sum: within the float32 accumulation bound
    plus half a 16-bit ulp (one rounding of the float32 result), and equal to the device's
    own float32 result rounded once."""
    m, n, k = 256, 256, 512
    x = rand_x(m, k, torch.bfloat16, 5)
    w = rand_x(n, k, torch.bfloat16, 6, spread=False)
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), "fp4")
    bc_d, bs_d = vq.vq_mx_quant(w.to(DEV), "fp4")
    y32 = vq.vq_mx_gemm(ac_d, as_d, "fp4", bc_d, bs_d, "fp4", torch.float32)
    y16 = vq.vq_mx_gemm(ac_d, as_d, "fp4", bc_d, bs_d, "fp4", out)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(out))
    ac, asc = mx.quantize(numerics.to_f32(npb(x), "bf16"), "fp4")
    bc, bsc = mx.quantize(numerics.to_f32(npb(w), "bf16"), "fp4")
    exact = mx.gemm(ac, asc, "fp4", bc, bsc, "fp4")
    mag = np.abs(mx.dequantize(ac, asc, "fp4")) @ np.abs(mx.dequantize(bc, bsc, "fp4")).T
    bound = (k / 32 + 2) * 2.0 ** -24 * mag
    got = y16.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - exact)
    assert np.all(err <= bound + 0.5 * ulp16(np.abs(exact) + bound, out))


# ------------------------------------------------------------------ rotated route

@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("off", [0, -7])
def test_mx_quant_rotated_bit_exact(vq, fmt, dtype, off):
    """Rows rotated by the 128-point block Hadamard transform, scaled by 2^off, then MX codes
    and scales: bit for bit against oracle/mx.quantize_rotated."""
    m, k = 300, 640
    x = rand_x(m, k, dtype, 23 + off)
    codes, scales = vq.vq_mx_quant(x.to(DEV), fmt, had_block=128, exp_offset=off)
    torch.cuda.synchronize()
    name = "bf16" if dtype == torch.bfloat16 else "fp16"
    rc, rs = mx.quantize_rotated(numerics.to_f32(npb(x), name), fmt, exp_offset=off)
    assert np.array_equal(codes.cpu().numpy(), mx.pack(rc, fmt))
    assert np.array_equal(device_scales(scales, m, k)[:, :m], step_major(rs, m)[:, :m])


@pytest.mark.parametrize("fmt", ["fp4", "fp6"])
@pytest.mark.parametrize("m,k,pad", [(1, 128, 0), (3, 128, 64), (37, 384, 128), (9, 12288, 0), (1000, 1920, 0)])
def test_mx_quant_rotated_shapes(vq, fmt, m, k, pad):
    """Single rows, a single Hadamard block per row, rows whose block count leaves half a
    wave tile (K = 384: 12 blocks), the widest rows, and a pitch wider than K."""
    full = rand_x(m, k + pad, torch.bfloat16, 3 * m + k + pad)
    x = full.to(DEV)[:, :k]
    codes, scales = vq.vq_mx_quant(x, fmt, had_block=128)
    torch.cuda.synchronize()
    rc, rs = mx.quantize_rotated(numerics.to_f32(npb(full)[:, :k], "bf16"), fmt)
    assert np.array_equal(codes.cpu().numpy(), mx.pack(rc, fmt))
    assert np.array_equal(device_scales(scales, m, k)[:, :m], step_major(rs, m)[:, :m])


@pytest.mark.parametrize("fa", ["fp4", "fp6"])
def test_mx_gemm_rotated_operands(vq, fa):
    """Rotated activations (offset 0) against weights rotated offline (offset -7): the MX GEMM
    output within the float32 bound of the oracle's exact sum of the rotated operands, and
    that sum close to the unrotated float64 product x . w^T."""
    m, n, k = 257, 320, 1024
    x = rand_x(m, k, torch.bfloat16, 61)
    w = rand_x(n, k, torch.bfloat16, 62, spread=False)
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), fa, had_block=128)
    bc_d, bs_d = vq.vq_mx_quant(w.to(DEV), "fp4", had_block=128, exp_offset=-7)
    y = vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", torch.float32)
    torch.cuda.synchronize()
    xf, wf = numerics.to_f32(npb(x), "bf16"), numerics.to_f32(npb(w), "bf16")
    ac, asc = mx.quantize_rotated(xf, fa)
    bc, bsc = mx.quantize_rotated(wf, "fp4", exp_offset=-7)
    exact = check_gemm(y.cpu().numpy(), ac, asc, fa, bc, bsc)
    ref = xf.astype(np.float64) @ wf.astype(np.float64).T
    # Sanity of the composition (rotation, offset -7, no 1/128 in the GEMM): the FP4 weights
    # dominate the quantization error (about 0.1 relative here); a wrong offset would be off
    # by a power of two (relative error >= 0.5).
    rel = np.linalg.norm(exact - ref) / np.linalg.norm(ref)
    assert rel < 0.25, rel


def test_fullsize_w4a4_ffn_down_sampled_rows(vq):
    """17776 x 12288 activations against 3072 x 12288 weights (the FFN-down shape), MXFP4 both."""
    x, w = gen.make_x(4), gen.make_w(4)
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), "fp4")
    bc_d, bs_d = vq.vq_mx_quant(w.to(DEV), "fp4")
    y = vq.vq_mx_gemm(ac_d, as_d, "fp4", bc_d, bs_d, "fp4", torch.float32)
    torch.cuda.synchronize()
    m = x.shape[0]
    rows = np.unique(np.concatenate([[0, 1, 255, 256, m - 1], np.random.default_rng(4).choice(m, 12, replace=False)]))
    ac, asc = mx.quantize(numerics.to_f32(npb(x)[rows], "bf16"), "fp4")
    bc, bsc = mx.quantize(numerics.to_f32(npb(w), "bf16"), "fp4")
    assert np.array_equal(ac_d[torch.from_numpy(rows).to(DEV)].cpu().numpy(), mx.pack(ac, "fp4"))
    check_gemm(y[torch.from_numpy(rows).to(DEV)].cpu().numpy(), ac, asc, "fp4", bc, bsc)


@pytest.mark.parametrize("fa", ["fp4", "fp6"])
def test_mx_gemm_remainder_split(vq, fa):
    """Every tile of a 4-tile GEMM with K = 6144 is split into two K ranges whose float32
    partials are added once: within the same bound, close to the unsplit GEMM, identical
    across calls, and the workspace is left zeroed."""
    m, n, k = 300, 320, 6144
    assert vq._lib.vq_mx_gemm_workspace_bytes(m, n, k) > 0
    x = rand_x(m, k, torch.bfloat16, 77)
    w = rand_x(n, k, torch.bfloat16, 78, spread=False)
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), fa)
    bc_d, bs_d = vq.vq_mx_quant(w.to(DEV), "fp4")
    ws = torch.zeros(vq._lib.vq_mx_gemm_workspace_bytes(m, n, k), dtype=torch.uint8, device=DEV)
    y1 = vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", torch.float32, ws=ws)
    y2 = vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", torch.float32, ws=ws)
    y0 = vq.vq_mx_gemm(ac_d, as_d, fa, bc_d, bs_d, "fp4", torch.float32, ws=False)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert not ws[:4096].any()
    ac, asc = mx.quantize(numerics.to_f32(npb(x), "bf16"), fa)
    bc, bsc = mx.quantize(numerics.to_f32(npb(w), "bf16"), "fp4")
    check_gemm(y1.cpu().numpy(), ac, asc, fa, bc, bsc)
    check_gemm(y0.cpu().numpy(), ac, asc, fa, bc, bsc)

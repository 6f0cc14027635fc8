"""GPU parity of the activation decomposition (SemanticDialect page, Methodology 2.2).

vq_quant_residual and vq_qgemm_dequant_residual are compared with the oracle
(oracle/decompose.py) on the same seeded inputs: the stacked operand (first-quantizer
codes of the listed rows, then their residual codes) and its scales bit for bit, and
every output element bit for bit (the order fl32(y1 + y2), rounded once, is the oracle's).
"""
import numpy as np
import pytest
import torch

import gen
from oracle import decompose, linear
from oracle import quantizer as oq

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


def rand_x(m, k, dtype, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[:, g.integers(0, k, 3)] *= 25.0
    return gen.to_storage(x, "bf16" if dtype == torch.bfloat16 else "fp16")


def rows_t(rows):
    return torch.tensor(rows, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("bits1,bits2", [(8, 8), (4, 4), (8, 4), (6, 8)])
def test_residual_codes_bit_exact(vq, dtype, bits1, bits2):
    m, k = 300, 640
    x = rand_x(m, k, dtype, 100 + bits1 + bits2)
    rows = [0, 1, 150, 255, 256, 299]
    c, s = vq.vq_quant_residual(x.to(DEV), rows_t(rows), bits1, bits2)
    torch.cuda.synchronize()
    name = "bf16" if dtype == torch.bfloat16 else "fp16"
    q1, s1 = oq.quant_act(npb(x), name, bits1, "token")
    q2, rs2 = decompose.residual_quant(npb(x), name, bits1, bits2, rows)
    R = len(rows)
    assert np.array_equal(c.cpu().numpy()[:R], q1[rows])
    assert np.array_equal(s.cpu().numpy()[:R].view(np.uint32), s1[rows].view(np.uint32))
    assert np.array_equal(c.cpu().numpy()[R:], q2)
    assert np.array_equal(s.cpu().numpy()[R:].view(np.uint32), rs2.view(np.uint32))


def test_residual_edge_rows(vq):
    m, k = 64, 256
    x = rand_x(m, k, torch.bfloat16, 7).clone()
    x[3] = 0  # all-zero row: s1 = 0, residual 0
    q = np.random.default_rng(1).integers(-127, 128, k)
    q[0] = 127
    x[5] = torch.from_numpy((q * 2.0 ** -4).astype(np.float32)).to(torch.bfloat16)  # exactly representable
    rows = [3, 5, 63, 9]
    c, s = vq.vq_quant_residual(x.to(DEV), rows_t(rows + [64, -1]), 8, 8)
    torch.cuda.synchronize()
    c2, s2 = c[6:], s[6:]  # residual half of the stacked operand (6 listed rows)
    q2, rs2 = decompose.residual_quant(npb(x), "bf16", 8, 8, rows)
    assert np.array_equal(c2.cpu().numpy()[:4], q2)
    assert np.array_equal(s2.cpu().numpy()[:4], rs2)
    assert not c2[:2].any() and not s2[:2].any()
    # Indices outside [0, m) yield zero codes and scales in both halves.
    assert not c[4:6].any() and not s[4:6].any()
    assert not c2[4:].any() and not s2[4:].any()
    # No listed rows: nothing to do.
    c0, s0 = vq.vq_quant_residual(x.to(DEV), rows_t([]), 8, 8)
    assert c0.numel() == 0 and s0.numel() == 0


@pytest.mark.parametrize("w_bits", [8, 4])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float16, torch.float32])
def test_gemm_with_residual_bit_exact(vq, w_bits, out):
    m, n, k = 300, 320, 640
    x = rand_x(m, k, torch.bfloat16, 5)
    w = (torch.randn(n, k, generator=torch.Generator().manual_seed(6)) * 0.02).to(torch.bfloat16)
    rows = [0, 2, 127, 255, 256, 257, 298, 299]
    xd, wd = x.to(DEV), w.to(DEV)
    wc, ws = vq.vq_pack_weights(wd, w_bits)
    ac, as_ = vq.vq_quant_act(xd, 4, "token")
    c2, s2 = vq.vq_quant_residual(xd, rows_t(rows), 4, 8)
    y = vq.vq_qgemm_dequant_residual(ac, as_, wc, ws, w_bits, c2, s2, rows_t(rows), out)
    torch.cuda.synchronize()
    wcodes, _, wsc = linear.prepare_weights(npb(w), "bf16", w_bits)
    oname = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[out]
    r = decompose.forward(npb(x), "bf16", 4, 8, rows, wcodes, wsc, oname)
    got = npb(y) if out == torch.bfloat16 else y.cpu().numpy()
    want = r["y_store"]
    assert np.array_equal(got.view(np.uint16 if out != torch.float32 else np.uint32),
                          want.view(np.uint16 if out != torch.float32 else np.uint32))
    # Rows outside the set equal the plain GEMM's output.
    plain = vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, None, out, True)
    keep = torch.ones(m, dtype=torch.bool)
    keep[rows] = False
    assert torch.equal(plain[keep.to(DEV)], y[keep.to(DEV)])
    assert not torch.equal(plain[rows_t(rows).long()], y[rows_t(rows).long()])


def test_gemm_with_no_residual_rows_is_the_plain_gemm(vq):
    m, n, k = 128, 192, 256
    x = rand_x(m, k, torch.bfloat16, 9).to(DEV)
    w = (torch.randn(n, k, generator=torch.Generator().manual_seed(10)) * 0.02).to(torch.bfloat16).to(DEV)
    wc, ws = vq.vq_pack_weights(w, 8)
    ac, as_ = vq.vq_quant_act(x, 8, "token")
    e = torch.empty((0, k), dtype=torch.int8, device=DEV)  # no listed rows
    y = vq.vq_qgemm_dequant_residual(ac, as_, wc, ws, 8, e, torch.empty(0, device=DEV), rows_t([]))
    assert torch.equal(y, vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, None, torch.bfloat16, True))


def test_fullsize_c2_with_five_percent_decomposed(vq):
    """The fused-QKV layer (17776 x 1920 -> 5760) with 889 seeded salient tokens."""
    x, w = gen.make_x(2), gen.make_w(2)
    m = x.shape[0]
    rows = np.sort(np.random.default_rng(2024).choice(m, 889, replace=False)).astype(np.int32)
    xd, wd = x.to(DEV), w.to(DEV)
    wc, ws = vq.vq_pack_weights(wd, 8)
    ac, as_ = vq.vq_quant_act(xd, 8, "token")
    rd = torch.from_numpy(rows).to(DEV)
    c2, s2 = vq.vq_quant_residual(xd, rd, 8, 8)
    y = vq.vq_qgemm_dequant_residual(ac, as_, wc, ws, 8, c2, s2, rd, torch.bfloat16)
    torch.cuda.synchronize()
    # Sampled rows: decomposed and plain ones, including both ends.
    pick = np.unique(np.concatenate([rows[:6], rows[-6:], [0, 1, m - 1], rows[::150]]))
    wcodes, _, wsc = linear.prepare_weights(npb(w), "bf16", 8)
    xs = npb(x)[pick]
    sel = np.flatnonzero(np.isin(pick, rows))
    r = decompose.forward(xs, "bf16", 8, 8, sel, wcodes, wsc, "bf16")
    assert np.array_equal(npb(y[torch.from_numpy(pick).to(DEV)]), r["y_store"])
    # The residual codes of the sampled decomposed rows.
    slot = np.searchsorted(rows, pick[sel]) + len(rows)
    q2, rs2 = decompose.residual_quant(npb(x), "bf16", 8, 8, pick[sel])
    assert np.array_equal(c2.cpu().numpy()[slot], q2)
    assert np.array_equal(s2.cpu().numpy()[slot], rs2)

"""GPU parity of the 64-byte K-piece weight layout (VQ_W_KBLOCK).

The layout is defined in include/vq.h: byte c of weight row r's codes sits at
(c / 64) * n * 64 + r * 64 + c % 64.  The tests read the device's pieces back into rows
with that formula written out here (not the binding's helper), compare the packed codes
and scales with the oracle bit for bit, and run every GEMM kernel on both layouts: the
int32 accumulators and the outputs must equal the oracle's, and the two layouts must give
the same bits.  The cases cover each kernel the shapes select: the ping-pong kernel (int8,
more than 16 tiles), the few-tile kernel, the remainder split with int8 and 4-bit weights,
the dual-scale partition staged in 64-code stages and in one 128-code stage (partitions of
64 and 128 codes, the last piece half used), 4-bit weights with 128-code stages and with
64-code stages (K % 128 == 64: a stage reads half a piece), the block Hadamard path, the
scratch-free entry and the residual decomposition.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import decompose

pytestmark = pytest.mark.gpu

DEV = "cuda"
KB = 0x100


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def npb(t):
    return gen.as_numpy_bits(t.cpu())


def rows_of_pieces(flat, n, row_bytes):
    """Row-major [n x row_bytes] bytes of weight codes stored in 64-byte K pieces."""
    r = np.arange(n)[:, None]
    c = np.arange(row_bytes)[None, :]
    return flat[(c // 64) * n * 64 + r * 64 + c % 64]


def assert_same(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}"


def make(m, n, k, n_out, seed):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((m, k)) * np.exp2(g.integers(-2, 3, size=(1, k)))).astype(np.float32)
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    idx = np.sort(g.choice(k, n_out, replace=False)).astype(np.int32) if n_out else None
    if n_out:
        x[:, idx] *= 30.0
    return gen.to_storage(x, "bf16"), gen.to_storage(w, "bf16"), idx


CASES = [
    # name, m, n, k, w_bits, a_bits, n_out, had
    ("pingpong_int8", 1100, 1030, 1920, 8, 8, 0, 0),
    ("pingpong_int8_ragged", 257, 4100, 448, 8, 8, 0, 0),
    ("few_tiles_int8", 300, 200, 320, 8, 8, 0, 0),
    ("split_int8", 1100, 1030, 6144, 8, 8, 0, 0),
    ("dual_int8", 600, 520, 1920, 8, 8, 30, 0),
    ("w4_128code_stages", 600, 520, 1920, 4, 8, 0, 0),
    ("w4_64code_stages", 600, 520, 1984, 4, 6, 0, 0),
    ("dual_w4_part64", 600, 520, 3072, 4, 8, 30, 0),
    ("dual_w4_part128", 300, 260, 3072, 4, 8, 100, 0),
    ("dual_w4_64code_stages", 300, 260, 1984, 4, 8, 30, 0),
    ("split_w4", 1100, 1030, 6144, 4, 6, 0, 0),
    ("hadamard_w4a4", 300, 260, 1024, 4, 4, 0, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kblock_weights_match_oracle_and_row_major(vq, case):
    name, m, n, k, wb, ab, n_out, had = case
    print(f"kblock case: {case}", flush=True)
    x, w, idx = make(m, n, k, n_out, m + n + k + n_out)
    xd, wd = x.to(DEV), w.to(DEV)
    idx_d = None if idx is None else torch.from_numpy(idx).to(DEV)
    wc_r, ws_r = vq.vq_pack_weights(wd, wb, idx_d, had)
    wc_b, ws_b = vq.vq_pack_weights(wd, wb, idx_d, had, kblock=True)
    ac, as_ = vq.vq_quant_act(xd, ab, "token", had, idx_d)
    kp = ac.shape[1]
    k0 = k if n_out else kp
    row_bytes = kp if wb == 8 else kp // 2
    assert tuple(wc_b.shape) == ((row_bytes + 63) // 64, n, 64)
    assert wc_b.numel() == vq.vq_weight_bytes(n, kp, wb | KB)
    y_r, acc_r = vq.vq_qgemm_dequant(ac, as_, wc_r, ws_r, wb, k0, torch.bfloat16, acc_debug=True)
    y_b, acc_b = vq.vq_qgemm_dequant(ac, as_, wc_b, ws_b, wb, k0, torch.bfloat16, acc_debug=True)
    torch.cuda.synchronize()

    # Packed codes and scales: the pieces read back into rows equal the oracle's packing.
    _, rpacked, rscales = oracle.linear.prepare_weights(npb(w), "bf16", wb, had, idx)
    flat = wc_b.cpu().numpy().reshape(-1).view(np.uint8)
    assert_same(rows_of_pieces(flat, n, row_bytes), np.asarray(rpacked).view(np.uint8), "packed codes in pieces")
    assert_same(ws_b.cpu().numpy(), rscales, "scales")
    assert_same(vq.vq_kblock_to_rows(wc_b, n, row_bytes).cpu().numpy().view(np.uint8),
                np.asarray(rpacked).view(np.uint8), "binding's row view")

    # Accumulators and outputs: the oracle's, and the row-major layout's bit for bit.
    wcodes, _, wscales = oracle.linear.prepare_weights(npb(w), "bf16", wb, had, idx)
    r = oracle.linear.forward(npb(x), "bf16", ab, "token", wcodes, wscales, had, idx, out_dtype="bf16")
    for p, want in enumerate(r["accs"]):
        assert_same(acc_b[p].cpu().numpy(), want, f"accumulators, partition {p}")
    assert_same(npb(y_b), r["y_store"], "outputs")
    assert torch.equal(acc_b, acc_r) and torch.equal(y_b.view(torch.int16), y_r.view(torch.int16))


@pytest.mark.parametrize("wb", [8, 4])
def test_kblock_weights_scratch_free_entry(vq, wb):
    """The scratch-free GEMM (its split in the library's static array) on K-piece weights."""
    m, n, k = 1100, 1030, 6144
    x, w, _ = make(m, n, k, 0, 7 + wb)
    wc_b, ws_b = vq.vq_pack_weights(w.to(DEV), wb, kblock=True)
    ac, as_ = vq.vq_quant_act(x.to(DEV), 8, "token")
    y_b = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    vq.vq_qgemm_dequant_noalloc(ac, as_, wc_b, ws_b, wb, y_b)
    torch.cuda.synchronize()
    wcodes, _, wscales = oracle.linear.prepare_weights(npb(w), "bf16", wb)
    r = oracle.linear.forward(npb(x), "bf16", 8, "token", wcodes, wscales, out_dtype="bf16")
    assert_same(npb(y_b), r["y_store"], "outputs")


def test_kblock_weights_residual_decomposition(vq):
    """Decomposed rows added back on K-piece weights: every output bit for bit."""
    m, n, k = 700, 600, 1024
    x, w, _ = make(m, n, k, 0, 11)
    rows = np.random.default_rng(5).choice(m, 40, replace=False).astype(np.int32)
    xd = x.to(DEV)
    rd = torch.from_numpy(rows).to(DEV)
    wc_b, ws_b = vq.vq_pack_weights(w.to(DEV), 8, kblock=True)
    ac, as_ = vq.vq_quant_act(xd, 4, "token")
    c2, s2 = vq.vq_quant_residual(xd, rd, 4, 8)
    y = vq.vq_qgemm_dequant_residual(ac, as_, wc_b, ws_b, 8, c2, s2, rd, torch.bfloat16)
    torch.cuda.synchronize()
    wcodes, _, wsc = oracle.linear.prepare_weights(npb(w), "bf16", 8)
    r = decompose.forward(npb(x), "bf16", 4, 8, rows, wcodes, wsc, "bf16")
    assert_same(npb(y), np.asarray(r["y_store"]), "outputs")


def test_kblock_binding_checks(vq):
    """A K-piece tensor of the wrong dtype or piece count is refused before any launch, and
    either layout gives the same output."""
    w = (torch.randn(64, 256) * 0.02).to(torch.bfloat16).to(DEV)
    ac, as_ = vq.vq_quant_act(torch.randn(32, 256).to(torch.bfloat16).to(DEV), 8, "token")
    wc8, ws8 = vq.vq_pack_weights(w, 8, kblock=True)
    wc4, ws4 = vq.vq_pack_weights(w, 4, kblock=True)
    assert tuple(wc8.shape) == (4, 64, 64) and tuple(wc4.shape) == (2, 64, 64)
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc8[:3].contiguous(), ws8, 8)  # a piece short
    with pytest.raises(TypeError):
        vq.vq_qgemm_dequant(ac, as_, wc4, ws4, 8)  # 4-bit pieces read as int8
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc4.view(torch.int8), ws4, 8)  # int8 pieces of the wrong count
    with pytest.raises(TypeError):
        vq.vq_qgemm_dequant(ac, as_, wc8.view(torch.uint8), ws8, 8)  # wrong dtype
    y8 = vq.vq_qgemm_dequant(ac, as_, wc8, ws8, 8)
    y4 = vq.vq_qgemm_dequant(ac, as_, wc4, ws4, 4)
    torch.cuda.synchronize()
    r8, rs8 = vq.vq_pack_weights(w, 8)
    r4, rs4 = vq.vq_pack_weights(w, 4)
    assert torch.equal(y8, vq.vq_qgemm_dequant(ac, as_, r8, rs8, 8))
    assert torch.equal(y4, vq.vq_qgemm_dequant(ac, as_, r4, rs4, 4))


# ------------------------------------------------------------------ MX weights in K pieces

MX_CASES = [
    # name, m, n, k, activation format, rotated operands
    ("fp4_two_substeps", 300, 320, 640, "fp4", False),   # K % 128 == 0: 128-deep stages, ping-pong
    ("fp4_one_substep", 257, 520, 192, "fp4", False),    # K % 128 == 64: 64-deep stages, last piece half used
    ("fp6", 300, 320, 640, "fp6", False),                # FP6 activations: 64-deep stages
    ("fp6_ragged", 257, 520, 192, "fp6", False),
    ("fp4_rotated", 257, 320, 1024, "fp4", True),
    ("fp6_rotated", 257, 320, 1024, "fp6", True),
    ("fp4_split", 300, 320, 6144, "fp4", False),         # remainder split through the workspace
    ("fp6_split", 300, 320, 6144, "fp6", False),
]


@pytest.mark.parametrize("case", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mx_kblock_weights_match_oracle_and_row_major(vq, case):
    """MXFP4 weights in 64-byte K pieces: the pieces read back into rows are the oracle's
    packed codes, the scales are unchanged, and the GEMM gives the row-major layout's
    output bit for bit, within the float32 summation bound of the oracle's exact sum."""
    from oracle import mx, numerics
    name, m, n, k, fa, rot = case
    print(f"mx kblock case: {case}", flush=True)
    g = np.random.default_rng(m + n + k)
    x32 = g.standard_normal((m, k)).astype(np.float32)
    x32 *= np.exp2(g.integers(-8, 9, size=(m, k // 32))).repeat(32, axis=1).astype(np.float32)
    x = gen.to_storage(x32, "bf16")
    w = gen.to_storage(g.standard_normal((n, k)).astype(np.float32), "bf16")
    kw_a = dict(had_block=128) if rot else {}
    kw_b = dict(had_block=128, exp_offset=-7) if rot else {}
    ac_d, as_d = vq.vq_mx_quant(x.to(DEV), fa, **kw_a)
    bc_r, bs_r = vq.vq_mx_quant(w.to(DEV), "fp4", **kw_b)
    bc_b, bs_b = vq.vq_mx_quant(w.to(DEV), "fp4", kblock=True, **kw_b)
    y_r = vq.vq_mx_gemm(ac_d, as_d, fa, bc_r, bs_r, "fp4", torch.float32)
    y_b = vq.vq_mx_gemm(ac_d, as_d, fa, bc_b, bs_b, "fp4", torch.float32)
    y16 = vq.vq_mx_gemm(ac_d, as_d, fa, bc_b, bs_b, "fp4", torch.bfloat16)
    torch.cuda.synchronize()
    assert tuple(bc_b.shape) == ((k // 2 + 63) // 64, n, 64)
    xf, wf = numerics.to_f32(npb(x), "bf16"), numerics.to_f32(npb(w), "bf16")
    if rot:
        ac, asc = mx.quantize_rotated(xf, fa)
        bc, bsc = mx.quantize_rotated(wf, "fp4", exp_offset=-7)
    else:
        ac, asc = mx.quantize(xf, fa)
        bc, bsc = mx.quantize(wf, "fp4")
    assert_same(rows_of_pieces(bc_b.cpu().numpy().reshape(-1), n, k // 2), mx.pack(bc, "fp4"), "codes in pieces")
    assert torch.equal(bs_b, bs_r), "scales"
    assert torch.equal(y_b, y_r), "outputs of the two layouts"
    assert torch.equal(y16, y_b.to(torch.bfloat16)), "16-bit output = float32 output rounded once"
    exact = mx.gemm(ac, asc, fa, bc, bsc, "fp4")
    mag = np.abs(mx.dequantize(ac, asc, fa)) @ np.abs(mx.dequantize(bc, bsc, "fp4")).T
    bound = (k / 32 + 2) * 2.0 ** -24 * mag
    err = np.abs(y_b.cpu().numpy().astype(np.float64) - exact)
    assert np.all(err <= bound + 1e-300), float((err / np.maximum(bound, 1e-300)).max())

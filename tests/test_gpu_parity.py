"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer results (codes, packed nibbles, masks, outlier indices, int32 accumulators,
routed bit widths) must match bit for bit.  Float scales are produced by the same
float32 operations on both sides and must match bit for bit too.  Outputs are checked
against the published gate (max relative error 2e-3 elementwise) and, because the
epilogue is pinned to one float32 operation order, also for bitwise identity.

Sizes: small cases span several 256 x 256 GEMM tiles with ragged M and N tails; the
full workload shapes are checked on sampled rows that the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import detect as odetect
from oracle import fwht as ofwht
from oracle import gemm as ogemm
from oracle import numerics as onum
from oracle import quantizer as oq
from oracle import route as oroute

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


def dtname(t):
    return {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[t.dtype]


def assert_same(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: {got.reshape(-1)[bad[:5]]} vs {want.reshape(-1)[bad[:5]]}"


def out_f32(t):
    return onum.to_f32(npb(t), dtname(t)) if t.dtype != torch.float32 else t.cpu().numpy()


def assert_outputs(y_gpu, y_ref_store, out_dtype, what):
    """The 2e-3 relative gate, plus bitwise identity of the stored outputs."""
    got = out_f32(y_gpu)
    ref = onum.to_f32(y_ref_store, out_dtype)
    err = np.abs(got.astype(np.float64) - ref)
    tol = 2e-3 * np.abs(ref.astype(np.float64))
    assert np.all((err <= tol) | ((ref == 0) & (got == 0))), f"{what}: gate violated, max rel {np.max(err / np.maximum(np.abs(ref), 1e-30))}"
    assert_same(npb(y_gpu) if out_dtype != "fp32" else y_gpu.cpu().numpy(), y_ref_store, what + " (bitwise)")


# ------------------------------------------------------------------ activation quantization


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_quant_per_token_c2_small(vq, bits):
    x = gen.make_x(2, m=549)
    codes, scales = vq.vq_quant_act(x.to(DEV), bits, "token")
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(x), "bf16", bits, "token")
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scales")


def test_quant_per_tensor_c1_full(vq):
    x = gen.make_x(1)
    codes, scales = vq.vq_quant_act(x.to(DEV), 8, "tensor")
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(x), "fp16", 8, "tensor")
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scale")


@pytest.mark.parametrize("m,k,dt,bits,pitch", [
    (1, 64, "fp16", 8, 0),       # one piece row: the smallest tensor
    (3, 192, "bf16", 6, 0),
    (70, 512, "bf16", 4, 64),    # rows with a wider pitch than K
    (512, 512, "fp16", 8, 0),    # 2^18 elements: the largest one-launch tensor
    (513, 512, "fp16", 8, 0),    # one row more: the two-pass path
    (600, 1024, "bf16", 6, 0),   # the flat maximum pass over contiguous rows
    (700, 1024, "fp16", 8, 128), # ... and over rows with a wider pitch
])
def test_quant_per_tensor_one_launch_and_two_pass(vq, m, k, dt, bits, pitch):
    """Dynamic per-tensor scales: tensors of at most 2^18 elements are quantized in one
    launch (every workgroup reduces the whole maximum), larger ones by a maximum pass and
    a code pass; both must give the oracle's codes and scale, also with the width read
    from the device."""
    g = np.random.default_rng(m * 7 + k)
    x32 = g.standard_normal((m, k + pitch)).astype(np.float32)
    x32[g.integers(0, m), g.integers(0, k)] = 9.0  # one large element sets the scale
    xs = gen.to_storage(x32, dt)
    xv = xs.to(DEV)[:, :k]
    for bd in (None, torch.tensor([bits], dtype=torch.int32, device=DEV)):
        codes, scales = vq.vq_quant_act(xv, 8 if bd is not None else bits, "tensor", bits_dev=bd)
        torch.cuda.synchronize()
        rc, rs = oq.quant_act(npb(xs)[:, :k], dt, bits, "tensor")
        assert_same(codes.cpu().numpy(), rc, f"codes ({'device' if bd is not None else 'host'} width)")
        assert_same(scales.cpu().numpy(), rs, "scale")
    zero = torch.zeros((m, k), dtype=xs.dtype, device=DEV)
    codes, scales = vq.vq_quant_act(zero, bits, "tensor")
    torch.cuda.synchronize()
    assert not codes.any() and scales.item() == 0.0


def test_quant_static_scale(vq):
    x = gen.make_x(1)
    s = torch.tensor([0.05], dtype=torch.float32)
    codes, scales = vq.vq_quant_act(x.to(DEV), 8, "static", static_scale=s.to(DEV))
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(x), "fp16", 8, "static", static_scale=s.numpy())
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scale")
    assert np.abs(rc).max() == 127  # the static scale clips


@pytest.mark.parametrize("dual", [False, True])
def test_quant_static_scale_one_launch(vq, dual):
    """Static per-tensor scales in one launch (the code pass also stores the given scales):
    codes and stored scales against the oracle over many workgroups, with the outlier
    partition's second scale, and with the scale output aliasing the given scales."""
    x = gen.make_x(3, m=700)
    idx = gen.w_outlier_channels(3).astype(np.int32) if dual else None
    idx_d = None if idx is None else torch.from_numpy(idx).to(DEV)
    s = torch.tensor([0.03, 0.6][: 2 if dual else 1], dtype=torch.float32)
    codes, scales = vq.vq_quant_act(x.to(DEV), 8, "static", idx=idx_d, static_scale=s.to(DEV))
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(x), "bf16", 8, "static", 0, idx, static_scale=s.numpy())
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scales")
    same = s.to(DEV)
    codes2, out = vq.vq_quant_act(x.to(DEV), 8, "static", idx=idx_d, static_scale=same, scales=same)
    torch.cuda.synchronize()
    assert out.data_ptr() == same.data_ptr()
    assert torch.equal(codes2, codes), "codes with the scales aliased"
    assert_same(same.cpu().numpy(), rs, "aliased scales")


@pytest.mark.parametrize("gran", ["token", "tensor"])
def test_quant_dual_c3_small(vq, gran):
    x = gen.make_x(3, m=300)
    idx = gen.w_outlier_channels(3).astype(np.int32)
    codes, scales = vq.vq_quant_act(x.to(DEV), 8, gran, idx=torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(x), "bf16", 8, gran, 0, idx)
    assert codes.shape == (300, 3136)
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scales")


@pytest.mark.parametrize("k,m,n_out,dt,gran", [
    (1088, 5000, 100, "bf16", "token"),   # one wave per row, a partial pass; the grid walks several rows per wave
    (4160, 37, 128, "fp16", "token"),     # two waves per row
    (9216, 21, 77, "bf16", "tensor"),     # four waves per row
    (17408, 9, 128, "bf16", "token"),     # eight waves per row, a partial last pass
    (32768, 5, 50, "fp16", "token"),      # eight waves of four passes
])
def test_quant_dual_row_lengths(vq, k, m, n_out, dt, gran):
    """Dual scale in every row-length regime: outlier channels in every pass (adjacent
    channels inside one 8-element piece, the row's first and last channels), each wave
    owning the outliers of its own passes."""
    rng = np.random.default_rng(k + n_out)
    inner = rng.choice(np.arange(3, k - 2), n_out - 5, replace=False)
    idx = np.sort(np.concatenate([[0, 1, 2, k - 2, k - 1], inner])).astype(np.int32)
    assert len(idx) == n_out and len(np.unique(idx)) == n_out
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, idx] *= 20.0
    t = gen.to_storage(x, dt)
    codes, scales = vq.vq_quant_act(t.to(DEV), 8, gran, idx=torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(t), dt, 8, gran, 0, idx)
    assert_same(codes.cpu().numpy(), rc, f"codes k={k}")
    assert_same(scales.cpu().numpy(), rs, f"scales k={k}")


@pytest.mark.parametrize("bits,gran", [(6, "token"), (8, "token"), (4, "tensor")])
def test_quant_hadamard_c4_small(vq, bits, gran):
    x = gen.make_x(4, m=40)
    codes, scales = vq.vq_quant_act(x.to(DEV), bits, gran, had_block=128)
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(x), "bf16", bits, gran, 128)
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scales")


@pytest.mark.parametrize("k", [64, 128, 1024, 1088, 4160, 8192, 9216, 17408, 32768])
def test_quant_row_lengths(vq, k):
    """Every row-length regime (waves per row 1, 2, 4, 8; partial passes)."""
    rng = np.random.default_rng(k)
    x = gen.to_storage(rng.standard_normal((9, k)).astype(np.float32), "bf16")
    for had in ([0, 128] if k % 128 == 0 else [0]):
        codes, scales = vq.vq_quant_act(x.to(DEV), 8, "token", had_block=had)
        torch.cuda.synchronize()
        rc, rs = oq.quant_act(npb(x), "bf16", 8, "token", had)
        assert_same(codes.cpu().numpy(), rc, f"codes k={k} had={had}")
        assert_same(scales.cpu().numpy(), rs, f"scales k={k} had={had}")


def test_quant_edge_rows(vq):
    """All-zero rows, a single row, exact ties, and fp16 input."""
    x = np.zeros((3, 128), dtype=np.float32)
    x[1, :5] = [1.984375, -0.5, 0.2578125, -0.0234375, 0.0078125]  # ties 16.5, -1.5, 0.5
    x[2, :] = -2.0
    t = gen.to_storage(x, "fp16")
    codes, scales = vq.vq_quant_act(t.to(DEV), 8, "token")
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(t), "fp16", 8, "token")
    assert_same(codes.cpu().numpy(), rc, "codes")
    assert_same(scales.cpu().numpy(), rs, "scales")
    assert rc[1, :5].tolist() == [127, -32, 16, -2, 0] and rs[0] == 0
    one = gen.make_x(2, m=1)
    codes, scales = vq.vq_quant_act(one.to(DEV), 8, "token")
    torch.cuda.synchronize()
    rc, rs = oq.quant_act(npb(one), "bf16", 8, "token")
    assert_same(codes.cpu().numpy(), rc, "codes m=1")


def test_runtime_bits_from_device(vq):
    x = gen.make_x(5, m=70)
    for b in (8, 4, 6):
        bd = torch.tensor([b], dtype=torch.int32, device=DEV)
        codes, scales = vq.vq_quant_act(x.to(DEV), 8, "token", bits_dev=bd)
        torch.cuda.synchronize()
        rc, rs = oq.quant_act(npb(x), "bf16", b, "token")
        assert_same(codes.cpu().numpy(), rc, f"codes bits={b}")
        assert_same(scales.cpu().numpy(), rs, f"scales bits={b}")


# ------------------------------------------------------------------ weights


@pytest.mark.parametrize("cfg,bits,had,dual,n", [(2, 8, 0, False, 320), (1, 8, 0, False, 512),
                                                  (3, 4, 0, True, 320), (3, 4, 0, False, 64),
                                                  (4, 4, 128, False, 96), (5, 4, 0, False, 130)])
def test_pack_weights(vq, cfg, bits, had, dual, n):
    w = gen.make_w(cfg, n=n)
    idx = gen.w_outlier_channels(cfg).astype(np.int32) if dual else None
    codes, scales = vq.vq_pack_weights(w.to(DEV), bits, None if idx is None else torch.from_numpy(idx).to(DEV), had)
    torch.cuda.synchronize()
    rcodes, rpacked, rs = oq.pack_weights(npb(w), dtname(w), bits, had, idx)
    assert_same(codes.cpu().numpy(), rpacked, "packed codes")
    assert_same(scales.cpu().numpy(), rs, "scales")


# ------------------------------------------------------------------ Hadamard


@pytest.mark.parametrize("in_dt,out_dt,norm", [(torch.bfloat16, torch.bfloat16, True),
                                               (torch.bfloat16, torch.float32, False),
                                               (torch.float16, torch.float16, True),
                                               (torch.float32, torch.float32, True)])
def test_hadamard_block(vq, in_dt, out_dt, norm):
    rng = np.random.default_rng(3)
    x32 = (rng.laplace(size=(37, 1152)) * 3).astype(np.float32)
    x = torch.from_numpy(x32).to(in_dt)
    y = vq.vq_hadamard_block(x.to(DEV), out_dt, norm)
    torch.cuda.synchronize()
    ref = ofwht.hadamard_block(onum.to_f32(npb(x), dtname(x)), 128, norm)
    assert_same(npb(y) if out_dt != torch.float32 else y.cpu().numpy(),
                onum.from_f32(ref, dtname(y)), "hadamard output")


def test_hadamard_c4_rows(vq):
    x = gen.make_x(4, m=16)
    y = vq.vq_hadamard_block(x.to(DEV), torch.bfloat16, True)
    torch.cuda.synchronize()
    ref = ofwht.hadamard_block(onum.to_f32(npb(x), "bf16"), 128, True)
    assert_same(npb(y), onum.from_f32(ref, "bf16"), "hadamard c4")


# ------------------------------------------------------------------ GEMM


def run_layer(vq, x, w, a_bits, w_bits, gran="token", had=0, idx=None, out_dtype=torch.bfloat16, acc=True):
    xd, wd = x.to(DEV), w.to(DEV)
    idx_d = None if idx is None else torch.from_numpy(idx).to(DEV)
    wc, ws = vq.vq_pack_weights(wd, w_bits, idx_d, had)
    ac, as_ = vq.vq_quant_act(xd, a_bits, gran, had, idx_d)
    k0 = x.shape[1] if idx is not None else ac.shape[1]
    res = vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, k0, out_dtype, gran == "token", acc_debug=acc)
    torch.cuda.synchronize()
    return (ac, as_, wc, ws) + (res if acc else (res, None))


def oracle_layer(x, w, a_bits, w_bits, gran="token", had=0, idx=None, out_dtype="bf16"):
    wcodes, _, wscales = oracle.linear.prepare_weights(npb(w), dtname(w), w_bits, had, idx)
    return oracle.linear.forward(npb(x), dtname(x), a_bits, gran, wcodes, wscales, had, idx, out_dtype=out_dtype)


@pytest.mark.parametrize("cfg,m,n", [(2, 549, 320), (2, 17, 5760 // 9), (5, 300, 320)])
def test_gemm_w8a8_and_w4a8(vq, cfg, m, n):
    x = gen.make_x(cfg, m=m)
    w = gen.make_w(cfg, n=n)
    wb = 8 if cfg == 2 else 4
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 8, wb)
    r = oracle_layer(x, w, 8, wb)
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "accumulators")
    assert_outputs(y, r["y_store"], "bf16", "output")


def test_gemm_dual_c3_small(vq):
    x = gen.make_x(3, m=300)
    w = gen.make_w(3, n=320)
    mask, idx_t, _ = vq.vq_detect_outliers(w.to(DEV))
    idx = idx_t.numpy()
    assert idx.tolist() == gen.w_outlier_channels(3).tolist()
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 8, 4, idx=idx)
    r = oracle_layer(x, w, 8, 4, idx=idx)
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "partition 0 accumulators")
    assert_same(acc[1].cpu().numpy(), r["accs"][1], "partition 1 accumulators")
    assert_outputs(y, r["y_store"], "bf16", "output")


def test_gemm_dual_two_outlier_steps(vq):
    """An outlier partition of 128 codes (two 64-code steps) with int8 weights."""
    x = gen.make_x(2, m=70)
    w = gen.make_w(2, n=96)
    idx = np.sort(np.random.default_rng(1).choice(1920, 100, replace=False)).astype(np.int32)
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 8, 8, idx=idx)
    r = oracle_layer(x, w, 8, 8, idx=idx)
    assert ac.shape[1] == 1920 + 128
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "partition 0")
    assert_same(acc[1].cpu().numpy(), r["accs"][1], "partition 1")
    assert_outputs(y, r["y_store"], "bf16", "output")


def test_gemm_dual_w4_partition_of_128(vq):
    """4-bit weights with an outlier partition of 128 codes: with K a multiple of 128 the
    main loop takes 128-code stages and the partition is staged as one whole stage."""
    x = gen.make_x(3, m=70)
    w = gen.make_w(3, n=96)
    idx = np.sort(np.random.default_rng(2).choice(3072, 100, replace=False)).astype(np.int32)
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 8, 4, idx=idx)
    r = oracle_layer(x, w, 8, 4, idx=idx)
    assert ac.shape[1] == 3072 + 128
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "partition 0")
    assert_same(acc[1].cpu().numpy(), r["accs"][1], "partition 1")
    assert_outputs(y, r["y_store"], "bf16", "output")


def test_gemm_dual_w4_k_not_multiple_of_128(vq):
    """4-bit weights, dual scale, K = 1984 (31 x 64): the 64-code-stage kernel, with the
    outlier partition staged as one 64-code stage."""
    x = gen.make_x(3, m=70)[:, :1984].contiguous()
    w = gen.make_w(3, n=96)[:, :1984].contiguous()
    idx = np.sort(np.random.default_rng(3).choice(1984, 20, replace=False)).astype(np.int32)
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 8, 4, idx=idx)
    r = oracle_layer(x, w, 8, 4, idx=idx)
    assert ac.shape[1] == 1984 + 64
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "partition 0")
    assert_same(acc[1].cpu().numpy(), r["accs"][1], "partition 1")
    assert_outputs(y, r["y_store"], "bf16", "output")


def test_gemm_hadamard_w4a6_c4_small(vq):
    x = gen.make_x(4, m=40)
    w = gen.make_w(4, n=288)
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 6, 4, had=128)
    r = oracle_layer(x, w, 6, 4, had=128)
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "accumulators")
    assert_outputs(y, r["y_store"], "bf16", "output")


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.float32])
def test_gemm_per_tensor_c1_full(vq, out_dtype):
    x = gen.make_x(1)
    w = gen.make_w(1)
    ac, as_, wc, ws, y, acc = run_layer(vq, x, w, 8, 8, gran="tensor", out_dtype=out_dtype)
    name = "fp16" if out_dtype == torch.float16 else "fp32"
    r = oracle_layer(x, w, 8, 8, gran="tensor", out_dtype=name)
    assert_same(acc[0].cpu().numpy(), r["accs"][0], "accumulators")
    assert_outputs(y, r["y_store"], name, "output")


@pytest.mark.parametrize("m,n,k", [(1, 1, 64), (1, 4, 64), (3, 7, 128), (255, 257, 192), (257, 255, 64),
                                   (513, 100, 320),
                                   (1100, 1030, 128),   # 25 tiles: the tiled kernels, ragged both ways
                                   (4097, 1030, 64)])   # 85 tiles
def test_gemm_ragged_shapes(vq, m, n, k):
    rng = np.random.default_rng(m * 1000 + n)
    qa = torch.from_numpy(rng.integers(-127, 128, size=(m, k)).astype(np.int8))
    qw = rng.integers(-7, 8, size=(n, k)).astype(np.int8)
    sa = torch.from_numpy(rng.uniform(0.001, 0.1, size=m).astype(np.float32))
    sb = torch.from_numpy(rng.uniform(0.001, 0.1, size=n).astype(np.float32))
    for bits in (8, 4):
        b = torch.from_numpy(qw if bits == 8 else oq.pack_int4(qw))
        y, acc = vq.vq_qgemm_dequant(qa.to(DEV), sa.to(DEV), b.to(DEV), sb.to(DEV), bits, None, torch.bfloat16,
                                     True, acc_debug=True)
        torch.cuda.synchronize()
        accs, yf, ys = ogemm.qgemm_dequant(qa.numpy(), sa.numpy(), True, qw, sb.numpy(), k, "bf16")
        assert_same(acc[0].cpu().numpy(), accs[0], f"acc bits={bits}")
        assert_outputs(y, ys, "bf16", f"y bits={bits}")


@pytest.mark.parametrize("m,n,k,out,gran,pitch", [
    (1, 1, 64, torch.bfloat16, "token", 0),
    (31, 33, 320, torch.float16, "token", 0),     # ten 32-deep steps: a partial load batch
    (256, 512, 512, torch.float16, "tensor", 0),  # the 256 x 512 x 512 layer
    (300, 200, 6144, torch.bfloat16, "token", 3), # 192 steps; a row pitch that forbids vector stores
    (97, 130, 1920, torch.float32, "token", 0),
    (1000, 1000, 1920, torch.bfloat16, "token", 0),  # 16 tiles: the largest few-tile shape
    (1025, 1000, 1920, torch.bfloat16, "token", 0),  # 20 tiles: the tiled kernel
])
def test_gemm_few_tiles(vq, m, n, k, out, gran, pitch):
    """Layers of at most 16 tiles of 256 x 256 (int8 weights, no outlier partition) run one
    32 x 32 block per wave with register operands; accumulators and outputs must equal the
    oracle's, as for the tiled kernels."""
    rng = np.random.default_rng(m + n + k)
    qa = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    sa = rng.uniform(0.001, 0.1, size=m if gran == "token" else 1).astype(np.float32)
    sb = rng.uniform(0.001, 0.1, size=n).astype(np.float32)
    big = torch.empty((m, n + pitch), dtype=out, device=DEV)
    y = big[:, :n]
    _, acc = vq.vq_qgemm_dequant(torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV),
                                 torch.from_numpy(qw).to(DEV), torch.from_numpy(sb).to(DEV), 8, None, out,
                                 gran == "token", acc_debug=True, y=y)
    torch.cuda.synchronize()
    accs, yf, ys = ogemm.qgemm_dequant(qa, sa, gran == "token", qw, sb, k, dtname(y))
    assert_same(acc[0].cpu().numpy(), accs[0], "accumulators")
    assert_outputs(y, ys, dtname(y), "output")


def test_gemm_extreme_accumulators(vq):
    """|acc| near the int32 bound of the largest K; int4 path's 16x scaling stays in range."""
    m, n, k = 64, 64, 12288
    qa = torch.full((m, k), 127, dtype=torch.int8)
    qa[1::2] = -127
    qw = np.full((n, k), 7, dtype=np.int8)
    qw[::3] = -7
    sa = torch.ones(m, dtype=torch.float32)
    sb = torch.ones(n, dtype=torch.float32)
    y, acc = vq.vq_qgemm_dequant(qa.to(DEV), sa.to(DEV), torch.from_numpy(oq.pack_int4(qw)).to(DEV), sb.to(DEV),
                                 4, None, torch.float32, True, acc_debug=True)
    torch.cuda.synchronize()
    accs, yf, ys = ogemm.qgemm_dequant(qa.numpy(), sa.numpy(), True, qw, sb.numpy(), k, "fp32")
    assert_same(acc[0].cpu().numpy(), accs[0], "acc")
    assert np.abs(accs[0]).max() == 127 * 7 * 12288


# ------------------------------------------------------------------ detection and routing


def test_detect_full_c3_weights(vq):
    w = gen.make_w(3)
    mask, idx, norms = vq.vq_detect_outliers(w.to(DEV))
    r = oracle.linear.detect_on(npb(w), "bf16")
    assert_same(mask.numpy().astype(bool), r["mask"], "mask")
    assert_same(idx.numpy(), r["idx"], "outlier indices")
    np.testing.assert_allclose(norms.numpy(), r["norms"], rtol=1e-12)
    assert odetect.decision_margin(r["norms"]) > 1e-6


def test_detect_c2_activations_and_kfac(vq):
    x = gen.make_x(2, m=2048)
    for kfac in (1.0, 0.6745):
        mask, idx, norms = vq.vq_detect_outliers(x.to(DEV), 3.5, 2.0, kfac)
        r = oracle.linear.detect_on(npb(x), "bf16", 3.5, 2.0, kfac)
        assert_same(idx.numpy(), r["idx"], f"indices kfac={kfac}")


def test_detect_worked_example(vq):
    # columns whose L2 norms are the first hand-worked vector: one row holding v.
    v = np.array([[1.0, 1.1, 0.9, 1.2, 0.8, 1.05, 6.0, 0.95]], dtype=np.float32)
    t = torch.zeros((1, 16), dtype=torch.float32)
    t[0, :8] = torch.from_numpy(v[0])
    t[0, 8:] = 1.0
    mask, idx, norms = vq.vq_detect_outliers(t.to(torch.float16).to(DEV))
    r = oracle.linear.detect_on(npb(t.to(torch.float16)), "fp16")
    assert_same(idx.numpy(), r["idx"], "indices")


@pytest.mark.parametrize("cols", [1, 2, 7, 1000, 1001, 16384, 20008])
def test_detect_order_statistics_exact(vq, cols):
    """Median and MAD are exact order statistics of the device norms: the flag rule applied
    by the oracle to those same norms gives the same mask and index order, for even and odd
    counts, ties, and counts beyond the LDS-resident case."""
    g = np.random.default_rng(cols)
    rows = 24
    x = g.standard_normal((rows, cols)).astype(np.float32)
    x[:, : cols // 3] = x[:, :1]  # a third of the columns share one norm (ties)
    x[:, g.integers(0, cols, max(1, cols // 50))] *= 8.0
    t = torch.from_numpy(x).to(torch.bfloat16)
    if cols % 8:  # rows must start on 16-byte boundaries: use a padded pitch
        pad = torch.zeros((rows, (cols + 7) // 8 * 8), dtype=torch.bfloat16)
        pad[:, :cols] = t
        xd = pad.to(DEV)[:, :cols]
    else:
        xd = t.to(DEV)
    for kfac in (1.0, 0.6745):
        mask, idx, norms = vq.vq_detect_outliers(xd, 3.5, 2.0, kfac)
        fm, fidx, _, _, _ = odetect.flag_outliers(norms.numpy(), 3.5, 2.0, kfac)
        assert_same(mask.numpy().astype(bool), fm, "mask")
        assert_same(idx.numpy(), fidx, "indices")
    r = oracle.linear.detect_on(npb(t), "bf16")
    np.testing.assert_allclose(norms.numpy(), r["norms"], rtol=1e-12)


@pytest.mark.parametrize("cols", [3000, 5001])
def test_detect_norms_over_many_binades(vq, cols):
    """Column norms spread over sixty binades: the leading digits of the float64 patterns
    differ between columns, so the selection's histograms take the per-lane path as well as
    the wave-aggregated one; median, MAD and flags still match the rule on the device norms
    and the oracle's own decision."""
    g = np.random.default_rng(cols)
    x = g.standard_normal((16, cols)).astype(np.float32)
    x *= np.exp2(g.integers(-30, 30, cols)).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    pad = torch.zeros((16, (cols + 7) // 8 * 8), dtype=torch.bfloat16)
    pad[:, :cols] = t
    mask, idx, norms = vq.vq_detect_outliers(pad.to(DEV)[:, :cols])
    fm, fidx, _, _, _ = odetect.flag_outliers(norms.numpy())
    assert_same(mask.numpy().astype(bool), fm, "mask")
    assert_same(idx.numpy(), fidx, "indices")
    r = oracle.linear.detect_on(npb(t), "bf16")
    np.testing.assert_allclose(norms.numpy(), r["norms"], rtol=1e-12)
    assert_same(idx.numpy(), r["idx"], "indices against the oracle")
    assert idx.numel() > 0


def test_detect_zero_mad(vq):
    """More than half of the norms equal: MAD = 0, so every larger norm above alpha * median is flagged."""
    x = torch.ones((4, 64), dtype=torch.float32)
    x[:, 5] = 3.0
    x[:, 9] = 1.5   # above the median but not above 2 * median
    x[:, 40] = 0.5
    mask, idx, norms = vq.vq_detect_outliers(x.to(torch.float16).to(DEV))
    fm, fidx, _, med, mad = odetect.flag_outliers(norms.numpy())
    assert mad == 0.0
    assert_same(idx.numpy(), np.array([5], np.int32), "indices")
    assert_same(mask.numpy().astype(bool), fm, "mask")


def test_detect_count_on_device(vq):
    w = gen.make_w(3)
    cnt = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    _, idx, _ = vq.vq_detect_outliers(w.to(DEV), n_out_dev=cnt)
    torch.cuda.synchronize()
    assert cnt.item() == idx.numel()


def test_route_pairs_and_tie(vq):
    got_bits = []
    for layer in range(42):
        x, y, g = gen.make_route_pair(5, layer)
        bits, gamma = vq.vq_route_rel_l1(x.to(DEV), y.to(DEV), 0.1, 8, 4)
        torch.cuda.synchronize()
        gr = oroute.relative_l1(onum.to_f32(npb(x), "bf16"), onum.to_f32(npb(y), "bf16"))
        assert gamma.item() == pytest.approx(gr, rel=1e-13)
        assert bits.item() == oroute.route_bits(gr, 0.1)
        got_bits.append(bits.item())
    assert 8 in got_bits and 4 in got_bits
    x = torch.tensor([1, -2, 3, -4], dtype=torch.float32)
    for yv, want in (([2, -2, 3, -4], 4), ([3, -2, 3, -4], 8)):
        bits, gamma = vq.vq_route_rel_l1(x.to(DEV), torch.tensor(yv, dtype=torch.float32).to(DEV), 0.1, 8, 4)
        torch.cuda.synchronize()
        assert bits.item() == want


def test_routed_quant_matches_route(vq):
    """The device route feeds the quantizer with no host round trip."""
    x = gen.make_x(5, m=64)
    for layer in (0, 1, 2, 3):
        xp, yp, g = gen.make_route_pair(5, layer)
        bits, gamma = vq.vq_route_rel_l1(xp.to(DEV), yp.to(DEV), 0.1, 8, 4)
        codes, scales = vq.vq_quant_act(x.to(DEV), 8, "token", bits_dev=bits)
        torch.cuda.synchronize()
        b = oroute.route_bits(oroute.relative_l1(onum.to_f32(npb(xp), "bf16"), onum.to_f32(npb(yp), "bf16")))
        rc, rs = oq.quant_act(npb(x), "bf16", b, "token")
        assert_same(codes.cpu().numpy(), rc, f"codes layer {layer}")


# ------------------------------------------------------------------ determinism


def test_runs_are_bitwise_deterministic(vq):
    x = gen.make_x(3, m=300).to(DEV)
    w = gen.make_w(3, n=320).to(DEV)
    idx = torch.from_numpy(gen.w_outlier_channels(3).astype(np.int32)).to(DEV)
    outs = []
    for _ in range(2):
        wc, ws = vq.vq_pack_weights(w, 4, idx)
        ac, as_ = vq.vq_quant_act(x, 8, "token", 0, idx)
        y = vq.vq_qgemm_dequant(ac, as_, wc, ws, 4, 3072, torch.bfloat16, True)
        torch.cuda.synchronize()
        outs.append((ac.cpu(), as_.cpu(), wc.cpu(), ws.cpu(), y.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))

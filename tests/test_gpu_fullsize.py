"""GPU parity at the full workload shapes, in the launch configuration the benchmark times.

The whole layer runs on the GPU at its real size; the oracle recomputes sampled rows
one by one (per-token quantization and the GEMM rows are row-local, so a sampled row's
codes, scale, accumulators and outputs have exactly one correct value).  Sampled rows
include the first and last rows, both sides of every 256-row tile boundary near them,
and seeded random rows.
"""
import numpy as np
import pytest
import torch

import gen
import oracle
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


def sample_rows(m, seed, n_random=24):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 255, 256, 257, m - 257, m - 256, m - 2, m - 1, (m // 256) * 256 - 1, (m // 256) * 256}
    rows = fixed | set(rng.choice(m, n_random, replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < m), dtype=np.int64)


def check_rows(vq, cfg, x, w, a_bits, w_bits, gran="token", had=0, idx=None, bits_dev=None, seed=0):
    """Run the whole layer on the GPU, then compare sampled rows with the oracle."""
    xd, wd = x.to(DEV), w.to(DEV)
    idx_d = None if idx is None else torch.from_numpy(idx).to(DEV)
    wc, ws = vq.vq_pack_weights(wd, w_bits, idx_d, had)
    ac, as_ = vq.vq_quant_act(xd, a_bits, gran, had, idx_d, bits_dev=bits_dev)
    k0 = x.shape[1] if idx is not None else ac.shape[1]
    y = vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, k0, torch.bfloat16, True)
    torch.cuda.synchronize()

    rcodes, rpacked, rws = oracle.linear.prepare_weights(npb(w), "bf16", w_bits, had, idx)
    assert np.array_equal(wc.cpu().numpy(), rpacked), "packed weights"
    assert np.array_equal(ws.cpu().numpy(), rws), "weight scales"
    rows = sample_rows(x.shape[0], seed)
    xs = npb(x)[rows]
    qa, sa = oq.quant_act(xs, "bf16", a_bits, gran, had, idx)
    assert np.array_equal(ac[torch.from_numpy(rows).to(DEV)].cpu().numpy(), qa), "activation codes"
    assert np.array_equal(as_[torch.from_numpy(rows).to(DEV)].cpu().numpy(), sa), "activation scales"
    accs, yf, ys = ogemm.qgemm_dequant(qa, sa, True, rcodes, rws, k0, "bf16")
    got = npb(y[torch.from_numpy(rows).to(DEV)])
    bad = np.flatnonzero(got.reshape(-1) != ys.reshape(-1))
    gotf = onum.to_f32(got, "bf16").astype(np.float64)
    reff = onum.to_f32(ys, "bf16").astype(np.float64)
    rel = np.max(np.abs(gotf - reff) / np.maximum(np.abs(reff), 1e-30))
    assert rel <= 2e-3, f"relative error {rel}"
    assert bad.size == 0, f"{bad.size} output mismatches in sampled rows"
    return rows


def test_fullsize_c1_w8a8_per_tensor(vq):
    x, w = gen.make_x(1), gen.make_w(1)
    xd, wd = x.to(DEV), w.to(DEV)
    wc, ws = vq.vq_pack_weights(wd, 8)
    ac, as_ = vq.vq_quant_act(xd, 8, "tensor")
    y = vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, None, torch.float16, False)
    torch.cuda.synchronize()
    wcodes, _, wsc = oracle.linear.prepare_weights(npb(w), "fp16", 8)
    r = oracle.linear.forward(npb(x), "fp16", 8, "tensor", wcodes, wsc)
    assert np.array_equal(ac.cpu().numpy(), r["qa"])
    assert np.array_equal(y.cpu().numpy().view(np.uint16), r["y_store"].view(np.uint16))


def test_fullsize_c2_w8a8_fused_qkv(vq):
    check_rows(vq, 2, gen.make_x(2), gen.make_w(2), 8, 8, seed=2)


def test_fullsize_c3_w4a8_dual_scale(vq):
    w = gen.make_w(3)
    _, idx_t, _ = vq.vq_detect_outliers(w.to(DEV))
    idx = idx_t.numpy()
    assert idx.tolist() == oracle.linear.detect_on(npb(w), "bf16")["idx"].tolist()
    check_rows(vq, 3, gen.make_x(3), w, 8, 4, idx=idx, seed=3)


def test_fullsize_c4_w4a6_hadamard(vq):
    check_rows(vq, 4, gen.make_x(4), gen.make_w(4), 6, 4, had=128, seed=4)


def test_fullsize_c4_standalone_hadamard(vq):
    x = gen.make_x(4)
    y = vq.vq_hadamard_block(x.to(DEV), torch.bfloat16, True)
    torch.cuda.synchronize()
    rows = sample_rows(x.shape[0], 44, 16)
    ref = ofwht.hadamard_block(onum.to_f32(npb(x)[rows], "bf16"), 128, True)
    assert np.array_equal(npb(y[torch.from_numpy(rows).to(DEV)]), onum.from_f32(ref, "bf16"))


def oracle_route(layer):
    xp, yp, _ = gen.make_route_pair(5, layer)
    return oroute.route_bits(oroute.relative_l1(onum.to_f32(npb(xp), "bf16"), onum.to_f32(npb(yp), "bf16")))


@pytest.mark.parametrize("layer,route", [(0, 4), (1, 4), (3, 8)])
def test_fullsize_c5_routed_layer(vq, layer, route):
    """One 3072 x 3072 layer of the routed batch on the full 35552-row CFG batch, with the
    width read on the device from the route (layers 0 and 1 route to 4-bit activations,
    layer 3, the first with Gamma above 0.1, to INT8)."""
    xp, yp, _ = gen.make_route_pair(5, layer)
    bits, gamma = vq.vq_route_rel_l1(xp.to(DEV), yp.to(DEV), 0.1, 8, 4)
    torch.cuda.synchronize()
    want = oracle_route(layer)
    assert want == route and bits.item() == want
    check_rows(vq, 5, gen.make_x(5), gen.make_w(5, layer=layer), want, 4, bits_dev=bits, seed=50 + layer)


def test_fullsize_c5_routed_step_42_layers(vq):
    """The whole routed step as the benchmark runs it: 42 layers on the 35552-row batch,
    each routed on the device and quantized with the width read from the route, its GEMM
    writing into one output buffer.  The first two layers of each route are checked on
    sampled rows against the oracle; every route matches the oracle's."""
    c = gen.CONFIGS[5]
    x = gen.make_x(5)
    xd = x.to(DEV)
    m, k = x.shape
    routes = [oracle_route(l) for l in range(c["layers"])]
    checked = [l for l in range(c["layers"]) if routes[l] == 4][:2] + [l for l in range(c["layers"]) if routes[l] == 8][:2]
    assert len(checked) == 4
    rows = sample_rows(m, 500, 12)
    rows_d = torch.from_numpy(rows).to(DEV)
    codes = torch.empty((m, k), dtype=torch.int8, device=DEV)
    scales = torch.empty(m, dtype=torch.float32, device=DEV)
    y = torch.empty((m, c["N"]), dtype=torch.bfloat16, device=DEV)
    seen = {}
    for layer in range(c["layers"]):
        w = gen.make_w(5, layer=layer)
        wc, ws = vq.vq_pack_weights(w.to(DEV), 4)
        xp, yp, _ = gen.make_route_pair(5, layer)
        bits, _ = vq.vq_route_rel_l1(xp.to(DEV), yp.to(DEV), 0.1, 8, 4)
        vq.vq_quant_act(xd, 8, "token", bits_dev=bits, codes=codes, scales=scales)
        vq.vq_qgemm_dequant(codes, scales, wc, ws, 4, y=y)
        assert bits.item() == routes[layer], f"layer {layer}"
        if layer in checked:
            seen[layer] = (w, codes[rows_d].cpu().numpy(), scales[rows_d].cpu().numpy(), npb(y[rows_d]))
    torch.cuda.synchronize()
    for layer, (w, qa_got, sa_got, y_got) in seen.items():
        bits = routes[layer]
        rcodes, _, rws = oracle.linear.prepare_weights(npb(w), "bf16", 4)
        qa, sa = oq.quant_act(npb(x)[rows], "bf16", bits, "token")
        assert np.array_equal(qa_got, qa), f"layer {layer} codes"
        assert np.array_equal(sa_got, sa), f"layer {layer} scales"
        _, _, ys = ogemm.qgemm_dequant(qa, sa, True, rcodes, rws, k, "bf16")
        assert np.array_equal(y_got, ys), f"layer {layer} outputs ({bits}-bit route)"

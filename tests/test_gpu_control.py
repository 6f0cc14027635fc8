"""GPU parity of the per-block step control (6Bit-Diffusion page, Methodology B.1-B.3;
oracle/control.py).

The hand-worked decision table (tests/golden/control.json) is replayed through the
device state with inputs built so that E and Gamma equal the table's values exactly;
on random deltas and block pairs E and Gamma match the oracle within float64
summation-order rounding and the decisions match the oracle's; the outlier count comes
from the device detection.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import gen
from oracle import control, numerics, route

pytestmark = pytest.mark.gpu

DEV = "cuda"
GOLD = os.path.join(os.path.dirname(__file__), "golden", "control.json")


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def params_of(vq, p: control.Params):
    return vq.ControlParams(p.skip_threshold, p.drift_threshold, p.max_skips, p.bits_hi, p.bits_lo,
                            p.route_threshold, p.outlier_ratio_max)


def pair_with_ratio(v, n, dtype=torch.float32):
    """(old, new) with sum|new - old| / sum|old| == v exactly (v dyadic, or 0.1 as 1/10)."""
    if v == "inf":
        return torch.zeros(n, dtype=dtype, device=DEV), torch.ones(n, dtype=dtype, device=DEV)
    if v == 0.1:
        return torch.full((n,), 10.0, dtype=dtype, device=DEV), torch.full((n,), 11.0, dtype=dtype, device=DEV)
    return torch.ones(n, dtype=dtype, device=DEV), torch.full((n,), 1.0 + v, dtype=dtype, device=DEV)


def read_state(st):
    raw = st.cpu().numpy().view(np.uint8)
    return int(raw[:4].view(np.int32)[0]), float(raw[8:16].view(np.float64)[0])


@pytest.mark.parametrize("n", [1, 4096, 1 << 20])
def test_golden_sequences_on_device(vq, n):
    gold = json.load(open(GOLD))
    p = params_of(vq, control.Params(**gold["params"]))
    for seq in gold["sequences"]:
        st = vq.vq_control_state(DEV)
        for i, s in enumerate(seq["steps"]):
            kw = {}
            if s["e"] is not None:
                kw["delta_old"], kw["delta_new"] = pair_with_ratio(s["e"], n)
            if s["gamma"] is not None:
                kw["x_prev"], kw["y_prev"] = pair_with_ratio(s["gamma"], n, torch.bfloat16 if s["gamma"] != 0.1 else
                                                             torch.float32)
            if "n_out" in s:
                kw["n_out_dev"] = torch.tensor([s["n_out"]], dtype=torch.int32, device=DEV)
                kw["channels"] = s["channels"]
            skip, bits, e, g = vq.vq_step_control(st, p, **kw)
            torch.cuda.synchronize()
            where = f'{seq["name"]}, step {i}, n={n}'
            assert (bool(skip.item()), bits.item()) == (s["skip"], s["bits"]), where
            assert read_state(st) == (s["skips"], s["drift"]), where
            if s["e"] is None:
                assert math.isnan(e.item())
            elif s["e"] == "inf":
                assert math.isinf(e.item())
            else:
                assert e.item() == s["e"], where
            if s["gamma"] is None:
                assert math.isnan(g.item())
            else:
                assert g.item() == s["gamma"], where


@pytest.mark.parametrize("dtype,n", [(torch.bfloat16, 1000), (torch.float16, 65536 + 17), (torch.float32, 3 << 20)])
def test_random_blocks_match_oracle(vq, dtype, n):
    g = np.random.default_rng(n)
    name = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[dtype]
    p = control.Params(skip_threshold=0.05, drift_threshold=0.12, max_skips=3, route_threshold=0.1)
    dp = params_of(vq, p)
    st = vq.vq_control_state(DEV)
    ost = control.State()
    base = g.standard_normal(n).astype(np.float32)
    seen = set()
    for step in range(8):
        # Deltas drift slowly for a while, then jump; the block input/output differ by a varying amount.
        scale = 0.02 if step < 5 else 0.3
        d_old = base + scale * g.standard_normal(n).astype(np.float32)
        d_new = d_old + scale * g.standard_normal(n).astype(np.float32)
        x = g.standard_normal(n).astype(np.float32)
        y = x + (0.02 + 0.03 * (step % 4)) * g.standard_normal(n).astype(np.float32)
        ts = {k: torch.from_numpy(v).to(dtype) for k, v in (("d_old", d_old), ("d_new", d_new), ("x", x), ("y", y))}
        f = {k: numerics.to_f32(gen.as_numpy_bits(t), name) if dtype != torch.float32 else t.numpy()
             for k, t in ts.items()}
        skip, bits, e, gm = vq.vq_step_control(st, dp, delta_new=ts["d_new"].to(DEV), delta_old=ts["d_old"].to(DEV),
                                               x_prev=ts["x"].to(DEV), y_prev=ts["y"].to(DEV))
        torch.cuda.synchronize()
        oe = control.stability(f["d_new"], f["d_old"])
        og = route.relative_l1(f["x"], f["y"])
        assert e.item() == pytest.approx(oe, rel=1e-12)
        assert gm.item() == pytest.approx(og, rel=1e-12)
        # Decisions are compared away from the thresholds (the sums differ only in their order).
        for v, t in ((oe, p.skip_threshold), (ost.drift + oe, p.drift_threshold), (og, p.route_threshold)):
            assert abs(v - t) > 1e-9 * max(abs(t), 1e-300)
        oskip, obits, ost = control.step(ost, p, oe, og)
        assert (bool(skip.item()), bits.item()) == (oskip, obits), f"step {step}"
        seen.add(obits)
        sk, dr = read_state(st)
        assert sk == ost.skips and dr == pytest.approx(ost.drift, rel=1e-12)
    assert seen == {0, 4, 8}  # skips, routed 4-bit and forced or routed INT8 steps all occur


def test_outlier_count_from_detection_forces_unquantized(vq):
    w = gen.make_w(3).to(DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    _, idx, _ = vq.vq_detect_outliers(w, n_out_dev=cnt)
    k = w.shape[1]
    assert idx.numel() > 0
    st = vq.vq_control_state(DEV)
    x = torch.ones(256, dtype=torch.bfloat16, device=DEV)
    lo = control.Params(outlier_ratio_max=idx.numel() / k / 2)   # ratio above the limit
    hi = control.Params(outlier_ratio_max=idx.numel() / k * 2)   # ratio below the limit
    skip, bits, _, _ = vq.vq_step_control(st, params_of(vq, lo), x_prev=x, y_prev=x, n_out_dev=cnt, channels=k)
    torch.cuda.synchronize()
    assert skip.item() == 0 and bits.item() == 16
    skip, bits, _, g = vq.vq_step_control(st, params_of(vq, hi), x_prev=x, y_prev=x, n_out_dev=cnt, channels=k)
    torch.cuda.synchronize()
    assert skip.item() == 0 and bits.item() == 4 and g.item() == 0.0


def test_routed_bits_feed_the_quantizer(vq):
    """The decision's width goes to vq_quant_act's bits_dev with no host round trip."""
    x = gen.make_x(2, m=64).to(DEV)
    st = vq.vq_control_state(DEV)
    p = params_of(vq, control.Params(route_threshold=0.1, bits_hi=8, bits_lo=4))
    a = torch.ones(128, dtype=torch.float32, device=DEV)
    _, bits, _, _ = vq.vq_step_control(st, p, x_prev=a, y_prev=a * 1.5)   # Gamma 0.5 -> 8
    c8, s8 = vq.vq_quant_act(x, 4, "token", bits_dev=bits)
    r8, rs8 = vq.vq_quant_act(x, 8, "token")
    _, bits, _, _ = vq.vq_step_control(st, p, x_prev=a, y_prev=a)         # Gamma 0 -> 4
    c4, s4 = vq.vq_quant_act(x, 8, "token", bits_dev=bits)
    r4, rs4 = vq.vq_quant_act(x, 4, "token")
    torch.cuda.synchronize()
    assert torch.equal(c8, r8) and torch.equal(s8, rs8)
    assert torch.equal(c4, r4) and torch.equal(s4, rs4)

"""The remainder split of the integer GEMM is bit-identical to the unsplit GEMM.

Tiles past the last whole round of the persistent grid are split into two K ranges
whose int32 partials meet in a workspace (integer sums are exact in any order).
Outputs and raw accumulators are compared with the same GEMM run without the
workspace, for int8 and int4 weights (64- and 128-code stages), the dual-scale outlier
partition, ragged tiles and float32 outputs, and for a shape whose leftover tiles are
too many to split; repeated calls check that each call leaves the workspace zeroed.
"""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def operands(vq, m, n, k, w_bits, a_bits, seed, dual=False):
    g = torch.Generator(device=DEV).manual_seed(seed)  # drawn on the device: the shapes are large
    x = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    idx = None
    if dual:
        idx = torch.tensor(sorted(np.random.default_rng(seed).choice(k, 20, replace=False)), dtype=torch.int32,
                           device=DEV)
    wc, ws = vq.vq_pack_weights(w, w_bits, idx=idx)
    ac, as_ = vq.vq_quant_act(x, a_bits, "token", idx=idx)
    return ac, as_, wc, ws


@pytest.mark.parametrize("m,n,k,w_bits,dual,out", [
    (17776, 3072, 12288, 4, False, torch.bfloat16),  # 840 tiles: 72 left over, 128-code stages
    (300, 4400, 6144, 8, False, torch.float16),      # 36 tiles, ragged M and N
    (1000, 900, 8192, 4, False, torch.bfloat16),     # 16 tiles, 4-bit weights in 128-code stages
    (600, 520, 6144, 4, True, torch.float32),        # dual-scale outlier partition, 9 tiles
    (520, 33000, 6144, 8, True, torch.bfloat16),     # 387 tiles: 131 left over (one range each), dual
    (512, 33280, 8192, 8, False, torch.bfloat16),    # 260 tiles: 4 left over
])
def test_split_equals_unsplit(vq, m, n, k, w_bits, dual, out):
    ac, as_, wc, ws = operands(vq, m, n, k, w_bits, 8, m + n + k, dual)
    k0 = k
    need = vq._lib.vq_qgemm_workspace_bytes(m, n, k0)
    if need == 0:  # too many leftover tiles for two ranges each: the plain GEMM either way
        y0 = vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, k0, out, True, ws=False)
        assert torch.equal(y0, vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, k0, out, True))
        return
    y0, a0 = vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, k0, out, True, acc_debug=True, ws=False)
    for rep in range(3):
        y1, a1 = vq.vq_qgemm_dequant(ac, as_, wc, ws, w_bits, k0, out, True, acc_debug=True)
        torch.cuda.synchronize()
        assert torch.equal(a0, a1), f"accumulators, call {rep}"
        assert torch.equal(y0.view(torch.int16) if out != torch.float32 else y0.view(torch.int32),
                           y1.view(torch.int16) if out != torch.float32 else y1.view(torch.int32)), f"call {rep}"
    # Every call leaves the arrival counters at zero.
    wsb = vq._GEMM_WS[(ac.device, torch.cuda.current_stream(ac.device).cuda_stream)]
    assert not wsb[:4096].any()


def test_caller_workspace_and_no_split_shape(vq):
    m, n, k = 512, 4608, 6144  # 36 tiles
    ac, as_, wc, ws = operands(vq, m, n, k, 8, 8, 3)
    need = vq._lib.vq_qgemm_workspace_bytes(m, n, k)
    buf = torch.zeros(need, dtype=torch.uint8, device=DEV)
    y1 = vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, ws=buf)
    y0 = vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, ws=False)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and not buf[:4096].any()
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, ws=buf[: need // 2])

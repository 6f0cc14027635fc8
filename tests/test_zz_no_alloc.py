"""The scratch-free GEMM entry point against the one that takes a workspace.

vq_qgemm_dequant_noalloc, called through the C ABI with caller-allocated inputs and
outputs only, must reproduce vq_qgemm_dequant bit for bit: on two calls in a row (the
second with a smaller input, so that the static scratch holds the first call's state) and
on shapes with and without the remainder split that uses the scratch.
"""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16, F16, F32 = 1, 0, 2


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _operands(vq, m, n, k, b_bits, n_out, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    idx = None
    if n_out:
        idx = torch.sort(torch.randperm(k, generator=torch.Generator().manual_seed(seed))[:n_out])[0]
        idx = idx.to(torch.int32).to(DEV)
    wc, ws = vq.vq_pack_weights(w, b_bits, idx)
    ac, as_ = vq.vq_quant_act(x, 8, "token", idx=idx)
    return ac, as_, wc, ws


def _reference(vq, ac, as_, wc, ws, b_bits, k0, out_dt, y):
    m, kp = ac.shape
    n = wc.shape[0]
    need = int(vq._lib.vq_qgemm_workspace_bytes(m, n, k0))
    wsp = torch.zeros(max(need, 16), dtype=torch.uint8, device=DEV)
    st = vq._lib.vq_qgemm_dequant(_p(ac), _p(as_), 1, _p(wc), b_bits, _p(ws), m, n, kp, k0, _p(y), out_dt,
                                  y.stride(0), None, _p(wsp) if need else None, None)
    assert st == 0
    return need


def _noalloc(vq, ac, as_, wc, ws, b_bits, k0, out_dt, y):
    m, kp = ac.shape
    n = wc.shape[0]
    return vq._lib.vq_qgemm_dequant_noalloc(_p(ac), _p(as_), 1, _p(wc), b_bits, _p(ws), m, n, kp, k0, _p(y),
                                            out_dt, y.stride(0), None)


# (first call, second smaller call): (m, n, k, weight bits, outlier channels, output dtype)
CASES = [
    # both shapes take the remainder split (K of 96 stages), so the scratch is used twice
    ((300, 4400, 6144, 8, 0, BF16), (200, 4352, 6144, 8, 0, BF16)),
    ((520, 640, 8192, 4, 0, F16), (260, 300, 6144, 4, 0, F16)),
    # no split (the ping-pong W8A8 kernel), then a split shape; dual scale with 4-bit weights
    ((1000, 4400, 1920, 8, 0, BF16), (300, 4400, 6144, 8, 0, F32)),
    ((700, 512, 3072, 4, 30, BF16), (300, 320, 6144, 4, 0, BF16)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_matches_workspace_entry(vq, first, second):
    for i, (m, n, k, b_bits, n_out, out_dt) in enumerate((first, second)):
        ac, as_, wc, ws = _operands(vq, m, n, k, b_bits, n_out, seed=1000 * i + m + n + k)
        kp = ac.shape[1]
        k0 = k if n_out else kp
        dt = {BF16: torch.bfloat16, F16: torch.float16, F32: torch.float32}[out_dt]
        y_ref = torch.empty((m, n), dtype=dt, device=DEV)
        y = torch.full((m, n), 7.0, dtype=dt, device=DEV)
        need = _reference(vq, ac, as_, wc, ws, b_bits, k0, out_dt, y_ref)
        assert need <= vq._lib.vq_qgemm_scratch_bytes()
        print(f"noalloc call {i}: m={m} n={n} k={k} b_bits={b_bits} n_out={n_out} workspace={need}", flush=True)
        assert _noalloc(vq, ac, as_, wc, ws, b_bits, k0, out_dt, y) == 0
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16 if dt != torch.float32 else torch.int32),
                           y_ref.view(torch.int16 if dt != torch.float32 else torch.int32)), f"call {i}"


def test_noalloc_rejects_splits_beyond_the_scratch(vq):
    # 356 tiles of 256 x 256 on 256 compute units leave 100, each split into two K ranges
    # (96 stages): 100 x 2 partials of 256 KB, more than the scratch holds; rejected
    # before anything is enqueued (the buffers are real, so nothing could be misread).
    m, n, k = 178 * 256, 512, 6144
    need = int(vq._lib.vq_qgemm_workspace_bytes(m, n, k))
    assert need > vq._lib.vq_qgemm_scratch_bytes()
    a = torch.zeros((m, k), dtype=torch.int8, device=DEV)
    sa = torch.ones(m, dtype=torch.float32, device=DEV)
    b = torch.zeros((n, k), dtype=torch.int8, device=DEV)
    sb = torch.ones(n, dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    st = vq._lib.vq_qgemm_dequant_noalloc(_p(a), _p(sa), 1, _p(b), 8, _p(sb), m, n, k, k, _p(y), BF16, n, None)
    assert st == 2  # VQ_ERR_SHAPE
    with pytest.raises(vq.VQError):
        vq.vq_qgemm_dequant_noalloc(a, sa, b, sb, 8, y)

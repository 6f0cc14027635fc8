"""The Python binding rejects device buffers that the C ABI cannot describe or that are
too small (no kernel is launched on them)."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def vq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_vq_amd as m
    return m


def test_rejects_strided_columns_and_bad_outputs(vq):
    x = torch.randn(64, 256, device=DEV).to(torch.bfloat16)
    with pytest.raises(ValueError):
        vq.vq_quant_act(x.t(), 8)  # column-major view
    with pytest.raises(ValueError):
        vq.vq_quant_act(x, 8, codes=torch.empty((63, 256), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):
        vq.vq_quant_act(x, 8, scales=torch.empty(10, dtype=torch.float32, device=DEV))
    w = torch.randn(128, 256, device=DEV).to(torch.bfloat16)
    wc, ws = vq.vq_pack_weights(w, 8)
    ac, as_ = vq.vq_quant_act(x, 8)
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, y=torch.empty((64, 127), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, y=torch.empty((128, 64), dtype=torch.bfloat16, device=DEV).t())
    with pytest.raises(ValueError):
        vq.vq_calib_static_scale(x, 8, hist=torch.empty(100, dtype=torch.int32, device=DEV))
    with pytest.raises(TypeError):
        vq.vq_quant_act(x.cpu(), 8)
    # A row slice with a wider pitch is a valid output.
    big = torch.empty((64, 192), dtype=torch.bfloat16, device=DEV)
    y = vq.vq_qgemm_dequant(ac, as_, wc, ws, 8, y=big[:, 32:160])
    assert torch.equal(y, vq.vq_qgemm_dequant(ac, as_, wc, ws, 8))


def test_rejects_inputs_the_kernels_would_misread(vq):
    """Index, scale and code inputs are checked for device, dtype, contiguity and length
    before any launch: a host or int64 index tensor, short scales or codes of the wrong
    width must raise instead of reaching a kernel."""
    x = torch.randn(64, 256, device=DEV).to(torch.bfloat16)
    w = torch.randn(128, 256, device=DEV).to(torch.bfloat16)
    idx = torch.tensor([3, 17], dtype=torch.int32)
    with pytest.raises(TypeError):
        vq.vq_pack_weights(w, 4, idx)  # host index tensor (as vq_detect_outliers returns it)
    with pytest.raises(TypeError):
        vq.vq_pack_weights(w, 4, idx.to(DEV).long())  # int64 index
    with pytest.raises(TypeError):
        vq.vq_quant_act(x, 8, idx=idx)
    with pytest.raises(ValueError):
        vq.vq_quant_act(x, 8, "static", static_scale=torch.ones(1, device=DEV), idx=idx.to(DEV))  # needs 2 scales
    with pytest.raises(TypeError):
        vq.vq_quant_act(x, 8, bits_dev=torch.tensor([8], device=DEV, dtype=torch.int64))
    wc8, ws8 = vq.vq_pack_weights(w, 8)
    wc4, ws4 = vq.vq_pack_weights(w, 4)
    ac, as_ = vq.vq_quant_act(x, 8)
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc8, ws8[:100], 8)  # short column scales
    with pytest.raises(TypeError):
        vq.vq_qgemm_dequant(ac, as_, wc4, ws4, 8)  # packed nibbles passed as 8-bit codes
    with pytest.raises(TypeError):
        vq.vq_qgemm_dequant(ac, as_.cpu(), wc8, ws8, 8)
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac, as_, wc8, ws8, 8, k0=192)  # two partitions need two scales per row/column
    with pytest.raises(ValueError):
        vq.vq_qgemm_dequant(ac[:, :128].contiguous(), as_, wc8, ws8, 8)  # K of a and b disagree
    torch.cuda.synchronize()


def test_prepared_calls_match_direct_calls(vq):
    """prepare() records a call's launches once; replaying them on new data written into
    the same input tensors gives what a direct call gives."""
    g = torch.Generator(device=DEV).manual_seed(3)
    x = torch.randn(256, 512, generator=g, device=DEV).to(torch.float16)
    w = (torch.randn(512, 512, generator=g, device=DEV) * 0.02).to(torch.float16)
    wc, ws = vq.vq_pack_weights(w, 8)
    quant, (codes, scales) = vq.prepare(vq.vq_quant_act, x, 8, "tensor")
    gemm, y = vq.prepare(vq.vq_qgemm_dequant, codes, scales, wc, ws, 8, None, torch.float16, False, ws=False)
    for rep in range(3):
        x.copy_(torch.randn(256, 512, generator=g, device=DEV).to(torch.float16))
        quant()
        gemm()
        c2, s2 = vq.vq_quant_act(x, 8, "tensor")
        y2 = vq.vq_qgemm_dequant(c2, s2, wc, ws, 8, None, torch.float16, False, ws=False)
        torch.cuda.synchronize()
        assert torch.equal(codes, c2) and torch.equal(scales, s2) and torch.equal(y, y2), f"replay {rep}"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # launches follow the current stream
        y.zero_()
        quant()
        gemm()
    side.synchronize()
    assert torch.equal(y, y2)
    with pytest.raises(ValueError):
        vq.prepare(vq.vq_outlier_part_len, 3)

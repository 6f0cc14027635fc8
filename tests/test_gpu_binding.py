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

"""Later tiles of the persistent W8A8 GEMM: the whole output is bit-identical to the same
GEMM run with the int32-accumulator test hook, whose epilogue stores every output at the
tile change (the hook's accumulators are checked against the oracle in the parity tests).

With more tiles than workgroups, each workgroup's tile change stores part of a whole
16-bit tile during its next tile's first K stages; these shapes give each workgroup two
or more tiles, with whole and ragged tiles, both weight layouts, fp16 and bf16 outputs,
and K just above and below the length the deferral needs.
"""
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


@pytest.mark.parametrize("m,n,k,kblock,out", [
    (8192, 4096, 512, True, torch.bfloat16),      # 512 whole tiles: two per workgroup
    (8192 + 100, 4096 + 64, 576, False, torch.float16),  # ragged last row and column of tiles
    (17776, 5760, 1920, True, torch.bfloat16),    # the fused-QKV shape: six or seven per workgroup
    (8192, 4096, 448, True, torch.bfloat16),      # seven 64-code stages: too short to defer
])
def test_later_tiles_match_the_hook_path(vq, m, n, k, kblock, out):
    print(f"\ncase m={m} n={n} k={k} kblock={kblock} out={out}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(m + n + k)
    x = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    wc, ws = vq.vq_pack_weights(w, 8, kblock=kblock)
    ac, sa = vq.vq_quant_act(x, 8, "token")
    y = vq.vq_qgemm_dequant(ac, sa, wc, ws, 8, None, out)
    y_hook, _ = vq.vq_qgemm_dequant(ac, sa, wc, ws, 8, None, out, True, acc_debug=True)
    y_again = vq.vq_qgemm_dequant(ac, sa, wc, ws, 8, None, out)
    torch.cuda.synchronize()
    a, b, c = (t.view(torch.int16) for t in (y, y_hook, y_again))
    assert torch.equal(a, b), f"{int((a != b).sum())} outputs differ from the hook path"
    assert torch.equal(a, c), "two calls differ"

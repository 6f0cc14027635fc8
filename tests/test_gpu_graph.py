"""Steps captured in a HIP graph replay to the eager results.

A step (activation quantization and the GEMM with its epilogue) is captured once and
replayed several times, with eager work on the same buffers between the replays; every
replay must reproduce the eager output bit for bit.  Cases: per-token and dynamic
per-tensor quantization (the latter clears its maxima with a fill kernel, no memset), and
a GEMM whose leftover tiles are split along K through a workspace that every call must
leave zeroed for the next replay.
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


@pytest.mark.parametrize("m,n,k,gran", [
    (1000, 640, 1920, "token"),
    (1000, 640, 1920, "tensor"),
    (300, 320, 6144, "token"),   # 4 tiles, split into two K ranges through the workspace
])
def test_graph_replays_match_eager(vq, m, n, k, gran):
    g = torch.Generator(device=DEV).manual_seed(m + n + k)
    x = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    x2 = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    wc, wsc = vq.vq_pack_weights(w, 8)
    codes = torch.empty((m, k), dtype=torch.int8, device=DEV)
    scales = torch.empty(m if gran == "token" else 1, dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    need = vq._lib.vq_qgemm_workspace_bytes(m, n, k)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV) if need else False
    if k == 6144:
        assert need > 0

    def step(src):
        vq.vq_quant_act(src, 8, gran, codes=codes, scales=scales)
        vq.vq_qgemm_dequant(codes, scales, wc, wsc, 8, k, torch.bfloat16, gran == "token", y=y, ws=ws)

    step(x)
    torch.cuda.synchronize()
    y_ref = y.clone()
    step(x2)
    torch.cuda.synchronize()
    y_ref2 = y.clone()
    assert not torch.equal(y_ref, y_ref2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(x)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"
        step(x2)  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref2), f"eager after replay {rep}"
    if need:
        assert not ws[:4096].any()

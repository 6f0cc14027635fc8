"""Steps captured in a HIP graph replay to the eager results.

A step (activation quantization and the GEMM with its epilogue) is captured once and
replayed several times, with eager work on the same buffers between the replays; every
replay must reproduce the eager output bit for bit.  Cases: per-token and dynamic
per-tensor quantization (the latter clears its maxima with a fill kernel, no memset), a
GEMM whose leftover tiles are split along K through a workspace that every call must
leave zeroed for the next replay, the tiny per-tensor layer (one-launch quantizer,
few-tile GEMM) with the unquantized bf16 layer, and split GEMMs on two streams at once.
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
    (300, 4400, 6144, "token"),  # 36 tiles, split into two K ranges through the workspace
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


def test_default_workspace_under_capture(vq, monkeypatch):
    """ws=None under graph capture: with no workspace cached for the capturing stream the
    binding refuses before any launch (a buffer created there would be cached with its zero
    fill only recorded); after one eager call on that stream the cached, zeroed buffer
    serves the capture and every replay."""
    m, n, k = 300, 4400, 6144  # 36 tiles, two K ranges each: the workspace is used
    assert vq._lib.vq_qgemm_workspace_bytes(m, n, k) > 0
    g = torch.Generator(device=DEV).manual_seed(7)
    x = torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    wc, wsc = vq.vq_pack_weights(w, 8)
    ac, as_ = vq.vq_quant_act(x, 8)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    y_ref = vq.vq_qgemm_dequant(ac, as_, wc, wsc, 8, ws=False)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for key in [key for key in vq._GEMM_WS if key[1] == side.cuda_stream]:
        del vq._GEMM_WS[key]  # pooled stream handles repeat: start without a cached buffer
    with torch.cuda.stream(side):
        with monkeypatch.context() as mp:  # as seen from inside a capture
            mp.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
            with pytest.raises(RuntimeError, match="workspace"):
                vq.vq_qgemm_dequant(ac, as_, wc, wsc, 8, y=y)
        vq.vq_qgemm_dequant(ac, as_, wc, wsc, 8, y=y)  # eager: creates and zero-fills the buffer
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            vq.vq_qgemm_dequant(ac, as_, wc, wsc, 8, y=y)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"


def test_small_layer_and_dense_layer_in_one_graph(vq):
    """The 256 x 512 x 512 per-tensor layer (one-launch quantizer, few-tile GEMM) and the
    unquantized bf16 layer, captured together and replayed with eager work on the same
    buffers between replays: every replay equals the eager results."""
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn(256, 512, generator=g, device=DEV).to(torch.float16)
    x2 = torch.randn(256, 512, generator=g, device=DEV).to(torch.float16)
    w = (torch.randn(512, 512, generator=g, device=DEV) * 0.02).to(torch.float16)
    wc, wsc = vq.vq_pack_weights(w, 8)
    codes = torch.empty((256, 512), dtype=torch.int8, device=DEV)
    scales = torch.empty(1, dtype=torch.float32, device=DEV)
    y = torch.empty((256, 512), dtype=torch.float16, device=DEV)
    yd = torch.empty((256, 512), dtype=torch.float16, device=DEV)

    def step(src):
        vq.vq_quant_act(src, 8, "tensor", codes=codes, scales=scales)
        vq.vq_qgemm_dequant(codes, scales, wc, wsc, 8, 512, torch.float16, False, y=y, ws=False)
        vq.vq_gemm_dense(src, w, y=yd)

    step(x)
    torch.cuda.synchronize()
    ref = (y.clone(), yd.clone(), scales.clone())
    step(x2)
    torch.cuda.synchronize()
    ref2 = (y.clone(), yd.clone(), scales.clone())
    assert not torch.equal(ref[0], ref2[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(x)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        y.zero_()
        yd.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(yd, ref[1]) and torch.equal(scales, ref[2]), f"replay {rep}"
        step(x2)
        torch.cuda.synchronize()
        assert torch.equal(y, ref2[0]) and torch.equal(yd, ref2[1]), f"eager after replay {rep}"


def test_two_streams_keep_separate_workspaces(vq):
    """Split GEMMs on two streams at once, each with the binding's default workspace (one
    per device and stream): both results equal the unsplit GEMM."""
    m, n, k = 300, 4400, 6144  # 36 tiles, two K ranges each
    g = torch.Generator(device=DEV).manual_seed(8)
    xs = [torch.randn(m, k, generator=g, device=DEV).to(torch.bfloat16) for _ in range(2)]
    w = (torch.randn(n, k, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    wc, wsc = vq.vq_pack_weights(w, 8)
    ops = [vq.vq_quant_act(x, 8) for x in xs]
    want = [vq.vq_qgemm_dequant(a, s, wc, wsc, 8, ws=False) for a, s in ops]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = [None, None]
    for rep in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                outs[i] = vq.vq_qgemm_dequant(ops[i][0], ops[i][1], wc, wsc, 8)
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i], want[i]), f"stream {i}, call {rep}"
    keys = [key for key in vq._GEMM_WS if key[1] in (streams[0].cuda_stream, streams[1].cuda_stream)]
    assert len(keys) == 2

"""HIP-graph capture of the hot path: replays must reproduce the eager result exactly, every time,
with other eager work and synchronizations between replays (the library issues no memset nodes)."""
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import workloads

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    dev = "cuda"
    x_cpu, w_cpu = workloads.tiny()
    x = x_cpu.to(dev)
    wp, ws, wS = nv.nvfp4_quantize(w_cpu.to(dev))
    bp = nv.nvfp4_prepack_weight(wp, ws)
    M, K = x.shape
    N = w_cpu.shape[0]
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    S = torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    yd = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

    def run():
        nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=qws)
        nv.nvfp4_gemm(nv.W4A4, packed, scales, S, bp, wS, N, K, torch.float32, out=y)
        nv.nvfp4_dequantize(packed, scales, S, torch.bfloat16, out=yd)

    run()
    torch.cuda.synchronize()
    ref = (packed.clone(), scales.clone(), S.clone(), y.clone(), yd.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (packed, scales, S, y, yd):
            t.zero_()
        _ = (x * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp in zip((packed, scales, S, y, yd), ref):
            assert torch.equal(got, exp), f"replay {rep} differs"

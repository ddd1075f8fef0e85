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


def test_graph_replay_all_paths():
    """One captured graph holding every other kernel family: W4A4 with a K split (partials plus the
    reduction), the streaming W4A16 kernel, the tiled W4A16 kernel, fake quantization, the
    NVFP4-output GEMM, and MXFP4 quantize + GEMM; each replay equals the eager run bit for bit."""
    dev = "cuda"
    g = torch.Generator().manual_seed(7)
    M, N, K = 512, 512, 4096           # 128x128 tiles with a K split
    x = torch.randn(M, K, generator=g).to(torch.bfloat16).to(dev)
    w = (0.02 * torch.randn(N, K, generator=g)).to(torch.bfloat16).to(dev)
    x16 = torch.randn(16, K, generator=g).to(torch.bfloat16).to(dev)
    x300 = torch.randn(300, K, generator=g).to(torch.bfloat16).to(dev)
    wp, ws, wS = nv.nvfp4_quantize(w)
    bp = nv.nvfp4_prepack_weight(wp, ws)
    mb, mbs = nv.nvfp4_mx_quantize(w)
    packed = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    S = torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    gws = torch.empty(max(nv.nvfp4_gemm_workspace_bytes(nv.W4A4, M, N, K),
                          nv.nvfp4_gemm_workspace_bytes(nv.W4A16, 16, N, K),
                          nv.nvfp4_gemm_workspace_bytes(nv.W4A16, 300, N, K), 1), dtype=torch.uint8, device=dev)
    So = torch.tensor([1.0 / 2688.0], dtype=torch.float32, device=dev)
    rws = torch.empty(max(nv.nvfp4_gemm_requant_workspace_bytes(nv.W4A4, M, N, K), 1), dtype=torch.uint8,
                      device=dev)
    outs = {
        "y44": torch.empty((M, N), dtype=torch.bfloat16, device=dev),
        "y16": torch.empty((16, N), dtype=torch.float32, device=dev),
        "y300": torch.empty((300, N), dtype=torch.bfloat16, device=dev),
        "fake": torch.empty((M, K), dtype=torch.bfloat16, device=dev),
        "rp": torch.empty((M, N // 2), dtype=torch.uint8, device=dev),
        "rs": torch.empty((M, N // 16), dtype=torch.uint8, device=dev),
        "ma": torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
        "mas": torch.empty((M, K // 32), dtype=torch.uint8, device=dev),
        "my": torch.empty((M, N), dtype=torch.float32, device=dev),
    }

    def run():
        nv.nvfp4_quantize(x, S, static=False, packed=packed, scales=scales, workspace=qws)
        nv.nvfp4_gemm(nv.W4A4, packed, scales, S, bp, wS, N, K, torch.bfloat16, out=outs["y44"], workspace=gws)
        nv.nvfp4_gemm(nv.W4A16, x16, None, None, bp, wS, N, K, torch.float32, out=outs["y16"], workspace=gws)
        nv.nvfp4_gemm(nv.W4A16, x300, None, None, bp, wS, N, K, torch.bfloat16, out=outs["y300"], workspace=gws)
        nv.nvfp4_fake_quantize(x, S, static=True, out=outs["fake"])
        nv.nvfp4_gemm_requant(nv.W4A4, packed, scales, S, bp, wS, N, K, So, packed=outs["rp"], scales=outs["rs"],
                              workspace=rws)
        nv.nvfp4_mx_quantize(x, packed=outs["ma"], scales=outs["mas"])
        nv.nvfp4_mx_gemm(outs["ma"], outs["mas"], mb, mbs, out=outs["my"])

    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs.values():
            t.zero_()
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs"

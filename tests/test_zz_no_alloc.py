"""The quantize entry point that allocates nothing (nvfp4_quantize_noalloc), called through the C ABI.

Its dynamic pass keeps the partial maxima in the library's own device scratch instead of a
workspace.  It must give exactly the bytes and tensor scale of nvfp4_quantize_bs (quantization is
an encoding: bit-exact is the bar) on consecutive calls; the second call is smaller than the first
and its input's maximum is far below the first's, so a partial left in the shared scratch by the
first call and read by the second would change the second's tensor scale.
"""
import numpy as np
import pytest
import torch

import nvfp4_quantized_gemm_amd as nv
import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(x, static_S=None, block_size=16):
    """(packed, scales, S) from nvfp4_quantize_bs and from nvfp4_quantize_noalloc on the same input."""
    M, K = x.shape
    ref = nv.nvfp4_quantize(x, None if static_S is None else torch.tensor([static_S], device=DEV),
                            block_size=block_size)
    packed = torch.full((M, K // 2), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((M, K // block_size), 0xA5, dtype=torch.uint8, device=DEV)
    S = torch.full((1,), -1.0, dtype=torch.float32, device=DEV) if static_S is None else \
        torch.tensor([static_S], dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    nv.nvfp4_quantize_noalloc(x, S, packed, scales, static=static_S is not None, block_size=block_size)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return ref, (packed, scales, S)


def _assert_same(ref, got, label):
    print(f"[no-alloc] {label}", flush=True)
    assert torch.equal(got[0], ref[0]), f"{label}: codes differ"
    assert torch.equal(got[1], ref[1]), f"{label}: scale bytes differ"
    assert got[2].view(torch.int32).item() == ref[2].view(torch.int32).item(), f"{label}: tensor scale differs"


def test_noalloc_quantize_matches_workspace_entry_point():
    # first call: the PixArt fc2 activation (4096 x 4608 bf16, outlier channels), which fills all of
    # the scratch's partial maxima
    _, x1, _ = workloads.pixart()[3]
    x1d = x1.to(DEV)
    ref1, got1 = _both(x1d)
    _assert_same(ref1, got1, "4096x4608 bf16 dynamic")
    S1 = got1[2].item()

    # second call, smaller, with a maximum far below the first's
    g = torch.Generator().manual_seed(7)
    x2 = torch.randn(300, 1152, generator=g, dtype=torch.float32)
    ref2, got2 = _both(x2.to(DEV))
    _assert_same(ref2, got2, "300x1152 fp32 dynamic")
    assert got2[2].item() < S1 / 4
    # and against the oracle
    op, os_, oS = oracle.quantize(x2.numpy())
    assert np.array_equal(got2[0].cpu().numpy(), op) and np.array_equal(got2[1].cpu().numpy(), os_)
    assert np.float32(got2[2].item()).view(np.uint32) == np.float32(oS).view(np.uint32)

    # static mode (no scratch) and the other block sizes
    ref3, got3 = _both(x1d, static_S=float(np.float32(S1)))
    _assert_same(ref3, got3, "4096x4608 bf16 static")
    for b in (32, 64):
        ref4, got4 = _both(x2.to(DEV)[:64], block_size=b)
        _assert_same(ref4, got4, f"64x1152 fp32 dynamic, block {b}")


def test_noalloc_quantize_empty_and_validation():
    """M == 0 writes S = 0 like the workspace entry point; bad arguments are refused on the host."""
    L = nv.lib()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    S = torch.full((1,), 5.0, dtype=torch.float32, device=DEV)
    p = torch.empty((0, 32), dtype=torch.uint8, device=DEV)
    s = torch.empty((0, 4), dtype=torch.uint8, device=DEV)
    nv.nvfp4_quantize_noalloc(x, S, p, s)
    torch.cuda.synchronize()
    assert S.item() == 0.0
    import ctypes
    P = ctypes.c_void_p(0x10000)
    assert L.nvfp4_quantize_noalloc(P, nv.BF16, 4, 24, 24, 16, P, P, P, nv.SCALE_DYNAMIC, None) == nv.Status.ERR_SHAPE
    assert L.nvfp4_quantize_noalloc(P, nv.BF16, 4, 32, 32, 16, P, P, None, nv.SCALE_DYNAMIC, None) == \
        nv.Status.ERR_NULL

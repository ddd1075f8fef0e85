"""GPU property tests: Hypothesis draws blocks and tensor scales (the adversarial kinds of the oracle
property tests: exact ties, E4M3 midpoints, subnormal scales, saturation, signed zeros) and the
GPU quantizer must produce the oracle's bytes exactly, for fp32 and bf16 inputs, static and
dynamic tensor scales and block sizes 16, 32 and 64; dequantization must give the oracle's bits
[NVFP4-DiT page, Methodology section 1, Definition III.1 and Algorithm 1 / Eq. 9 block sizes].
Draws are derandomized, so every run sees the same cases."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import nvfp4_quantized_gemm_amd as nv
import oracle
from test_gpu_parity import DEV, np_x
from test_oracle_properties import static_case

pytestmark = pytest.mark.gpu

GPU_SETTINGS = settings(max_examples=120, deadline=None, derandomize=True,
                        suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


def _check(x_cpu: torch.Tensor, S, b: int):
    xd = x_cpu.to(DEV)
    Sd = None if S is None else torch.tensor([S], dtype=torch.float32, device=DEV)
    p, s, Sg = nv.nvfp4_quantize(xd, Sd, block_size=b)
    torch.cuda.synchronize()
    op, os_, oS = oracle.quantize(np_x(x_cpu), S=S, block=b)
    assert np.float32(Sg.item()).view(np.uint32) == np.float32(oS).view(np.uint32)
    assert np.array_equal(s.cpu().numpy(), os_), "scale bytes"
    assert np.array_equal(p.cpu().numpy(), op), "codes"
    y = nv.nvfp4_dequantize(p, s, Sg, torch.float32)
    torch.cuda.synchronize()
    y32, _ = oracle.dequantize(op, os_, oS)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), y32.view(np.uint32)), "dequantized bits"


@GPU_SETTINGS
@given(static_case(), st.sampled_from([16, 32, 64]), st.booleans(), st.booleans())
def test_quantize_property(case, b, dynamic, bf16):
    x, S = case
    if not np.isfinite(x).all():
        return
    reps = b // 16
    # repeat the drawn blocks so that K is a multiple of the block size
    xr = np.tile(x, (1, reps)) if x.shape[1] % b else x
    t = torch.from_numpy(np.ascontiguousarray(xr))
    if bf16:
        t = t.to(torch.bfloat16)
    if dynamic:
        amax = float(t.float().abs().max())
        if amax < 2.0 ** -100:  # the tensor scale would be subnormal: outside the contract
            return
        _check(t, None, b)
    else:
        _check(t, S, b)

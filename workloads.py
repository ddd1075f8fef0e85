"""Seeded synthetic inputs for the NVFP4 quantize / GEMM workloads.

This module only draws random tensors with the shapes, value distributions and planted structure
of the diffusion-transformer workloads; it performs none of the quantization arithmetic and is
shared by the parity tests, the benchmark and the smoke check.  All draws use a CPU
``torch.Generator`` so the same bytes reach the GPU path and the CPU oracle.

Workloads (DiT linear layers, X [M, K] activations and W [N, K] weights, Y = X W^T):
  * ``tiny``      seed 0: X fp32 [256, 1152] ~ N(0, 1), W fp32 [1152, 1152] ~ N(0, 0.02).
  * ``pixart``    seed 1: PixArt-style block linears at M = 4096 tokens (128x128 latent, patch 2),
                  hidden 1152: qkv 1152->3456, proj 1152->1152, fc1 1152->4608, fc2 4608->1152.
                  X ~ N(0, 1) with 1 % of channels (round(0.01 K), chosen by randperm) scaled x20,
                  W ~ N(0, 0.02); both cast to bf16.  Each linear draws its own X.
  * ``w4a16``     seed 2: bf16 activations M in {1, 16, 256, 4096} x K; weights N(0, 0.02) with
                  Laplace-like tails: w = 0.02 z for |z| <= 2, else 0.02 sign(z) (2 + Exp(1)).
                  up: N 12288, K 3072; down: N 3072, K 12288.
  * ``video``     seed 3: M = 16 frames x (64x40 latent, patch 2) = 10240 tokens, hidden 3072:
                  qkv 3072->9216, fc1 3072->12288, fc2 12288->3072.  X = 0.5 t c with t ~ Student-t(4)
                  per element (z / sqrt(chi2_4 / 4)) and a per-channel c ~ LogNormal(0, 1); W ~ N(0, 0.02).
  * ``sweep``     seed 4: bf16 [M, K], M in {4096, 32768}, K in {1152, 3072, 12288}: N(0, 1) with planted
                  blocks (16 consecutive values along K): x[0, 0] = 10.5 so that the dynamic tensor scale is
                  exactly 2^-8; every 97th block all zero (alternately +0.0 and -0.0); every 89th block tiny
                  (N(0,1) * 2^-(12+j), j cycling 0..7) to reach subnormal E4M3 scales and flushed blocks;
                  every 83rd block built from exact ties (see ``_tie_blocks``).  The static variant scales every
                  101st block by 2^10 so that |x| far exceeds 6 * 448 * 2^-8.
"""
from __future__ import annotations


import torch

PIXART_LINEARS = (("qkv", 3456, 1152), ("proj", 1152, 1152), ("fc1", 4608, 1152), ("fc2", 1152, 4608))
VIDEO_LINEARS = (("qkv", 9216, 3072), ("fc1", 12288, 3072), ("fc2", 3072, 12288))
W4A16_LINEARS = (("up", 12288, 3072), ("down", 3072, 12288))
W4A16_MS = (1, 16, 256, 4096)
SWEEP_SHAPES = tuple((m, k) for m in (4096, 32768) for k in (1152, 3072, 12288))
PIXART_M = 4096
VIDEO_M = 10240


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


# ---- tiny: fp32 W4A4 linear -------------------------------------------------------------------

def tiny(M: int = 256, K: int = 1152, N: int = 1152, seed: int = 0):
    g = _gen(seed)
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    w = 0.02 * torch.randn(N, K, generator=g, dtype=torch.float32)
    return x, w


# ---- PixArt-style block linears ----------------------------------------------------------------

def pixart_activation(M: int, K: int, g: torch.Generator) -> torch.Tensor:
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    n_out = int(round(0.01 * K))
    idx = torch.randperm(K, generator=g)[:n_out]
    x[:, idx] *= 20.0
    return x.to(torch.bfloat16)


def pixart(M: int = PIXART_M, seed: int = 1, linears=PIXART_LINEARS):
    """List of (name, X bf16 [M, K], W bf16 [N, K]) in block order."""
    g = _gen(seed)
    out = []
    for name, N, K in linears:
        x = pixart_activation(M, K, g)
        w = (0.02 * torch.randn(N, K, generator=g, dtype=torch.float32)).to(torch.bfloat16)
        out.append((name, x, w))
    return out


# ---- weight-only variant --------------------------------------------------------------------------

def laplace_tailed_weight(N: int, K: int, g: torch.Generator) -> torch.Tensor:
    z = torch.randn(N, K, generator=g, dtype=torch.float32)
    u = torch.rand(N, K, generator=g, dtype=torch.float32)
    tail = torch.sign(z) * (2.0 - torch.log1p(-u))  # 2 + Exp(1) beyond two sigma
    return 0.02 * torch.where(z.abs() <= 2.0, z, tail)


def w4a16(seed: int = 2, linears=W4A16_LINEARS, ms=W4A16_MS):
    """Dict name -> (W fp32 [N, K], {M: A bf16 [M, K]})."""
    g = _gen(seed)
    out = {}
    for name, N, K in linears:
        w = laplace_tailed_weight(N, K, g)
        acts = {m: torch.randn(m, K, generator=g, dtype=torch.float32).to(torch.bfloat16) for m in ms}
        out[name] = (w, acts)
    return out


# ---- video DiT shape ------------------------------------------------------------------------------

def video_activation(M: int, K: int, g: torch.Generator) -> torch.Tensor:
    c = torch.exp(torch.randn(K, generator=g, dtype=torch.float32))
    z = torch.randn(M, K, generator=g, dtype=torch.float32)
    chi2 = torch.zeros(M, K, dtype=torch.float32)
    for _ in range(4):
        chi2 += torch.randn(M, K, generator=g, dtype=torch.float32) ** 2
    t = z / torch.sqrt(chi2 / 4.0)
    return (0.5 * t * c).to(torch.bfloat16)


def video(M: int = VIDEO_M, seed: int = 3, linears=VIDEO_LINEARS):
    g = _gen(seed)
    out = []
    for name, N, K in linears:
        x = video_activation(M, K, g)
        w = (0.02 * torch.randn(N, K, generator=g, dtype=torch.float32)).to(torch.bfloat16)
        out.append((name, x, w))
    return out


# ---- quantize / dequantize sweep ---------------------------------------------------------------------

def e4m3_positive_values():
    """The 126 positive finite OCP E4M3FN values, ascending (input construction only)."""
    vals = [k * 2.0 ** -9 for k in range(1, 8)]
    for E in range(1, 16):
        for m in range(8):
            if E == 15 and m == 7:
                continue
            vals.append((1.0 + m / 8.0) * 2.0 ** (E - 7))
    return vals


_TIES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)  # midpoints of the E2M1 grid


def _tie_blocks(c: torch.Tensor, S: float, g: torch.Generator) -> torch.Tensor:
    """Blocks of the exact-tie family, one row per index in c: every value sits on a decision boundary.

    Even c: anchor 6 e S (the block maximum maps exactly to scale e), the other 15 values t e S for
    the E2M1 midpoints t.  Odd c: the anchor is the midpoint between e and the next E4M3 value
    times 6 S (an exact E4M3 rounding tie).  e cycles over the 126 positive E4M3 values; signs are
    random; every value is exact in bfloat16.
    """
    vals = torch.tensor(e4m3_positive_values(), dtype=torch.float64)
    n = len(vals)
    i = c % n
    e = vals[i]
    nxt = vals[torch.clamp(i + 1, max=n - 1)]
    mid = (c % 2 == 1) & (i + 1 < n)
    anchor = torch.where(mid, 0.5 * (e + nxt), e) * 6.0 * S
    ties = torch.tensor(_TIES, dtype=torch.float64)
    j = torch.arange(15)
    t = ties[(c[:, None] + j[None, :]) % len(_TIES)]
    out = torch.cat([anchor[:, None], t * e[:, None] * S], dim=1)
    signs = torch.where(torch.rand(c.numel(), 16, generator=g) < 0.5, -1.0, 1.0).double()
    signs[:, 0] = torch.where(c % 3 == 0, -1.0, 1.0).double()
    return out * signs


def sweep(M: int, K: int, seed: int = 4, static: bool = False):
    """bf16 [M, K] with the planted block families.  static=True adds the x2^10 blocks."""
    assert K % 16 == 0
    g = _gen(seed)
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    nb = M * K // 16
    blocks = x.view(nb, 16)
    S = 2.0 ** -8  # forced by the planted maximum 10.5 = 6 * 448 * 2^-8
    b = torch.arange(nb)
    zero = (b % 97 == 0) & (b > 0)
    tie = (b % 83 == 0) & (b > 0) & ~zero
    tiny_ = (b % 89 == 0) & (b > 0) & ~zero & ~tie
    zi = torch.nonzero(zero).flatten()
    blocks[zi] = 0.0
    neg = zi[(zi // 97) % 2 == 1]
    blocks[neg] = -0.0
    ti = torch.nonzero(tiny_).flatten()
    j = (ti // 89) % 8
    scale = torch.pow(2.0, -(12 + j).float())
    blocks[ti] = torch.randn(ti.numel(), 16, generator=g) * scale[:, None]
    tb = torch.nonzero(tie).flatten()
    blocks[tb] = _tie_blocks(tb // 83, S, g).float()
    x[0, 0] = 10.5
    x = x.to(torch.bfloat16)
    if static:
        xb = x.view(nb, 16)
        big = (b % 101 == 0) & (b > 0)
        xb[big] = xb[big] * 1024.0
    return x


SWEEP_STATIC_S = 2.0 ** -8


def workload_names():
    return ("tiny", "pixart", "w4a16", "video", "sweep")


def flops_linear(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def describe():
    lines = []
    for name, N, K in PIXART_LINEARS:
        lines.append(f"pixart {name}: M={PIXART_M} N={N} K={K} GF={flops_linear(PIXART_M, N, K) / 1e9:.1f}")
    for name, N, K in VIDEO_LINEARS:
        lines.append(f"video {name}: M={VIDEO_M} N={N} K={K} GF={flops_linear(VIDEO_M, N, K) / 1e9:.1f}")
    return "\n".join(lines)


if __name__ == "__main__":
    print(describe())

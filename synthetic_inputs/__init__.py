"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle's tests.

This module only draws numbers and stores them in the formats the kernels take
(fp32, bf16 bit patterns, OCP e4m3fn codes with a per-tensor dequant scale).
It holds none of the method's arithmetic: no GEMM, no activation, no reduction.
Conversions to bf16 / e4m3fn use PyTorch's CPU casts (library routines).

Workload recipes follow the pages' shapes:
  * "Tensor parallelism" (algorithm page), section "Code": the deterministic
    generator rnd(n, s) = ((i*2654435761 + s) mod 1000)/1000 - 0.5 and the
    Megatron MLP at (m, d, f, t) = (8, 32, 128, 4).
  * Everything else: PCG64 normals N(0, sigma) / uniforms, fixed seeds.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0  # largest finite OCP e4m3fn magnitude


def page3_rnd(n: int, s: int) -> np.ndarray:
    """The page's own input generator (algorithm page "Tensor parallelism",
    section "Code"): element i is ((i*2654435761 + s) mod 1000)/1000 - 0.5,
    computed in integers then divided in fp32, as the listing types it."""
    i = np.arange(n, dtype=np.uint64)
    r = (i * np.uint64(2654435761) + np.uint64(s)) % np.uint64(1000)
    return (r.astype(np.float32) / np.float32(1000.0)) - np.float32(0.5)


def normal_f32(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    """PCG64 standard normals (fp32) scaled by sigma."""
    g = np.random.default_rng(seed)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def uniform_f32(shape, seed: int, lo: float = -0.5, hi: float = 0.5) -> np.ndarray:
    g = np.random.default_rng(seed)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def small_ints(shape, seed: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """Integers in [lo, hi] as fp32: exact in bf16 and in e4m3fn (scale 1)."""
    g = np.random.default_rng(seed)
    return g.integers(lo, hi + 1, size=shape).astype(np.float32)


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 numpy -> torch.bfloat16 CPU tensor (PyTorch's round-to-nearest-even cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bfloat16 tensor."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def to_e4m3_current(x: np.ndarray):
    """Per-tensor current scaling of an input tensor to OCP e4m3fn.

    Returns (codes uint8 torch tensor, dequant scale as np.float32), with
    x ~= decode(code) * scale.  scale = amax/448 (1 when amax == 0); the
    values are multiplied by fp32(448/amax) and cast with PyTorch's
    float8_e4m3fn conversion (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    if amax == 0:
        inv = np.float32(1.0)
        scale = np.float32(1.0)
    else:
        inv = np.float32(np.float32(E4M3_MAX) / amax)
        scale = np.float32(amax / np.float32(E4M3_MAX))
    y = torch.from_numpy(x * inv).clamp_(-E4M3_MAX, E4M3_MAX)
    q = y.to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def to_mxfp8(x: np.ndarray):
    """MXFP8 inputs (OCP Microscaling: 32-element blocks along the last axis,
    one power-of-two scale per block, e4m3fn elements) for a [rows, K] fp32
    array, K % 32 == 0.  Returns (codes uint8 torch [rows, K], scale
    exponents uint8 torch [rows, K/32], row-major).  The block exponent is
    floor(log2 amax) from torch.frexp, minus 8, biased by 127 and clamped to
    [0, 254] (0 for an all-zero block); elements are cast with PyTorch's
    float8_e4m3fn conversion after clamping to +-448."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    rows, k = t.shape
    b = t.reshape(rows, k // 32, 32)
    amax = b.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                        # amax = m * 2^ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex - 1 - 8 + 127, torch.zeros_like(ex)).clamp(0, 254)
    scaled = torch.ldexp(b, (127 - e).unsqueeze(2).to(torch.float32))
    codes = scaled.clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).reshape(rows, k)
    return codes.contiguous(), e.to(torch.uint8).contiguous()


def to_e4m3_exact(x: np.ndarray) -> torch.Tensor:
    """Cast values that are exactly representable in e4m3fn (e.g. small ints)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8)


def ring_chunk_order(T: int, C: int, rank: int) -> list[int]:
    """Arrival order of sequence chunks at `rank` under a ring all-gather:
    the rank's own chunks first, then those of ranks rank-1, rank-2, ... (mod T),
    ascending within a rank.  Chunks are numbered by token position; rank q
    owns chunks q*C/T .. (q+1)*C/T - 1."""
    assert C % T == 0
    per = C // T
    order = []
    for step in range(T):
        q = (rank - step) % T
        order.extend(range(q * per, (q + 1) * per))
    return order


def dest_range_order(T: int, rank: int) -> list[int]:
    """Order in which a row-parallel GEMM produces destination token ranges
    so that finished ranges can leave early: rank+1, rank+2, ..., own last."""
    return [(rank + 1 + i) % T for i in range(T)]


# ---------------------------------------------------------------------------
# Workload recipes (shapes, seeds, distributions)
# ---------------------------------------------------------------------------

def c1_tiny_mlp(generator: str = "page3"):
    """Tiny TP MLP, fp32: X[8,32], A[32,128] (4 column shards of [32,32]),
    B[128,32] (4 row shards of [32,32]).  generator='page3' uses the page's
    rnd() with seeds 1,2,3; 'pcg' uses PCG64 uniforms in [-0.5, 0.5) seed 1."""
    m, d, f, t = 8, 32, 128, 4
    if generator == "page3":
        x = page3_rnd(m * d, 1).reshape(m, d)
        a = page3_rnd(d * f, 2).reshape(d, f)
        b = page3_rnd(f * d, 3).reshape(f, d)
    else:
        g = np.random.default_rng(1)
        x = g.uniform(-0.5, 0.5, size=(m, d)).astype(np.float32)
        a = g.uniform(-0.5, 0.5, size=(d, f)).astype(np.float32)
        b = g.uniform(-0.5, 0.5, size=(f, d)).astype(np.float32)
    return dict(m=m, d=d, f=f, t=t, x=x, a=a, b=b)

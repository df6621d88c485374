"""Helpers shared by the tests: moving data between torch tensors, the
seeded generators and the oracle's float64 arrays."""
import numpy as np
import torch

from oracle import formats


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a torch tensor (bf16 / fp32 / e4m3 codes as uint8)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return formats.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return formats.e4m3_to_f64(t.view(torch.uint8).numpy())
    raise TypeError(t.dtype)


def nerr(gpu, ref) -> float:
    g = gpu if isinstance(gpu, np.ndarray) else f64(gpu)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(g - r) / (1.0 + np.abs(r)))) if r.size else 0.0


TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}

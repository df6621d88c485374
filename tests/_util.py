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


def assert_mx_close(codes, e, h, delta, frac=1e-2):
    """An MXFP8 tensor produced on the GPU from fp32 values against the
    exact values h (float64), where delta bounds the error of the GPU's fp32
    evaluation of each value (accumulation and activation).  MX quantisation
    is monotone, so each block exponent must be that of some amax within
    delta of the exact block amax, and each code that of some value within
    delta of h at the GPU's block scale; and at most a fraction `frac` of
    the blocks / codes may differ from the quantisation of h itself."""
    e_ref = formats.mx_e4m3_quantize(h)[1]
    rows, k = h.shape
    hb = np.abs(h).reshape(rows, k // 32, 32)
    db = np.asarray(delta).reshape(rows, k // 32, 32)
    amax_lo = np.max(np.maximum(hb - db, 0), axis=2)
    amax_hi = np.max(hb + db, axis=2)

    def exp_of(a):
        out = np.zeros(a.shape, dtype=np.int64)
        nz = a > 0
        f = np.floor(np.log2(a[nz])).astype(np.int64)
        f -= (np.ldexp(1.0, f) > a[nz]).astype(np.int64)
        out[nz] = np.clip(f - 8 + 127, 0, 254)
        return out

    eg = e.astype(np.int64)
    assert np.all((eg >= exp_of(amax_lo)) & (eg <= exp_of(amax_hi)))
    assert np.mean(eg != e_ref) < frac
    X = formats.e8m0_to_f64(np.repeat(e, 32, axis=1))
    lo = formats.e4m3_to_f64(formats.e4m3_encode((h - delta) / X))
    hi = formats.e4m3_to_f64(formats.e4m3_encode((h + delta) / X))
    got = formats.e4m3_to_f64(codes)
    assert np.all((got >= lo) & (got <= hi))
    same = np.repeat(e == e_ref, 32, axis=1)
    ref_codes = formats.e4m3_encode(h / X)
    assert np.mean(same & (codes != ref_codes)) < frac


def assert_fp8_h_consistent(h_gpu, codes_gpu, s_gpu, ref, max_flip=2e-3):
    """The fp8 current-scaling step of H on the GPU against the oracle's
    chain (ops.tp_mlp_fwd_fp8 result `ref`):
    * the codes and the scale are exactly the quantisation of the bf16 H the
      GPU stored (the same fp32 arithmetic on the same values);
    * so, with the same amax, a code can differ from the oracle's only where
      the GPU's bf16 H differs from the oracle's rounding of the exact H
      (an fp32 accumulation rounding a value near a bf16 boundary the other
      way); such a one-ulp step crosses one of e4m3's rounding boundaries
      at most one time in 8, so code differences stay well below the bf16
      ones;
    * code differences stay below `max_flip`.  (bf16 differences are
      frequent among the smallest |H|, GeLU's negative tail, where the
      epilogue's fp32 evaluation is accurate to an absolute 3e-7 rather than
      to a bf16 ulp, but there one bf16 ulp is far from e4m3's steps at the
      scale of the largest |H|.)  A different amax can only come from the
      largest element rounding the other way.
    Returns the fractions of bf16 and of code differences."""
    from oracle import ops as _ops
    q = _ops.quantize_current(h_gpu, "e4m3")
    assert np.array_equal(codes_gpu, q["codes"])
    assert s_gpu == q["s"]
    hb_diff = h_gpu != ref["Hb"]
    flips = codes_gpu != ref["Hq_codes"]
    if q["amax"] == ref["amax"]:
        assert not np.any(flips & ~hb_diff)
        # a one-ulp bf16 step (2^-7 .. 2^-8 of a value across a binade)
        # crosses one of e4m3's rounding boundaries (2^-3 .. 2^-4 of a value
        # apart; coarser still among e4m3's subnormals) with probability at
        # most 2^-7 / 2^-4 = 1/8
        assert np.mean(flips) <= np.mean(hb_diff) / 8 + 1e-5, (np.mean(flips), np.mean(hb_diff))
        assert np.mean(flips) < max_flip, np.mean(flips)
    else:
        assert np.any(hb_diff & ((np.abs(h_gpu) == q["amax"]) | (np.abs(ref["Hb"]) == ref["amax"])))
    return float(np.mean(hb_diff)), float(np.mean(flips))

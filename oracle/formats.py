"""Number formats, written from their bit definitions (oracle side).

bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits -- the upper half of
an IEEE fp32.  OCP e4m3fn (the fp8 format of the FP8 recipes in "Collective
GEMMs in Tensor Sequence Parallelism", section "Supported quantization
recipes"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0 is
subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity; the largest
finite magnitude is 1.75 * 2^8 = 448.

Encoders round to the nearest representable value, ties to the even code,
and (e4m3fn) saturate finite overflow to +-448 ("satfinite").

MXFP8 (the "MXFP8 block scaling" recipe of "Collective GEMMs in Tensor
Sequence Parallelism", section "Supported quantization recipes"; the format
is the OCP Microscaling (MX) specification v1.0): blocks of 32 consecutive
elements share one scale X = 2^(E - 127) stored as an 8-bit exponent E
(E8M0, 255 = NaN); each element is an e4m3fn code P_i and the block holds
the values X * P_i.  Quantising a block V: E = floor(log2 max|V_i|) - 8 + 127
(8 being the exponent of e4m3fn's largest normal, 448 = 1.75 * 2^8), clamped
to [0, 254] (E = 0 for an all-zero block, a choice the spec leaves free), and
P_i = e4m3fn(V_i / X), nearest-even and saturating, since max|V_i| / X lies
in [256, 512).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
# non-negative finite values, ascending, indexed by code 0x00..0x7E
_E4M3_POS = E4M3_TABLE[:0x7F].copy()


def e4m3_to_f64(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3fn code to each value (float64 compare), ties to the even
    code, saturating to +-448; NaN -> 0x7F; the sign is kept for zero."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    idx = np.searchsorted(_E4M3_POS, a, side="left")  # _POS[idx-1] < a <= _POS[idx]
    idx = np.clip(idx, 1, len(_E4M3_POS) - 1)
    lo = idx - 1
    hi = idx
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a <= 0.0, 0, code)
    code = np.where(a >= E4M3_MAX, 0x7E, code)  # satfinite
    code = code.astype(np.uint8)
    neg = np.signbit(x)
    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even mantissa), returning
    uint16 bit patterns.  Written as a choice between the two neighbouring
    bf16 values (truncated, and one bf16 ulp further from zero) using exact
    float64 distances.  Past the largest finite bf16 the farther neighbour is
    2^128 (infinity), as in IEEE round-to-nearest-even.  NaN -> quiet NaN."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    mag = u & np.uint32(0x7FFFFFFF)
    lo_bits = mag & np.uint32(0xFFFF0000)               # truncation toward zero
    hi_bits = lo_bits + np.uint32(0x10000)              # one bf16 ulp larger
    lo_v = lo_bits.view(np.float32).astype(np.float64)
    hi_is_inf = hi_bits == np.uint32(0x7F800000)
    safe_hi = np.where(hi_is_inf, np.uint32(0), hi_bits).astype(np.uint32)
    hi_v = np.where(hi_is_inf, 2.0 ** 128, safe_hi.view(np.float32).astype(np.float64))
    xv = mag.view(np.float32).astype(np.float64)
    finite = mag < np.uint32(0x7F800000)
    xv = np.where(finite, xv, 0.0)
    dlo = xv - lo_v
    dhi = hi_v - xv
    lo_even = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (dhi < dlo) | ((dhi == dlo) & ~lo_even)
    out = np.where(take_hi, hi_bits, lo_bits)
    out = np.where(finite, out, mag)                    # +-inf stay inf
    out = out | sign
    isnan = mag > np.uint32(0x7F800000)
    out = np.where(isnan, np.uint32(0x7FC00000), out)
    return (out >> np.uint32(16)).astype(np.uint16)


def round_bf16(x) -> np.ndarray:
    """float64 -> fp32 (nearest) -> bf16 (nearest even) -> float64."""
    return bf16_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32)))


# ----------------------------------------------------------------- e5m2
# OCP e5m2 (the gradient format of the hybrid fp8 recipes): 1 sign, 5
# exponent (bias 15), 2 mantissa bits; exponent field 0 is subnormal
# (m/4 * 2^-14); field 31 is inf (m = 0) or NaN; the largest finite
# magnitude is 1.75 * 2^15 = 57344.  The encoder saturates finite overflow
# to +-57344 (like e4m3fn's satfinite).
E5M2_MAX = 57344.0


def _e5m2_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return s * float("inf") if m == 0 else float("nan")
    if e == 0:
        return s * (m / 4.0) * 2.0 ** -14
    return s * (1.0 + m / 4.0) * 2.0 ** (e - 15)


E5M2_TABLE = np.array([_e5m2_value(c) for c in range(256)], dtype=np.float64)
_E5M2_POS = E5M2_TABLE[:0x7C].copy()          # 0x00 .. 0x7B: non-negative finite values, ascending


def e5m2_to_f64(codes) -> np.ndarray:
    return E5M2_TABLE[np.asarray(codes, dtype=np.uint8)]


def e5m2_encode(x) -> np.ndarray:
    """Nearest e5m2 code to each value (float64 compare), ties to the even
    code, saturating to +-57344; NaN -> 0x7F; the sign is kept for zero."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    idx = np.searchsorted(_E5M2_POS, a, side="left")
    idx = np.clip(idx, 1, len(_E5M2_POS) - 1)
    lo, hi = idx - 1, idx
    dlo = a - _E5M2_POS[lo]
    dhi = _E5M2_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a <= 0.0, 0, code)
    code = np.where(a >= E5M2_MAX, 0x7B, code)
    code = code.astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


# ------------------------------------------------------------------- MX
MX_BLOCK = 32


def e8m0_to_f64(codes) -> np.ndarray:
    """Scale value 2^(E - 127) of E8M0 codes (255, NaN, is not produced here)."""
    e = np.asarray(codes, dtype=np.int64)
    return np.ldexp(1.0, e - 127)


def mx_e4m3_quantize(v) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 (e4m3 elements) of V [rows, K], K % 32 == 0, blocks along the
    last axis.  Returns (codes uint8 [rows, K], scale exponents uint8
    [rows, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    rows, k = v.shape
    assert k % MX_BLOCK == 0
    blocks = v.reshape(rows, k // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(blocks), axis=2)
    e = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.floor(np.log2(amax[nz])).astype(np.int64) - 8 + 127
    # floor(log2) of a value just under a power of two can come out one high
    # in float64 log2; fix it against the definition 2^f <= amax < 2^(f+1)
    f = e - 127 + 8
    hi = nz & (np.ldexp(1.0, f) > amax)
    e[hi] -= 1
    e = np.clip(e, 0, 254)
    scale = np.ldexp(1.0, e - 127)
    codes = e4m3_encode(blocks / scale[:, :, None]).reshape(rows, k)
    return codes, e.astype(np.uint8)


def mx_e4m3_decode(codes, scales) -> np.ndarray:
    """Values X * P of MXFP8 codes [rows, K] with scale exponents [rows, K/32]."""
    c = e4m3_to_f64(codes)
    rows, k = c.shape
    x = e8m0_to_f64(scales)
    return (c.reshape(rows, k // MX_BLOCK, MX_BLOCK) * x[:, :, None]).reshape(rows, k)

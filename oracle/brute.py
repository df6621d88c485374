"""Pure-Python brute force for tiny shapes (oracle cross-check).

Triple loops with math.fsum (a correctly rounded sum of the float64
products), no numpy, so a transposed operand or a wrong index in oracle.ops
shows up as a disagreement.  Same formulas as oracle.ops, written out
element by element from the pages' statements ("Tensor and sequence
parallelism", sections "Derive column-parallel linear algebra" and "Derive
row-parallel linear algebra"; "Tensor parallelism", section "Code").
"""
from __future__ import annotations

import math
import struct


def matmul(a, b):
    """a: list of rows [m][k], b: [k][n] -> [m][n]."""
    m, k, n = len(a), len(b), len(b[0])
    assert all(len(r) == k for r in a)
    return [[math.fsum(a[i][p] * b[p][j] for p in range(k)) for j in range(n)] for i in range(m)]


def transpose(a):
    return [[a[i][j] for i in range(len(a))] for j in range(len(a[0]))]


def relu(a):
    return [[v if v > 0.0 else 0.0 for v in row] for row in a]


def relu_grad_mul(g, z):
    return [[gv if zv > 0.0 else 0.0 for gv, zv in zip(gr, zr)] for gr, zr in zip(g, z)]


def gelu_erf(a):
    return [[0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in row] for row in a]


def gelu_erf_grad_mul(g, z):
    out = []
    for gr, zr in zip(g, z):
        row = []
        for gv, zv in zip(gr, zr):
            cdf = 0.5 * (1.0 + math.erf(zv / math.sqrt(2.0)))
            pdf = math.exp(-0.5 * zv * zv) / math.sqrt(2.0 * math.pi)
            row.append(gv * (cdf + zv * pdf))
        out.append(row)
    return out


def add(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def mlp_fwd(x, w_up, w_down, act="relu"):
    z = matmul(x, w_up)
    h = relu(z) if act == "relu" else gelu_erf(z)
    return z, h, matmul(h, w_down)


def mlp_bwd(x, w_up, w_down, z, h, dy, act="relu"):
    dh = matmul(dy, transpose(w_down))
    dz = relu_grad_mul(dh, z) if act == "relu" else gelu_erf_grad_mul(dh, z)
    return dict(dW_down=matmul(transpose(h), dy), dW_up=matmul(transpose(x), dz),
                dX=matmul(dz, transpose(w_up)), dZ=dz)


def to_lists(arr):
    return [[float(v) for v in row] for row in arr]


# ------------------------------------------------------------------ formats
# Scalar round-to-nearest-even into a binary floating-point format, written
# from the format's definition (sign, exponent range, stored mantissa bits),
# independently of oracle.formats (which searches code tables): a value
# |x| = m * 2^E with E >= emin is represented on the grid of quantum
# 2^(E - mbits); below 2^emin the grid is the subnormal quantum 2^(emin -
# mbits).  x / quantum is exact in float64 (a power-of-two scaling), so
# Python's round() (ties to the even integer) rounds it exactly; the parity
# of that integer is the parity of the code's last mantissa bit.

def fp_rne(x, mbits, emin, fmax, saturate):
    if x != x:
        return float("nan")
    if x == 0.0:
        return x
    a = abs(x)
    _, e = math.frexp(a)                 # a = f * 2^e, f in [0.5, 1)
    E = max(e - 1, emin)
    q = math.ldexp(1.0, E - mbits)
    v = round(a / q) * q
    if v > fmax:
        v = fmax if saturate else float("inf")
    return math.copysign(v, x)


def e4m3(x):
    """OCP e4m3fn: 3 mantissa bits, smallest normal 2^-6, largest 448,
    finite overflow saturates."""
    return fp_rne(x, 3, -6, 448.0, True)


def e5m2(x):
    """OCP e5m2: 2 mantissa bits, smallest normal 2^-14, largest 57344,
    finite overflow saturates (as the encoders of the fp8 recipes do)."""
    return fp_rne(x, 2, -14, 57344.0, True)


def bf16(x):
    """bfloat16 of a float32 value: 7 mantissa bits, smallest normal 2^-126."""
    return fp_rne(x, 7, -126, math.ldexp(2.0 - 2.0 ** -7, 127), False)


def fp32(x):
    """Nearest fp32 value (struct's float conversion, ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _dot(a, b):
    return math.fsum(u * v for u, v in zip(a, b))


def _col(m, j):
    return [row[j] for row in m]


def current_scale(values, fmax, enc):
    """Current scaling of a list of fp32-representable values: amax, the
    fp32 reciprocal scale fmax / amax, the codes' values enc(fp32(v * inv))
    and the fp32 dequantisation factor amax / fmax (inv = s = 1 for amax 0)."""
    amax = max((abs(v) for v in values), default=0.0)
    if amax == 0.0:
        inv, s = 1.0, 1.0
    else:
        inv, s = fp32(fmax / amax), fp32(amax / fmax)
    return amax, inv, s, [enc(fp32(v * inv)) for v in values]


def mlp_fwd_fp8(xq, sx, wu, su, wd, sd, act):
    """fp8 current-scaling MLP forward, element by element: Z = sum xq*wu *
    sx*su; H = act(Z); Hb = bf16(H); Hq = e4m3(fp32(Hb * fp32(448/amax)));
    P = sum Hq*wd * fp32(amax/448)*sd.  Inputs: lists of decoded values."""
    M, F, D = len(xq), len(wu[0]), len(wd[0])
    sxu = fp32(sx) * fp32(su)
    z = [[_dot(xq[i], _col(wu, j)) * sxu for j in range(F)] for i in range(M)]
    h = [[act(v) for v in row] for row in z]
    hb = [[bf16(fp32(v)) for v in row] for row in h]
    amax, inv, s, flat = current_scale([v for row in hb for v in row], 448.0, e4m3)
    hq = [flat[i * F:(i + 1) * F] for i in range(M)]
    p = [[_dot(hq[i], _col(wd, c)) * (s * fp32(sd)) for c in range(D)] for i in range(M)]
    return dict(Z=z, H=h, Hb=hb, amax=amax, inv=inv, sH=s, Hq=hq, P=p)


def mlp_bwd_fp8(x8, sx, wu8, su, wd8, sd, z, h8, sh, dy, act_grad):
    """fp8 backward, element by element: e5m2 current scaling of dY and of
    dZ = bf16(dH * act'(Z)), the weights and activations as decoded e4m3
    values with their scales:
        dH = dYq W_down^T s_dY s_Wd;  dW_down = Hq^T dYq s_H s_dY;
        dW_up = Xq^T dZq s_X s_dZ;   dX = dZq W_up^T s_dZ s_Wu."""
    M, D, F = len(x8), len(x8[0]), len(wu8[0])
    _, _, s_dy, flat = current_scale([v for row in dy for v in row], 57344.0, e5m2)
    dyq = [flat[i * D:(i + 1) * D] for i in range(M)]
    dh = [[_dot(dyq[i], wd8[f]) * (s_dy * fp32(sd)) for f in range(F)] for i in range(M)]
    dz = [[bf16(fp32(dh[i][f] * act_grad(z[i][f]))) for f in range(F)] for i in range(M)]
    _, _, s_dz, flat = current_scale([v for row in dz for v in row], 57344.0, e5m2)
    dzq = [flat[i * F:(i + 1) * F] for i in range(M)]
    dw_down = [[_dot(_col(h8, f), _col(dyq, c)) * (fp32(sh) * s_dy) for c in range(D)] for f in range(F)]
    dw_up = [[_dot(_col(x8, d), _col(dzq, f)) * (fp32(sx) * s_dz) for f in range(F)] for d in range(D)]
    dx = [[_dot(dzq[i], wu8[d]) * (s_dz * fp32(su)) for d in range(D)] for i in range(M)]
    return dict(dYq=dyq, s_dY=s_dy, dH=dh, dZ=dz, dZq=dzq, s_dZ=s_dz, dW_down=dw_down, dW_up=dw_up, dX=dx)


def mx_quantize_row(v):
    """OCP MX (v1.0) with e4m3 elements, blocks of 32 along the row: per
    block X = 2^(floor(log2 amax) - 8) (8 = the exponent of e4m3's largest
    normal), scale code E = that exponent + 127 clamped to [0, 254] (0 for an
    all-zero block), elements e4m3(v / X).  Returns (values X*P, codes E)."""
    vals, exps = [], []
    for b in range(0, len(v), 32):
        blk = v[b:b + 32]
        amax = max(abs(t) for t in blk)
        if amax == 0.0:
            E = 0
        else:
            _, e = math.frexp(amax)          # floor(log2 amax) = e - 1
            E = min(max(e - 1 - 8 + 127, 0), 254)
        X = math.ldexp(1.0, E - 127)
        vals += [e4m3(t / X) * X for t in blk]
        exps.append(E)
    return vals, exps


def mlp_fwd_mx(x, wu_t, wd_t, act):
    """MXFP8 MLP forward, element by element: x [M, D], wu_t [F, D] and
    wd_t [D, F] already-decoded MX values (K-major rows); Z = x . wu_t^T,
    H = act(Z), H requantised to MXFP8 along its rows, P = Hmx . wd_t^T."""
    z = [[_dot(xr, wr) for wr in wu_t] for xr in x]
    h = [[act(t) for t in row] for row in z]
    hq = [mx_quantize_row(row) for row in h]
    p = [[_dot(hv, wr) for wr in wd_t] for hv, _ in hq]
    return dict(Z=z, H=h, Hq=[a for a, _ in hq], Hexp=[b for _, b in hq], P=p)

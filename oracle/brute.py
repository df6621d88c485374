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

"""The operations of one tensor-parallel rank's MLP share, in float64.

Sources (page title, section):
  [TP]   "Tensor parallelism" (algorithm page): "How it works" (the MLP
         Y = GeLU(X.A).B with A split by columns and B by rows; one sum of
         partials in forward, one in backward), "Code" (the Megatron MLP
         checker: ReLU, its derivative taken as 1 only where z > 0, and the
         backward of the loss 1/2 ||Y||^2 so that dY = Y).
  [TSP]  "Tensor and sequence parallelism": "Derive column-parallel linear
         algebra" (Y_t = X W_t; dW_t = X^T dY_t; dX_t = dY_t W_t^T is a full
         [M,K] partial), "Derive row-parallel linear algebra" (partial
         Y_t = X_t W_t of shape [M,N]; Y = sum_t Y_t; dW_t = X_t^T dY;
         dX_t = dY W_t^T), "Pair adjacent transformer projections".
  [CG]   "Collective GEMMs in Tensor Sequence Parallelism": "Collective GEMMs
         (CGEMM)" (sequence chunks give distinct output rows, no accumulation;
         the reduce-scatter delivers each rank its token range of the summed
         partial), "Supported quantization recipes" (FP8 current scaling).
  [WE]   "Tensor and sequence parallelism", "Worked example: Partitioning an
         MLP pair": an expansion weight and a gate weight, each column-
         partitioned, a gated activation applied locally, and a row-
         partitioned contraction producing a partial.  The page does not say
         which gated activation; the functions below take the gated-linear-
         unit form act(X W_gate) * (X W_up) (Shazeer, "GLU Variants Improve
         Transformer") with the activation as an argument; SiLU gives SwiGLU.

Matrices are row-major [rows, cols] as the pages write them: X[M,K], W[K,N].
Every function takes float64 arrays holding exactly the values the GPU
receives (decoded from bf16 / e4m3fn by oracle.formats).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from . import formats

ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH, ACT_SILU = 0, 1, 2, 3, 4
_SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
_GELU_TANH_C = 0.044715


# ---------------------------------------------------------------- activations
def relu(z):
    """[TP] "Code": max(z, 0)."""
    return np.maximum(z, 0.0)


def relu_grad(z):
    """[TP] "Code": the derivative is taken as 1 where z > 0 and 0 elsewhere
    (including z == 0)."""
    return (z > 0.0).astype(np.float64)


def gelu_erf(z):
    """GeLU, exact form: z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2))."""
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def gelu_erf_grad(z):
    """d/dz [z Phi(z)] = Phi(z) + z phi(z)."""
    cdf = 0.5 * (1.0 + erf(z / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return cdf + z * pdf


def gelu_tanh(z):
    """GeLU, tanh approximation (Hendrycks & Gimpel):
    0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))."""
    u = _SQRT_2_OVER_PI * (z + _GELU_TANH_C * z ** 3)
    return 0.5 * z * (1.0 + np.tanh(u))


def gelu_tanh_grad(z):
    u = _SQRT_2_OVER_PI * (z + _GELU_TANH_C * z ** 3)
    t = np.tanh(u)
    du = _SQRT_2_OVER_PI * (1.0 + 3.0 * _GELU_TANH_C * z * z)
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du


def silu(z):
    """SiLU (swish with unit slope): z * sigma(z), sigma the logistic function
    1 / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def silu_grad(z):
    """d/dz [z sigma(z)] = sigma(z) + z sigma(z) (1 - sigma(z))."""
    z = np.asarray(z, dtype=np.float64)
    sig = 1.0 / (1.0 + np.exp(-z))
    return sig + z * sig * (1.0 - sig)


def act_fwd(z, act: int):
    if act == ACT_NONE:
        return np.array(z, dtype=np.float64, copy=True)
    if act == ACT_RELU:
        return relu(z)
    if act == ACT_GELU_ERF:
        return gelu_erf(z)
    if act == ACT_GELU_TANH:
        return gelu_tanh(z)
    if act == ACT_SILU:
        return silu(z)
    raise ValueError(f"unknown activation {act}")


def act_grad(z, act: int):
    if act == ACT_NONE:
        return np.ones_like(z, dtype=np.float64)
    if act == ACT_RELU:
        return relu_grad(z)
    if act == ACT_GELU_ERF:
        return gelu_erf_grad(z)
    if act == ACT_GELU_TANH:
        return gelu_tanh_grad(z)
    if act == ACT_SILU:
        return silu_grad(z)
    raise ValueError(f"unknown activation {act}")


# ---------------------------------------------------------------------- GEMM
def gemm(a, b):
    """C = A.B in float64 (library matmul as the step)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.ndim == 2 and b.ndim == 2 and a.shape[1] == b.shape[0], (a.shape, b.shape)
    return a @ b


def op(m, trans: bool):
    """op(M) = M or M^T (a transpose by index, as the page's transpose())."""
    return np.asarray(m, dtype=np.float64).T if trans else np.asarray(m, dtype=np.float64)


# ------------------------------------------------------------------ sharding
def col_block(w, T: int, t: int):
    """Columns [t*N/T, (t+1)*N/T) of W[K,N] -- the column-parallel shard
    ([TSP] "Derive column-parallel linear algebra"; [TP] "Code" col_block)."""
    n = w.shape[1]
    assert n % T == 0
    s = n // T
    return w[:, t * s:(t + 1) * s]


def row_block(w, T: int, t: int):
    """Rows [t*K/T, (t+1)*K/T) of W[K,N] -- the row-parallel shard
    ([TSP] "Derive row-parallel linear algebra")."""
    k = w.shape[0]
    assert k % T == 0
    s = k // T
    return w[t * s:(t + 1) * s, :]


# ---------------------------------------------------------- seq_chunk_gemm
def seq_chunk_gemm(a, b, *, trans_a=False, trans_b=False, a_scale=1.0, b_scale=1.0,
                   act=ACT_NONE, dact_z=None, chunk_rows=None, chunk_order=None):
    """Y = act(op(A).op(B) * sa * sb), or, with dact_z given, the backward
    epilogue Y = (op(A).op(B) * sa * sb) * act'(Z).

    Returns (Y, Zpre) where Zpre is the pre-activation product.
    Chunking: the rows of Y (tokens) arrive as chunks in `chunk_order`; each
    chunk produces distinct output rows with no accumulation ([CG]
    "Collective GEMMs (CGEMM)", all-gather + GEMM), so the result is the
    unchunked product whatever the order; the arguments are only checked."""
    A = op(a, trans_a)
    B = op(b, trans_b)
    z = gemm(A, B) * (float(a_scale) * float(b_scale))
    if chunk_order is not None:
        assert chunk_rows is not None and z.shape[0] % chunk_rows == 0
        assert sorted(chunk_order) == list(range(z.shape[0] // chunk_rows))
    if dact_z is not None:
        return z * act_grad(np.asarray(dact_z, dtype=np.float64), act), z
    return act_fwd(z, act), z


# -------------------------------------------------------------- tp_mlp_fwd
def _stored(v, store):
    """The value a later step reads back: exact (store=None) or rounded to
    the storage format the path keeps intermediates in (store='bf16')."""
    if store is None:
        return v
    if store == "bf16":
        return formats.round_bf16(v)
    raise ValueError(store)


def tp_mlp_fwd(x, w_up_t, w_down_t, act=ACT_GELU_ERF, store=None):
    """One rank's MLP share ([TP] "How it works"; [TSP] "Pair adjacent
    transformer projections"):
        Z_t = X . W_up,t        (column-parallel, [M, F/T])
        H_t = act(Z_t)          (local activation)
        P_t = H_t . W_down,t    (row-parallel partial, [M, D])
    store='bf16': the second GEMM reads H_t as stored in bf16 (the
    intermediate activation is kept in the activation dtype); otherwise all
    of it is exact."""
    z = gemm(x, w_up_t)
    h = act_fwd(z, act)
    p = gemm(_stored(h, store), w_down_t)
    return dict(Z=z, H=h, P=p)


def tp_mlp_fwd_fp8(xq, sx, wq_up, s_up, wq_down, s_down, act=ACT_GELU_ERF):
    """fp8 current-scaling variant ([CG] "Supported quantization recipes",
    FP8 with current scaling), with the rounding points of the GPU path:
        Z   = (Xq . Wq_up) * sX * sWup            (operands decoded exactly)
        H_b = bf16(act(Z))                        (stored intermediate)
        amax = max |H_b|
        inv = fp32(448 / amax)   (1 when amax == 0)
        Hq  = e4m3(fp32(H_b * inv))               (nearest even, satfinite)
        sH  = fp32(amax / 448)   (1 when amax == 0)
        P   = (Hq . Wq_down) * sH * sWdown
    Inputs are decoded values (float64) of the e4m3 codes and fp32 scales."""
    z = gemm(xq, wq_up) * (float(np.float32(sx)) * float(np.float32(s_up)))
    h = act_fwd(z, act)
    hb = formats.round_bf16(h)
    q = quantize_current(hb, "e4m3")
    p = gemm(q["dec"], wq_down) * (q["s"] * float(np.float32(s_down)))
    return dict(Z=z, H=h, Hb=hb, amax=q["amax"], inv=q["inv"], sH=q["s"], Hq_codes=q["codes"], P=p)


def quantize_current(v, fmt: str):
    """Per-tensor current scaling ([CG] "Supported quantization recipes", FP8
    with current scaling; the formula is the reading the pages leave open)
    of a tensor v whose values are already fp32-representable (here always
    bf16 values), to fp8 format fmt ('e4m3', largest 448, or 'e5m2',
    largest 57344):
        amax = max |v|
        inv  = fp32(fmax / amax)      (1 when amax == 0)
        q    = enc(fp32(v * inv))     nearest even, saturating
        s    = fp32(amax / fmax)      (1 when amax == 0), the dequant factor
    The two fp32 roundings are the GPU path's: inv is an fp32 quotient and
    the scaled value an fp32 product, each rounded once."""
    enc, dec_tab, fmax = ((formats.e4m3_encode, formats.e4m3_to_f64, formats.E4M3_MAX) if fmt == "e4m3"
                          else (formats.e5m2_encode, formats.e5m2_to_f64, formats.E5M2_MAX))
    v = np.asarray(v, dtype=np.float64)
    amax = float(np.max(np.abs(v))) if v.size else 0.0
    a32 = np.float32(amax)
    assert float(a32) == amax, "amax must be fp32-representable"
    if amax == 0.0:
        inv32, s32 = np.float32(1.0), np.float32(1.0)
    else:
        inv32 = np.float32(np.float32(fmax) / a32)
        s32 = np.float32(a32 / np.float32(fmax))
    prod32 = (v.astype(np.float32) * inv32).astype(np.float32)
    codes = enc(prod32.astype(np.float64))
    return dict(codes=codes, dec=dec_tab(codes), inv=float(inv32), s=float(s32), amax=amax)


# ------------------------------------------------- partial_reduce_seqshard


def tp_mlp_bwd_fp8(x8, sx, wu8, su, wd8, sd, z, h8, sh, dy, act=ACT_GELU_ERF, dz_stored=None):
    """fp8 backward of one rank's MLP share (the backward the fp8 recipes of
    [CG] "Supported quantization recipes" imply; the pages do not spell it
    out): activations and weights in e4m3 with their forward scales,
    gradients in e5m2 with current scaling, the chain of tp_mlp_bwd:
        dYq = e5m2(fp32(dY * fp32(57344 / amax dY))),  s_dY = fp32(amax dY / 57344)
        dH  = (dYq . W_down,t^T) * s_dY * s_Wd
        dZ  = bf16(dH * act'(Z))                       (stored intermediate)
        dZq = e5m2(fp32(dZ * fp32(57344 / amax dZ))),  s_dZ
        dW_down,t = (Hq^T . dYq) * s_H * s_dY
        dW_up,t   = (Xq^T . dZq) * s_X * s_dZ
        dX_t      = (dZq . W_up,t^T) * s_dZ * s_Wu
    Inputs: decoded e4m3 values of X [M, D], W_up,t [D, F/T], W_down,t
    [F/T, D], H [M, F/T] with their fp32 scales; Z and dY as bf16 values.
    dz_stored: the stored bf16 dZ a GPU produced (its saved intermediate, an
    input of the later GEMMs); when given, the chain continues from it."""
    f = lambda v: float(np.float32(v))
    qy = quantize_current(dy, "e5m2")
    dyq, s_dy = qy["dec"], qy["s"]
    dh = gemm(dyq, np.asarray(wd8, dtype=np.float64).T) * (s_dy * f(sd))
    dz = formats.round_bf16(dh * act_grad(np.asarray(z, dtype=np.float64), act))
    if dz_stored is not None:
        dz = np.asarray(dz_stored, dtype=np.float64)
    qz = quantize_current(dz, "e5m2")
    dzq, s_dz = qz["dec"], qz["s"]
    dw_down = gemm(np.asarray(h8, dtype=np.float64).T, dyq) * (f(sh) * s_dy)
    dw_up = gemm(np.asarray(x8, dtype=np.float64).T, dzq) * (f(sx) * s_dz)
    dx = gemm(dzq, np.asarray(wu8, dtype=np.float64).T) * (s_dz * f(su))
    return dict(dYq=dyq, s_dY=s_dy, amax_dY=qy["amax"], dH=dh, dZ=dz, dZq=dzq, s_dZ=s_dz,
                amax_dZ=qz["amax"], dW_down=dw_down, dW_up=dw_up, dX=dx)


def fp8_delayed_scale(amax_history):
    """Dequantisation factor of a tensor under delayed scaling ([CG]
    "Supported quantization recipes", FP8 with delayed scaling; the page
    names the recipe only): the largest amax recorded over the history
    window, divided by 448 in fp32 (1 when every entry is 0)."""
    a = float(np.max(np.asarray(amax_history, dtype=np.float64))) if len(amax_history) else 0.0
    a32 = np.float32(a)
    return float(np.float32(a32 / np.float32(448.0))) if a32 > 0 else 1.0


def tp_mlp_fwd_fp8_delayed(xq, sx, wq_up, s_up, wq_down, s_down, s_h, act=ACT_GELU_ERF):
    """fp8 forward under delayed scaling: H is quantised with a scale s_H
    fixed before the step (from earlier steps' amax), so GEMM1 can write it
    as e4m3 directly; the step's own amax of H is recorded for later steps.
        Z   = (Xq . Wq_up) * sX * sWup
        H   = act(Z)
        inv = fp32(1 / s_H)
        Hq  = e4m3(fp32(H * inv))                 (nearest even, saturating)
        P   = (Hq . Wq_down) * s_H * sWdown
        amax = max |H|
    Inputs are decoded values (float64) of the e4m3 codes and fp32 scales."""
    z = gemm(xq, wq_up) * (float(np.float32(sx)) * float(np.float32(s_up)))
    h = act_fwd(z, act)
    inv32 = np.float32(np.float32(1.0) / np.float32(s_h))
    prod32 = (h * float(inv32)).astype(np.float32)
    hq_codes = formats.e4m3_encode(prod32.astype(np.float64))
    hq = formats.e4m3_to_f64(hq_codes)
    p = gemm(hq, wq_down) * (float(np.float32(s_h)) * float(np.float32(s_down)))
    amax = float(np.max(np.abs(h))) if h.size else 0.0
    return dict(Z=z, H=h, inv=float(inv32), Hq_codes=hq_codes, P=p, amax=amax)


def tp_mlp_fwd_mx(xq, xs, wuq_t, wus_t, wdq_t, wds_t, act=ACT_GELU_ERF):
    """MXFP8 block-scaling variant ([CG] "Supported quantization recipes",
    MXFP8 block scaling; format in oracle.formats) with the rounding points
    of the GPU path.  Every operand is MXFP8 with its blocks along the
    contraction dimension, so the weights come K-major (transposed):
        Z  = dec(Xq, Xs) . dec(Wq_up^T, Ws_up^T)^T          [M, F/T]
        H  = act(Z)
        Hq, Hs = MXFP8(H)   (blocks of 32 along F/T, no bf16 step)
        P  = dec(Hq, Hs) . dec(Wq_down^T, Ws_down^T)^T      [M, D]
    Inputs: e4m3 codes and E8M0 scale exponents (row-major [rows, K/32])."""
    z = gemm(formats.mx_e4m3_decode(xq, xs), formats.mx_e4m3_decode(wuq_t, wus_t).T)
    h = act_fwd(z, act)
    hq, hs = formats.mx_e4m3_quantize(h)
    p = gemm(formats.mx_e4m3_decode(hq, hs), formats.mx_e4m3_decode(wdq_t, wds_t).T)
    return dict(Z=z, H=h, Hq_codes=hq, Hq_scales=hs, P=p)


def partial_reduce_seqshard(partials, rank: int):
    """Local arithmetic of the reduce-scatter that follows a row-parallel GEMM
    ([CG] "Collective GEMMs (CGEMM)", GEMM + reduce-scatter; [TSP] "Derive
    row-parallel linear algebra"): rank r receives rows
    [r*M/T, (r+1)*M/T) of sum_t P_t.  partials: [T, M, D].
    rank = -1: each partial already holds only this rank's rows (a receive
    buffer [T, M/T, D]); the result is their sum."""
    p = np.asarray(partials, dtype=np.float64)
    T, M, _ = p.shape
    if rank < 0:
        return p.sum(axis=0)
    assert M % T == 0
    s = M // T
    return p[:, rank * s:(rank + 1) * s, :].sum(axis=0)


# -------------------------------------------------------------- tp_mlp_bwd
def tp_mlp_bwd(x, w_up_t, w_down_t, z, h, dy, act=ACT_GELU_ERF, store=None, dz_stored=None):
    """Backward of one rank's MLP share ([TSP] both derivations; [TP] "Code"):
        dH_t      = dY . W_down,t^T        (row-parallel input gradient shard)
        dZ_t      = dH_t * act'(Z_t)
        dW_down,t = H_t^T . dY             (row-parallel weight gradient)
        dW_up,t   = X^T . dZ_t             (column-parallel weight gradient)
        dX_t      = dZ_t . W_up,t^T        (full [M,D] partial, summed across
                                            ranks by all-reduce / reduce-scatter)
    Z and H are the saved forward values (inputs here).  store='bf16': the
    two GEMMs that consume dZ_t read it as stored in bf16.  dz_stored: the
    dZ_t a GPU stored (its saved intermediate): the two GEMMs that consume
    dZ_t read it instead."""
    dh = gemm(dy, np.asarray(w_down_t, dtype=np.float64).T)
    dz = dh * act_grad(np.asarray(z, dtype=np.float64), act)
    dw_down = gemm(np.asarray(h, dtype=np.float64).T, dy)
    dzs = _stored(dz, store) if dz_stored is None else np.asarray(dz_stored, dtype=np.float64)
    dw_up = gemm(np.asarray(x, dtype=np.float64).T, dzs)
    dx = gemm(dzs, np.asarray(w_up_t, dtype=np.float64).T)
    return dict(dH=dh, dZ=dz, dW_down=dw_down, dW_up=dw_up, dX=dx)


def linear_bwd(x, w, dy):
    """Backward of one sharded linear layer Y = X . W ([TSP] "Derive
    column-parallel linear algebra" and "Derive row-parallel linear
    algebra"; the attention projections of [TSP] "Pair adjacent transformer
    projections" are such layers):
        dW = X^T . dY      (same shape as W, [K, N])
        dX = dY . W^T      ([M, K]; for a column-parallel W it is a full
                            partial summed across ranks, for a row-parallel
                            W the rank's shard of the input gradient)
    The two products read the same dY and are independent of each other."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    assert x.shape[1] == w.shape[0] and dy.shape == (x.shape[0], w.shape[1]), (x.shape, w.shape, dy.shape)
    return dict(dW=gemm(x.T, dy), dX=gemm(dy, w.T))


# ------------------------------------------------------- gated MLP share
def gated_mlp_fwd(x, w_gate_t, w_up_t, w_down_t, act=ACT_SILU, store=None):
    """One rank's share of the gated MLP of [WE]:
        G_t = X . W_gate,t       (column-parallel, [M, F/T])
        U_t = X . W_up,t         (column-parallel, [M, F/T])
        H_t = act(G_t) * U_t     (gated activation, local, element-wise)
        P_t = H_t . W_down,t     (row-parallel partial, [M, D])
    store='bf16': the second GEMM reads H_t as stored in bf16."""
    g = gemm(x, w_gate_t)
    u = gemm(x, w_up_t)
    h = act_fwd(g, act) * u
    p = gemm(_stored(h, store), w_down_t)
    return dict(G=g, U=u, H=h, P=p)


def gated_mlp_bwd(x, w_gate_t, w_up_t, w_down_t, g, u, h, dy, act=ACT_SILU, store=None):
    """Backward of gated_mlp_fwd by the chain rule, with the layouts of
    [TSP] "Derive column-parallel linear algebra" / "Derive row-parallel
    linear algebra" for the three projections:
        dH_t      = dY . W_down,t^T
        dG_t      = dH_t * U_t * act'(G_t)
        dU_t      = dH_t * act(G_t)
        dW_down,t = H_t^T . dY
        dW_gate,t = X^T . dG_t,   dW_up,t = X^T . dU_t
        dX_t      = dG_t . W_gate,t^T + dU_t . W_up,t^T   (full [M,D] partial)
    G, U, H are the saved forward values.  store='bf16': the GEMMs that
    consume dG_t and dU_t read them as stored in bf16."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    dh = gemm(dy, np.asarray(w_down_t, dtype=np.float64).T)
    dg = dh * u * act_grad(g, act)
    du = dh * act_fwd(g, act)
    dw_down = gemm(np.asarray(h, dtype=np.float64).T, dy)
    dgs, dus = _stored(dg, store), _stored(du, store)
    xt = np.asarray(x, dtype=np.float64).T
    dx = gemm(dgs, np.asarray(w_gate_t, dtype=np.float64).T) + gemm(dus, np.asarray(w_up_t, dtype=np.float64).T)
    return dict(dH=dh, dG=dg, dU=du, dW_down=dw_down, dW_gate=gemm(xt, dgs), dW_up=gemm(xt, dus), dX=dx)


# ------------------------------------------------------- unsharded reference
def mlp_unsharded(x, a, b, act=ACT_RELU):
    """The unsharded layer Y = act(X A) B that the sharded ranks must match
    ([TP] "Overview" / "Code")."""
    pre = gemm(x, a)
    return dict(pre=pre, Y=gemm(act_fwd(pre, act), b))


def mlp_unsharded_bwd(x, a, b, pre, dy, act=ACT_RELU):
    dh = gemm(dy, np.asarray(b, dtype=np.float64).T) * act_grad(pre, act)
    return dict(dA=gemm(np.asarray(x, dtype=np.float64).T, dh),
                dB=gemm(np.asarray(act_fwd(pre, act)).T, dy),
                dX=gemm(dh, np.asarray(a, dtype=np.float64).T))


# ---------------------------------------------------------------- comparison
def normalized_error(gpu, ref):
    """max |g - r| / (1 + |r|), the parity measure of this path."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r) / (1.0 + np.abs(r))))

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded inputs.  Bars: bit-exact for integer-valued inputs and for
chunk-order permutations; max |gpu - ref| / (1 + |ref|) <= 1e-4 (fp32),
2e-2 (bf16), 6e-2 (fp8 e4m3)."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import formats, ops
from tests import _util
from tests._util import TOL, assert_mx_close, f64, nerr

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sequence_transformer_gemms_amd as tpm
    from sequence_transformer_gemms_amd import _abi


def dev_bf16(x):
    return si.to_bf16(x).cuda()


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ reduction
@pytest.mark.parametrize("D", [1024, 136])
def test_reduce_bf16_all_ranks(D):
    T, M = 4, 64
    parts = np.stack([si.normal_f32((M, D), 100 + t) for t in range(T)])
    P = si.to_bf16(parts).cuda()
    ref_in = f64(P)
    outs = []
    for r in range(T):
        out = torch.empty(M // T, D, dtype=torch.bfloat16, device="cuda")
        tpm.partial_reduce_seqshard(P, out, T=T, rank=r)
        outs.append(out)
    sync()
    for r in range(T):
        assert nerr(outs[r], ops.partial_reduce_seqshard(ref_in, r)) <= TOL["bf16"]
    # concatenation over ranks = full sum (all-reduce = reduce-scatter + all-gather)
    cat = np.concatenate([f64(o) for o in outs])
    assert nerr(cat, ref_in.sum(axis=0)) <= TOL["bf16"]


def test_reduce_integer_exact_and_receive_buffer_layout():
    T, M, D = 8, 128, 256
    parts = np.stack([si.small_ints((M, D), 200 + t, -15, 15) for t in range(T)])
    P = si.to_bf16(parts).cuda()
    out = torch.empty(M // T, D, dtype=torch.bfloat16, device="cuda")
    tpm.partial_reduce_seqshard(P, out, T=T, rank=5)
    # receive-buffer layout [T, M/T, D] (rank = -1)
    recv = P[:, 5 * (M // T):6 * (M // T), :].contiguous()
    out2 = torch.empty_like(out)
    tpm.partial_reduce_seqshard(recv, out2, T=T, rank=-1)
    sync()
    ref = ops.partial_reduce_seqshard(parts.astype(np.float64), 5)
    assert np.array_equal(f64(out), ref)          # |sum| <= 120 < 256: exact in bf16
    assert torch.equal(out, out2)


def test_reduce_fp32():
    T, M, D = 4, 8, 32
    parts = np.stack([si.uniform_f32((M, D), 300 + t) for t in range(T)])
    P = dev_f32(parts)
    out = torch.empty(M // T, D, dtype=torch.float32, device="cuda")
    tpm.partial_reduce_seqshard(P, out, T=T, rank=1)
    sync()
    assert nerr(out, ops.partial_reduce_seqshard(parts.astype(np.float64), 1)) <= TOL["f32"]


def test_reduce_c3_full_size():
    # 8 seeded bf16 partials [8192, 8192] -> rank slice [1024, 8192]
    T, M, D = 8, 8192, 8192
    P = torch.empty(T, M, D, dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        P[t] = dev_bf16(si.normal_f32((M, D), 100 + t))
    out = torch.empty(M // T, D, dtype=torch.bfloat16, device="cuda")
    for r in (0, 3, 7):
        tpm.partial_reduce_seqshard(P, out, T=T, rank=r)
        sync()
        held = np.stack([f64(P[t, r * (M // T):(r + 1) * (M // T)]) for t in range(T)])
        assert nerr(out, ops.partial_reduce_seqshard(held, -1)) <= TOL["bf16"]


# ------------------------------------------------------------------ GEMM
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


def _operands(M, N, K, ta, tb, gen, seed):
    a = gen((M, K), seed)
    b = gen((K, N), seed + 1)
    A = np.ascontiguousarray(a.T) if ta else a
    B = np.ascontiguousarray(b.T) if tb else b
    return a, b, A, B


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_gemm_bf16_integer_exact_all_layouts(ta, tb):
    # small integers: every fp32 partial sum is exact, so the result is
    # independent of tiling and must equal the oracle bit for bit
    M, N, K = (296 if ta else 300), 264, 200
    gen = lambda s, seed: si.small_ints(s, seed)
    a, b, A, B = _operands(M, N, K, ta, tb, gen, 11)
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(dev_bf16(A), dev_bf16(B), Y, trans_a=ta, trans_b=tb, M=M, N=N, K=K)
    sync()
    ref, _ = ops.seq_chunk_gemm(A, B, trans_a=ta, trans_b=tb)
    assert np.array_equal(f64(Y), ref)


@pytest.mark.parametrize("act", [_abi.ACT_NONE, _abi.ACT_RELU, _abi.ACT_GELU_ERF, _abi.ACT_GELU_TANH]
                         if torch.cuda.is_available() else [])
def test_gemm_bf16_activations_and_zsave(act):
    M, N, K = 640, 392, 328
    a, b, A, B = _operands(M, N, K, False, False, lambda s, seed: si.normal_f32(s, seed, 0.5), 21)
    Ad, Bd = dev_bf16(A), dev_bf16(B)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(Ad, Bd, Y, act=act, aux=Z)
    sync()
    y, z = ops.seq_chunk_gemm(f64(Ad), f64(Bd), act=act)
    assert nerr(Y, y) <= TOL["bf16"]
    assert nerr(Z, z) <= TOL["bf16"]


def test_gemm_chunk_order_is_bitwise_invariant():
    M, N, K = 1024, 512, 256
    a, b, A, B = _operands(M, N, K, False, False, lambda s, seed: si.normal_f32(s, seed), 31)
    Ad, Bd = dev_bf16(A), dev_bf16(B)
    outs = []
    for C, order in ((1, None), (4, [0, 3, 2, 1]), (8, [5, 0, 7, 1, 6, 2, 4, 3]), (16, list(range(15, -1, -1)))):
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        tpm.seq_chunk_gemm(Ad, Bd, Y, act=_abi.ACT_GELU_ERF, num_chunks=C, chunk_order=order)
        outs.append(Y)
    sync()
    for Y in outs[1:]:
        assert torch.equal(Y, outs[0])
    y, _ = ops.seq_chunk_gemm(f64(Ad), f64(Bd), act=_abi.ACT_GELU_ERF)
    assert nerr(outs[0], y) <= TOL["bf16"]


@pytest.mark.parametrize("act", [_abi.ACT_RELU, _abi.ACT_GELU_ERF] if torch.cuda.is_available() else [])
def test_gemm_dact_epilogue(act):
    M, N, K = 520, 256, 384
    a, b, A, B = _operands(M, N, K, False, True, lambda s, seed: si.normal_f32(s, seed), 41)
    Ad, Bd = dev_bf16(A), dev_bf16(B)
    Zd = dev_bf16(si.normal_f32((M, N), 43))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(Ad, Bd, Y, trans_b=True, epilogue=_abi.EPI_DACT, act=act, aux=Zd)
    sync()
    y, _ = ops.seq_chunk_gemm(f64(Ad), f64(Bd), trans_b=True, act=act, dact_z=f64(Zd))
    assert nerr(Y, y) <= TOL["bf16"]


def test_gemm_empty_and_k_zero():
    A = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    Y = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(A, B, Y)
    A = torch.zeros(64, 0, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((64, 64), 7.0, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(A, B, Y, M=64, N=64, K=0)
    sync()
    assert torch.count_nonzero(Y).item() == 0


def test_gemm_fp8_integer_exact_and_scaled():
    M, N, K = 300, 264, 320
    a = si.small_ints((M, K), 51, -4, 4)
    bt = si.small_ints((N, K), 52, -4, 4)        # B stored [N, K] (K-major)
    Aq, Bq = si.to_e4m3_exact(a).cuda(), si.to_e4m3_exact(bt).cuda()
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(Aq, Bq, Y, trans_b=True)
    sync()
    assert np.array_equal(f64(Y), a.astype(np.float64) @ bt.astype(np.float64).T)
    # normal values with per-tensor current scales
    x = si.normal_f32((M, K), 53)
    w = si.normal_f32((N, K), 54, 0.02)
    xq, sx = si.to_e4m3_current(x)
    wq, sw = si.to_e4m3_current(w)
    scales = dev_f32(np.array([sx, sw], dtype=np.float32))
    Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    tpm.seq_chunk_gemm(xq.cuda(), wq.cuda(), Yb, trans_b=True, a_scale=scales[0:1], b_scale=scales[1:2],
                       act=_abi.ACT_GELU_ERF, amax_out=amax, workspace=ws)
    sync()
    y, _ = ops.seq_chunk_gemm(f64(xq), f64(wq), trans_b=True, a_scale=sx, b_scale=sw, act=_abi.ACT_GELU_ERF)
    assert nerr(Yb, y) <= TOL["fp8"]
    assert amax.item() == float(np.max(np.abs(f64(Yb))))


# ------------------------------------------------------------- MLP, fp32 (C1)
@pytest.mark.parametrize("generator", ["page3", "pcg"])
def test_c1_tiny_mlp_fp32_fwd_bwd(generator):
    c = si.c1_tiny_mlp(generator)
    m, d, f, T = c["m"], c["d"], c["f"], c["t"]
    x, a, b = c["x"], c["a"], c["b"]
    X = dev_f32(x)
    P_all = torch.empty(T, m, d, dtype=torch.float32, device="cuda")
    Zs, Hs = [], []
    for t in range(T):
        wu = dev_f32(ops.col_block(a, T, t))
        wd = dev_f32(ops.row_block(b, T, t))
        Z = torch.empty(m, f // T, dtype=torch.float32, device="cuda")
        H = torch.empty_like(Z)
        tpm.tp_mlp_fwd(X, wu, wd, H, P_all[t], T=T, rank=t, act=_abi.ACT_RELU, Z_t=Z)
        Zs.append(Z)
        Hs.append(H)
    # all-reduce = reduce-scatter (each rank's slice) + all-gather
    Y = torch.empty(m, d, dtype=torch.float32, device="cuda")
    for r in range(T):
        tpm.partial_reduce_seqshard(P_all, Y[r * (m // T):(r + 1) * (m // T)], T=T, rank=r)
    sync()
    un = ops.mlp_unsharded(x.astype(np.float64), a.astype(np.float64), b.astype(np.float64), ops.ACT_RELU)
    for t in range(T):
        ref = ops.tp_mlp_fwd(x, ops.col_block(a, T, t), ops.row_block(b, T, t), ops.ACT_RELU)
        assert nerr(P_all[t], ref["P"]) <= TOL["f32"]
    assert nerr(Y, un["Y"]) <= TOL["f32"]
    # backward with the page's loss 1/2 ||Y||^2 -> dY = Y
    dY = Y.clone()
    dX_all = torch.empty(T, m, d, dtype=torch.float32, device="cuda")
    dWu, dWd = [], []
    for t in range(T):
        wu = dev_f32(ops.col_block(a, T, t))
        wd = dev_f32(ops.row_block(b, T, t))
        gu = torch.empty(d, f // T, dtype=torch.float32, device="cuda")
        gd = torch.empty(f // T, d, dtype=torch.float32, device="cuda")
        ws = tpm.alloc_workspace(_abi.OP_MLP_BWD, m, d, f, T, 1, _abi.F32)
        tpm.tp_mlp_bwd(X, wu, wd, Zs[t], Hs[t], dY, gu, gd, dX_all[t], T=T, rank=t, act=_abi.ACT_RELU,
                       workspace=ws)
        dWu.append(gu)
        dWd.append(gd)
    dX = torch.empty(m, d, dtype=torch.float32, device="cuda")
    for r in range(T):
        tpm.partial_reduce_seqshard(dX_all, dX[r * (m // T):(r + 1) * (m // T)], T=T, rank=r)
    sync()
    dy = f64(dY)
    unb = ops.mlp_unsharded_bwd(x.astype(np.float64), a.astype(np.float64), b.astype(np.float64), un["pre"], dy,
                                ops.ACT_RELU)
    for t in range(T):
        assert nerr(dWu[t], ops.col_block(unb["dA"], T, t)) <= TOL["f32"]
        assert nerr(dWd[t], ops.row_block(unb["dB"], T, t)) <= TOL["f32"]
    assert nerr(dX, unb["dX"]) <= TOL["f32"]


# ------------------------------------------------------------- MLP, bf16
def _mlp_inputs(M, D, F, T, seed=1, sx=1.0, sw=0.02):
    Ft = F // T
    x = si.normal_f32((M, D), seed, sx)
    wu = si.normal_f32((D, Ft), seed + 1, sw)
    wd = si.normal_f32((Ft, D), seed + 2, sw)
    return x, wu, wd


@pytest.mark.parametrize("act", [_abi.ACT_GELU_ERF, _abi.ACT_RELU] if torch.cuda.is_available() else [])
def test_mlp_fwd_bwd_bf16_small(act):
    M, D, F, T, C = 512, 256, 1024, 4, 8
    x, wu, wd = _mlp_inputs(M, D, F, T, sw=0.05)
    X, WU, WD = dev_bf16(x), dev_bf16(wu), dev_bf16(wd)
    Ft = F // T
    Z = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    H = torch.empty_like(Z)
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, C, _abi.BF16)
    done = torch.zeros(T, dtype=torch.int32, device="cuda")
    tpm.tp_mlp_fwd(X, WU, WD, H, P, T=T, rank=1, act=act, Z_t=Z, num_chunks=C, epoch=3, range_done=done,
                   workspace=ws)
    sync()
    ref = ops.tp_mlp_fwd(f64(X), f64(WU), f64(WD), act, store="bf16")
    assert nerr(Z, ref["Z"]) <= TOL["bf16"]
    assert nerr(H, ref["H"]) <= TOL["bf16"]
    assert nerr(P, ref["P"]) <= TOL["bf16"]
    assert done.tolist() == [3] * T          # every destination range published
    dy = si.normal_f32((M, D), 4)
    dY = dev_bf16(dy)
    gu = torch.empty(D, Ft, dtype=torch.bfloat16, device="cuda")
    gd = torch.empty(Ft, D, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    wsb = tpm.alloc_workspace(_abi.OP_MLP_BWD, M, D, F, T, C, _abi.BF16)
    # the backward takes the oracle's forward values as stored in bf16, on both sides
    zb, hb = formats.round_bf16(ref["Z"]), formats.round_bf16(ref["H"])
    tpm.tp_mlp_bwd(X, WU, WD, si.to_bf16(zb).cuda(), si.to_bf16(hb).cuda(), dY, gu, gd, dX, T=T, rank=1, act=act,
                   num_chunks=C, workspace=wsb)
    sync()
    rb = ops.tp_mlp_bwd(f64(X), f64(WU), f64(WD), zb, hb, f64(dY), act, store="bf16")
    assert nerr(gu, rb["dW_up"]) <= TOL["bf16"]
    assert nerr(gd, rb["dW_down"]) <= TOL["bf16"]
    assert nerr(dX, rb["dX"]) <= TOL["bf16"]
    # the workspace holds dZ after the call
    dZ = wsb[2048:2048 + M * Ft * 2].view(torch.bfloat16).view(M, Ft)
    assert nerr(dZ, rb["dZ"]) <= TOL["bf16"]


# --------------------------------------------------------------- gated MLP
ACTS_GATED = [_abi.ACT_SILU, _abi.ACT_GELU_ERF] if torch.cuda.is_available() else []


@pytest.mark.parametrize("act", [0, 1])      # none, ReLU: integer results
def test_gated_gemm_integer_exact(act):
    # EPI_GATED with integer inputs: G and U are exact integers, act(G) * U
    # too, so fp32 outputs equal the oracle bit for bit and bf16 outputs its
    # one rounding.  This pins the pairing of gate and up columns (32-column
    # blocks taken alternately from the two halves of [W_gate | W_up]), the
    # output column of every block and the ragged tails (304 = 256 + 48
    # rows, 136 = 128 + 8 output columns), chunked and unchunked.
    M, K, N = 304, 200, 136
    a = si.small_ints((M, K), 91)
    wg, wu = si.small_ints((K, N), 92), si.small_ints((K, N), 93)
    A, B = dev_bf16(a), dev_bf16(np.concatenate([wg, wu], axis=1))
    g, u = a.astype(np.float64) @ wg, a.astype(np.float64) @ wu
    h = ops.act_fwd(g, act) * u
    for C in (1, 4):
        Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        aux = torch.empty(M, 2 * N, dtype=torch.float32, device="cuda")
        tpm.seq_chunk_gemm(A, B, Y, epilogue=_abi.EPI_GATED, act=act, aux=aux, num_chunks=C,
                           chunk_order=list(range(C))[::-1])
        Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        tpm.seq_chunk_gemm(A, B, Yb, epilogue=_abi.EPI_GATED, act=act, num_chunks=C)
        sync()
        assert np.array_equal(f64(aux[:, :N]), g) and np.array_equal(f64(aux[:, N:]), u)
        assert np.array_equal(f64(Y), h)
        assert np.array_equal(f64(Yb), formats.round_bf16(h))


@pytest.mark.parametrize("act", ACTS_GATED)
def test_gated_gemm_float(act):
    M, K, N = 304, 512, 264
    x = si.normal_f32((M, K), 94)
    wg, wu = si.normal_f32((K, N), 95, 0.05), si.normal_f32((K, N), 96, 0.05)
    X, B = dev_bf16(x), dev_bf16(np.concatenate([wg, wu], axis=1))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    aux = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(X, B, Y, epilogue=_abi.EPI_GATED, act=act, aux=aux)
    sync()
    Bf = f64(B)
    g, u = f64(X) @ Bf[:, :N], f64(X) @ Bf[:, N:]
    assert nerr(aux[:, :N], g) <= TOL["bf16"] and nerr(aux[:, N:], u) <= TOL["bf16"]
    assert nerr(Y, ops.act_fwd(g, act) * u) <= TOL["bf16"]


def test_dgated_epilogue_integer_exact_and_split_k():
    # EPI_DGATED, no activation: dG = dH U and dU = dH G are exact integers.
    # Second shape: 4 output tiles and K = 4096, so the plan splits K and the
    # split-K finalisation runs the same epilogue.
    for (M, N, K, ws) in ((304, 136, 200, False), (512, 264, 4096, True)):
        dy = si.small_ints((M, K), 97)
        wd = si.small_ints((N, K), 98)              # W_down [F/T, D] as stored: op(B) = W_down^T
        gu = si.small_ints((M, 2 * N), 99)
        Y = torch.empty(M, 2 * N, dtype=torch.float32, device="cuda")
        aux = dev_f32(gu)
        w = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K) if ws else None
        if ws:
            assert w.numel() > 2048                  # split-K planned
        tpm.seq_chunk_gemm(dev_bf16(dy), dev_bf16(wd), Y, trans_b=True, epilogue=_abi.EPI_DGATED,
                           act=_abi.ACT_NONE, aux=aux, workspace=w)
        sync()
        dh = dy.astype(np.float64) @ wd.astype(np.float64).T
        assert np.array_equal(f64(Y[:, :N]), dh * gu[:, N:])
        assert np.array_equal(f64(Y[:, N:]), dh * gu[:, :N])


@pytest.mark.parametrize("act", ACTS_GATED)
def test_dgated_epilogue_float(act):
    M, N, K = 512, 264, 4096
    dy = si.normal_f32((M, K), 100)
    wd = si.normal_f32((N, K), 101, 0.02)
    gu = si.normal_f32((M, 2 * N), 102)
    w = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    Y = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    GU = dev_bf16(gu)
    tpm.seq_chunk_gemm(dev_bf16(dy), dev_bf16(wd), Y, trans_b=True, epilogue=_abi.EPI_DGATED, act=act, aux=GU,
                       workspace=w)
    sync()
    dh = f64(dev_bf16(dy)) @ f64(dev_bf16(wd)).T
    g, u = f64(GU)[:, :N], f64(GU)[:, N:]
    assert nerr(Y[:, :N], dh * u * ops.act_grad(g, act)) <= TOL["bf16"]
    assert nerr(Y[:, N:], dh * ops.act_fwd(g, act)) <= TOL["bf16"]


@pytest.mark.parametrize("act", ACTS_GATED)
def test_gated_mlp_fwd_bwd_small(act):
    """The gated MLP share through tp_gated_mlp_fwd / _bwd: 512 tokens,
    D = 256, F = 1024, T = 4, 8 chunks, rank 1.  The backward is fed the
    oracle's forward values rounded to bf16 (the same values on both sides)."""
    M, D, F, T, C, r = 512, 256, 1024, 4, 8, 1
    Ft = F // T
    x = si.normal_f32((M, D), 1)
    wg, wu = si.normal_f32((D, Ft), 2, 0.05), si.normal_f32((D, Ft), 5, 0.05)
    wd = si.normal_f32((Ft, D), 3, 0.05)
    X, WGU, WD = dev_bf16(x), dev_bf16(np.concatenate([wg, wu], axis=1)), dev_bf16(wd)
    Xf, WGUf, WDf = f64(X), f64(WGU), f64(WD)
    GU = torch.empty(M, 2 * Ft, dtype=torch.bfloat16, device="cuda")
    H = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    flags = torch.full((C,), 4, dtype=torch.int32, device="cuda")
    done = torch.zeros(T, dtype=torch.int32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_GATED_MLP_FWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_gated_mlp_fwd(X, WGU, WD, H, P, T=T, rank=r, act=act, GU_t=GU, num_chunks=C,
                         chunk_order=si.ring_chunk_order(T, C, r), chunk_ready=flags, epoch=4, range_done=done,
                         workspace=ws)
    sync()
    assert tpm.poll_device_error(ws) == 0 and done.tolist() == [4] * T
    ref = ops.gated_mlp_fwd(Xf, WGUf[:, :Ft], WGUf[:, Ft:], WDf, act, store="bf16")
    assert nerr(GU[:, :Ft], ref["G"]) <= TOL["bf16"] and nerr(GU[:, Ft:], ref["U"]) <= TOL["bf16"]
    assert nerr(H, ref["H"]) <= TOL["bf16"]
    assert nerr(P, ref["P"]) <= TOL["bf16"]
    # backward on the oracle's stored forward values
    gb, ub, hb = (formats.round_bf16(ref[k]) for k in ("G", "U", "H"))
    GUin, Hin = si.to_bf16(np.concatenate([gb, ub], axis=1)).cuda(), si.to_bf16(hb).cuda()
    dY = dev_bf16(si.normal_f32((M, D), 4))
    dWgu = torch.empty(D, 2 * Ft, dtype=torch.bfloat16, device="cuda")
    dWd = torch.empty(Ft, D, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    wsb = tpm.alloc_workspace(_abi.OP_GATED_MLP_BWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_gated_mlp_bwd(X, WGU, WD, GUin, Hin, dY, dWgu, dWd, dX, T=T, rank=r, act=act, num_chunks=C,
                         dy_chunk_order=si.ring_chunk_order(T, C, r), dy_ready=flags, epoch=4, workspace=wsb)
    sync()
    assert tpm.poll_device_error(wsb) == 0
    rb = ops.gated_mlp_bwd(Xf, WGUf[:, :Ft], WGUf[:, Ft:], WDf, gb, ub, hb, f64(dY), act, store="bf16")
    dGU = wsb[2048:2048 + M * 2 * Ft * 2].view(torch.bfloat16).view(M, 2 * Ft)   # [dG | dU] left in the workspace
    assert nerr(dGU[:, :Ft], rb["dG"]) <= TOL["bf16"] and nerr(dGU[:, Ft:], rb["dU"]) <= TOL["bf16"]
    assert nerr(dWgu[:, :Ft], rb["dW_gate"]) <= TOL["bf16"] and nerr(dWgu[:, Ft:], rb["dW_up"]) <= TOL["bf16"]
    assert nerr(dWd, rb["dW_down"]) <= TOL["bf16"]
    assert nerr(dX, rb["dX"]) <= TOL["bf16"]


# ------------------------------------------------------------------ MXFP8
def _mx_offsets(rows, kblocks):
    """Byte offset of scale (row, kb) in the scaled-MFMA layout, from its
    definition: 32-row groups, one 128-byte record per 4 blocks (128 K
    elements), 4 bytes per row inside a record."""
    r = np.arange(rows)[:, None]
    kb = np.arange(kblocks)[None, :]
    ks = kblocks // 4
    return (((r // 32) * ks + kb // 4) * 32 + r % 32) * 4 + kb % 4


def _mx_dev(codes, e):
    """Device codes + swizzled scales from row-major host arrays."""
    rows, k = codes.shape
    sw = tpm.mx_swizzle_scales(torch.from_numpy(np.ascontiguousarray(e, dtype=np.uint8)).cuda(), k)
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda(), sw


def _mx_unswizzle(sw, rows, k):
    return sw.cpu().numpy()[_mx_offsets(rows, k // 32)]


def test_mx_swizzle_layout():
    rows, k = 70, 384
    e = np.random.default_rng(111).integers(0, 255, size=(rows, k // 32)).astype(np.uint8)
    sw = tpm.mx_swizzle_scales(torch.from_numpy(e).cuda(), k)
    sync()
    assert sw.numel() == tpm.mx_scales_bytes(rows, k) == 96 * (k // 32)
    host = sw.cpu().numpy()
    assert np.array_equal(host[_mx_offsets(rows, k // 32)], e)
    pad = np.ones(host.size, bool)
    pad[_mx_offsets(rows, k // 32).ravel()] = False
    assert np.all(host[pad] == 0)                       # rows 70..95 of the last group


def _mx_int_operand(rows, k, seed):
    """Integer e4m3 codes (|v| <= 3) with block exponents 125..129: every
    product of the GEMM is a multiple of 2^-4 below 2^8, so fp32 sums of a
    few hundred of them are exact."""
    g = np.random.default_rng(seed)
    codes = si.to_e4m3_exact(si.small_ints((rows, k), seed)).numpy()
    e = g.integers(125, 130, size=(rows, k // 32)).astype(np.uint8)
    return codes, e


def test_mx_gemm_integer_exact():
    # pins the scaled MFMA's use of the block scales: which byte, which lane,
    # which operand; ragged rows (300) and columns (136)
    M, N, K = 300, 136, 512
    ac, ae = _mx_int_operand(M, K, 112)
    bc, be = _mx_int_operand(N, K, 113)
    A, As = _mx_dev(ac, ae)
    B, Bs = _mx_dev(bc, be)
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm_mx(A, As, B, Bs, Y)
    sync()
    ref = formats.mx_e4m3_decode(ac, ae) @ formats.mx_e4m3_decode(bc, be).T
    assert np.array_equal(f64(Y), ref)
    # chunked, with a split-K workspace (4 output tiles: the plan splits K)
    M2, N2, K2 = 512, 264, 4096
    ac, ae = _mx_int_operand(M2, K2, 114)
    bc, be = _mx_int_operand(N2, K2, 115)
    A, As = _mx_dev(ac, ae)
    B, Bs = _mx_dev(bc, be)
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M2, N2, K2, 1, 4, _abi.FP8_E4M3)
    assert ws.numel() > 2048
    Y2 = torch.empty(M2, N2, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm_mx(A, As, B, Bs, Y2, num_chunks=4, chunk_order=[3, 1, 0, 2], workspace=ws)
    sync()
    ref2 = formats.mx_e4m3_decode(ac, ae) @ formats.mx_e4m3_decode(bc, be).T
    assert np.array_equal(f64(Y2), ref2)


def test_mx_output_quantisation_exact():
    # no activation, exact fp32 products: the MXFP8 output (codes and block
    # exponents) must equal the oracle's quantisation of the exact values
    M, N, K = 260, 256, 384
    ac, ae = _mx_int_operand(M, K, 116)
    bc, be = _mx_int_operand(N, K, 117)
    A, As = _mx_dev(ac, ae)
    B, Bs = _mx_dev(bc, be)
    Yq = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    Ys = torch.zeros(tpm.mx_scales_bytes(M, N), dtype=torch.uint8, device="cuda")
    Z = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm_mx(A, As, B, Bs, Yq, y_scales=Ys, aux=Z)
    sync()
    z = formats.mx_e4m3_decode(ac, ae) @ formats.mx_e4m3_decode(bc, be).T
    qc, qe = formats.mx_e4m3_quantize(z)
    assert np.array_equal(Yq.cpu().numpy(), qc)
    assert np.array_equal(_mx_unswizzle(Ys, M, N), qe)
    assert np.array_equal(f64(Z), formats.round_bf16(z))


def _mx_float_operand(rows, k, seed, sigma):
    c, e = si.to_mxfp8(si.normal_f32((rows, k), seed, sigma))
    return c.numpy(), e.numpy()


def test_mlp_fwd_mx_small():
    M, D, F, T, C = 512, 512, 2048, 4, 8
    Ft = F // T
    xc, xe = _mx_float_operand(M, D, 1, 1.0)
    uc, ue = _mx_float_operand(Ft, D, 2, 0.02)           # W_up,t stored K-major [F/T, D]
    dc, de = _mx_float_operand(D, Ft, 3, 0.02)           # W_down,t stored K-major [D, F/T]
    X, Xs = _mx_dev(xc, xe)
    WU, WUs = _mx_dev(uc, ue)
    WD, WDs = _mx_dev(dc, de)
    H = torch.empty(M, Ft, dtype=torch.uint8, device="cuda")
    Hs = torch.zeros(tpm.mx_scales_bytes(M, Ft), dtype=torch.uint8, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    flags = torch.full((C,), 6, dtype=torch.int32, device="cuda")
    done = torch.zeros(T, dtype=torch.int32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MX_MLP_FWD, M, D, F, T, C, _abi.FP8_E4M3)
    tpm.tp_mlp_fwd_mx(X, Xs, WU, WUs, WD, WDs, H, Hs, P, T=T, rank=2, act=_abi.ACT_GELU_ERF, Z_t=Z, num_chunks=C,
                      chunk_order=si.ring_chunk_order(T, C, 2), chunk_ready=flags, epoch=6, range_done=done,
                      workspace=ws)
    sync()
    assert tpm.poll_device_error(ws) == 0 and done.tolist() == [6] * T
    ref = ops.tp_mlp_fwd_mx(xc, xe, uc, ue, dc, de, ops.ACT_GELU_ERF)
    assert nerr(Z, ref["Z"]) <= TOL["bf16"]
    hc, he = H.cpu().numpy(), _mx_unswizzle(Hs, M, Ft)
    # block exponents and codes: equal but for values the fp32 evaluation puts
    # on the other side of a rounding (or power-of-two) boundary
    # fp32 evaluation error of H: the accumulation of D products (at most D
    # ulps of their absolute sum) through act', plus the activation's own
    Xd, Ud = formats.mx_e4m3_decode(xc, xe), formats.mx_e4m3_decode(uc, ue)
    dz = D * 2.0 ** -24 * (np.abs(Xd) @ np.abs(Ud).T)
    delta = dz * np.abs(ops.act_grad(ref["Z"], ops.ACT_GELU_ERF)) + 2.0 ** -20 * np.abs(ref["H"]) + 1e-30
    assert_mx_close(hc, he, ref["H"], delta)
    assert nerr(P, ref["P"]) <= TOL["fp8"]


# --------------------------------------------------------------- fp8 backward
@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_cast_fp8_bit_exact(dt):
    # current-scaling cast, row-major and transposed codes: ragged 64x64 tiles
    rows, cols = 96, 160
    x = si.to_bf16(si.normal_f32((rows, cols), 131) * np.float32(7.0))
    X = x.cuda()
    code = _abi.FP8_E5M2 if dt == "e5m2" else _abi.FP8_E4M3
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    tpm.cast_fp8(X, code, q=q, qt=qt, scale_out=sc)
    sync()
    xv = f64(x)
    fmax = np.float32(57344.0 if dt == "e5m2" else 448.0)
    amax = np.float32(np.max(np.abs(xv)))
    inv = np.float32(fmax / amax)
    prod = (xv * float(inv)).astype(np.float32).astype(np.float64)
    want = formats.e5m2_encode(prod) if dt == "e5m2" else formats.e4m3_encode(prod)
    assert np.array_equal(q.cpu().numpy(), want)
    assert np.array_equal(qt.cpu().numpy(), want.T)
    assert sc.item() == float(np.float32(amax / fmax))


@pytest.mark.parametrize("dt", ["e4m3", "e5m2"])
def test_cast_fp8_nan_tiny_and_saturating(dt):
    # the cast's encoder at its edges: NaN elements (either sign; the amax
    # skips them and they encode as 0x7F), magnitudes spread down through the
    # format's subnormals to below half its smallest one (negative ones keep
    # the sign of zero), and values whose scaled product rounds past the
    # largest finite code (saturate)
    rows, cols = 64, 128
    rng = np.random.default_rng(137)
    x = si.to_bf16(si.normal_f32((rows, cols), 138))
    xi = x.view(torch.int16)
    top = 6.5   # fp32(top * fp32(fmax / top)) > fmax for both formats
    xi[0, :] = torch.from_numpy(formats.round_bf16(np.full(cols, top)).astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    k = np.arange(cols)
    tiny = np.where(k % 2 == 0, 1.0, -1.0) * top * 2.0 ** -(1 + k % 40) * (1.0 + (k % 7) / 8.0)
    xi[1, :] = torch.from_numpy(formats.round_bf16(tiny).astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    nan_pos = rng.choice(rows * cols - 2 * cols, size=9, replace=False) + 2 * cols
    for j, pos in enumerate(nan_pos):
        xi[pos // cols, pos % cols] = 0x7FC0 if j % 2 == 0 else -0x40   # +NaN / -NaN bf16
    X = x.cuda()
    code = _abi.FP8_E5M2 if dt == "e5m2" else _abi.FP8_E4M3
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    qt = torch.empty(cols, rows, dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    tpm.cast_fp8(X, code, q=q, qt=qt, scale_out=sc)
    sync()
    xv = f64(x)
    assert np.isnan(xv).sum() == 9
    fmax = np.float32(57344.0 if dt == "e5m2" else 448.0)
    amax = np.float32(np.nanmax(np.abs(xv)))
    assert amax == np.float32(top)
    inv = np.float32(fmax / amax)
    prod = (xv * float(inv)).astype(np.float32).astype(np.float64)
    assert np.all(prod[0] > fmax)
    want = formats.e5m2_encode(prod) if dt == "e5m2" else formats.e4m3_encode(prod)
    got = q.cpu().numpy()
    assert np.all(got[np.isnan(xv)] == 0x7F)
    assert np.array_equal(got, want)
    assert np.array_equal(qt.cpu().numpy(), want.T)
    assert sc.item() == float(np.float32(amax / fmax))


@pytest.mark.parametrize("strided", [False, True])
def test_cast_fp8_amax_many_rows_ragged_columns(strided):
    # more rows than the amax kernel's grid and a row of 258 16-byte groups
    # (the last load batch of a row only partly valid), on a contiguous matrix
    # (flat walk) and on a column slice of a wider one (row walk; the larger
    # values beyond the slice must not count); the largest magnitude sits in
    # the tail of a late row
    rows, cols = 4112, 2064
    x = si.to_bf16(si.normal_f32((rows, cols), 139))
    x[4100, 2063] = -9.75
    if strided:
        big = torch.full((rows, cols + 48), 100.0, dtype=torch.bfloat16)
        big[:, :cols] = x
        X = big.cuda()[:, :cols]
        assert X.stride() == (cols + 48, 1)
    else:
        X = x.cuda()
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    tpm.cast_fp8(X, _abi.FP8_E4M3, q=q, scale_out=sc)
    sync()
    xv = f64(x)
    amax = np.float32(np.max(np.abs(xv)))
    assert amax == np.float32(9.75)
    assert sc.item() == float(np.float32(amax / np.float32(448.0)))
    inv = np.float32(np.float32(448.0) / amax)
    want = formats.e4m3_encode((xv * float(inv)).astype(np.float32).astype(np.float64))
    assert np.array_equal(q.cpu().numpy(), want)


def test_fp8_mixed_format_gemm_integer_exact():
    # e5m2 x e4m3 and e4m3 x e5m2 through seq_chunk_gemm: integers in [-3, 3]
    # are exact in both formats, so the fp32 products are exact
    M, N, K = 200, 136, 512
    a, b = si.small_ints((M, K), 132), si.small_ints((N, K), 133)
    ref = a.astype(np.float64) @ b.astype(np.float64).T
    e5 = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e5m2).cuda()
    e4 = lambda v: torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn).cuda()
    for A, B in ((e5(a), e4(b)), (e4(a), e5(b))):
        Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
        tpm.seq_chunk_gemm(A, B, Y, trans_b=True)
        sync()
        assert np.array_equal(f64(Y), ref)


@pytest.mark.parametrize("M,D,F", [(512, 512, 2048), (528, 272, 320)])
def test_mlp_bwd_fp8_small(M, D, F):
    # the second shape leaves ragged 64 x 64 tiles in the casts and transposes
    # and ragged K in every GEMM
    T = 4
    Ft = F // T
    xq, sx = si.to_e4m3_current(si.normal_f32((M, D), 1))
    wuq, su = si.to_e4m3_current(si.normal_f32((D, Ft), 2, 0.02))      # the pages' layouts
    wdq, sd = si.to_e4m3_current(si.normal_f32((Ft, D), 3, 0.02))
    z = si.to_bf16(si.normal_f32((M, Ft), 134))
    h = si.to_bf16(np.abs(si.normal_f32((M, Ft), 135)))
    dy = si.to_bf16(si.normal_f32((M, D), 136))
    scales = dev_f32(np.array([sx, su, sd], np.float32))
    dWu = torch.empty(D, Ft, dtype=torch.bfloat16, device="cuda")
    dWd = torch.empty(Ft, D, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MLP_BWD_FP8, M, D, F, T, 1, _abi.FP8_E4M3)
    tpm.tp_mlp_bwd_fp8(xq.cuda(), wuq.cuda(), wdq.cuda(), z.cuda(), h.cuda(), dy.cuda(), dWu, dWd, dX, T=T, rank=0,
                       scales=scales, act=_abi.ACT_GELU_ERF, workspace=ws)
    sync()
    # the oracle's H codes: the forward's current-scaling cast of the same bf16 H
    hv = f64(h)
    amax_h = np.float32(np.max(np.abs(hv)))
    h8 = formats.e4m3_to_f64(formats.e4m3_encode((hv * float(np.float32(np.float32(448) / amax_h))).astype(np.float32)))
    sh = float(np.float32(amax_h / np.float32(448)))
    r = ops.tp_mlp_bwd_fp8(f64(xq), sx, f64(wuq), su, f64(wdq), sd, f64(z), h8, sh, f64(dy), ops.ACT_GELU_ERF)
    # dY's e5m2 codes are bit-exact (the same fp32 arithmetic on the same bf16 values)
    dy8 = ws[2048:2048 + M * D].cpu().numpy().reshape(M, D)
    assert np.array_equal(formats.e5m2_to_f64(dy8), r["dYq"])
    # the transposed copies of dY's and X's codes are exact transposes
    md = (M * D + 255) // 256 * 256
    dy8t = ws[2048 + md:2048 + md + M * D].cpu().numpy().reshape(D, M)
    assert np.array_equal(dy8t, dy8.T)
    x8t = ws[2048 + 2 * md:2048 + 2 * md + M * D].cpu().numpy().reshape(D, M)
    assert np.array_equal(x8t, xq.view(torch.uint8).numpy().T)
    off = 2048 + 3 * ((M * D + 255) // 256 * 256)
    mf = (M * Ft + 255) // 256 * 256
    dz = ws[off:off + 2 * M * Ft].view(torch.bfloat16).view(M, Ft)
    assert nerr(dz, r["dZ"]) <= TOL["bf16"]
    assert nerr(dWd, r["dW_down"]) <= TOL["fp8"]
    # the later GEMMs read the dZ the GPU stored: the oracle continues from it
    r2 = ops.tp_mlp_bwd_fp8(f64(xq), sx, f64(wuq), su, f64(wdq), sd, f64(z), h8, sh, f64(dy), ops.ACT_GELU_ERF,
                            dz_stored=f64(dz))
    dz8 = ws[off + 2 * mf:off + 2 * mf + M * Ft].cpu().numpy().reshape(M, Ft)
    assert np.array_equal(formats.e5m2_to_f64(dz8), r2["dZq"])          # same fp32 arithmetic on the same bf16
    assert nerr(dWu, r2["dW_up"]) <= TOL["fp8"]
    assert nerr(dX, r2["dX"]) <= TOL["fp8"]
    # the stored dZ differs from the oracle's own bf16 rounding of the exact
    # value by one ulp in about 1 % of the elements (fp32 accumulation and
    # GeLU' evaluated in fp32): the reason the later products are checked
    # on the GPU's own dZ
    assert np.mean(f64(dz) != r["dZ"]) < 2e-2


def test_mlp_bwd_fp8_chunk_fed_e5m2_dy_matches_resident():
    """dY arriving as e5m2 codes in chunks (quantised by its producers with
    one current scale, as an all-gather of quantised gradients delivers it),
    written by the side-stream writer on its own CUs while the dZ GEMM waits
    per chunk: every output bitwise equal to the call that casts a resident
    bf16 dY itself (the same codes and scale)."""
    M, D, F, T, C = 1024, 512, 2048, 4, 8
    Ft = F // T
    xq, sx = si.to_e4m3_current(si.normal_f32((M, D), 1))
    wuq, su = si.to_e4m3_current(si.normal_f32((D, Ft), 2, 0.02))
    wdq, sd = si.to_e4m3_current(si.normal_f32((Ft, D), 3, 0.02))
    z = si.to_bf16(si.normal_f32((M, Ft), 137)).cuda()
    h = si.to_bf16(np.abs(si.normal_f32((M, Ft), 138))).cuda()
    dy = si.to_bf16(si.normal_f32((M, D), 139)).cuda()
    X, WU, WD = xq.cuda(), wuq.cuda(), wdq.cuda()
    scales = dev_f32(np.array([sx, su, sd], np.float32))
    e = lambda *sh: torch.empty(*sh, dtype=torch.bfloat16, device="cuda")
    outs = []
    ws = tpm.alloc_workspace(_abi.OP_MLP_BWD_FP8, M, D, F, T, C, _abi.FP8_E4M3)
    ref = (e(D, Ft), e(Ft, D), e(M, D))
    tpm.tp_mlp_bwd_fp8(X, WU, WD, z, h, dy, *ref, T=T, rank=0, scales=scales, act=_abi.ACT_GELU_ERF, workspace=ws)
    # the producers' quantised dY: the same current-scaling cast
    dy8 = torch.empty(M, D, dtype=torch.uint8, device="cuda")
    s_dy = torch.empty(1, dtype=torch.float32, device="cuda")
    tpm.cast_fp8(dy, _abi.FP8_E5M2, q=dy8, scale_out=s_dy)
    sync()
    streams = tpm.masked_streams(producer_cus=8)
    compute, producer = streams
    landing = torch.zeros_like(dy8)
    ready = torch.zeros(C, dtype=torch.int32, device="cuda")
    counters = torch.zeros(C, dtype=torch.int32, device="cuda")
    order = si.ring_chunk_order(T, C, 1)
    ws2 = tpm.alloc_workspace(_abi.OP_MLP_BWD_FP8, M, D, F, T, C, _abi.FP8_E4M3)
    for epoch in (1, 2):
        got = (e(D, Ft), e(Ft, D), e(M, D))
        sync()
        tpm.tp_mlp_bwd_fp8(X, WU, WD, z, h, landing, *got, T=T, rank=1, scales=scales, act=_abi.ACT_GELU_ERF,
                           dy_scale=s_dy, num_chunks=C, dy_chunk_order=order, dy_ready=ready, epoch=epoch,
                           workspace=ws2, stream=compute)
        tpm.write_chunks(landing, dy8, C, order, ready, epoch, counters, stream=producer)
        sync()
        assert tpm.poll_device_error(ws2) == 0
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        landing.zero_()
    sync()
    streams.close()


# -------------------------------------------------------- fp8 delayed scaling
@pytest.mark.parametrize("M, D, F", [(256, 64, 512),
                                     # 17 x 16 tiles for GEMM1 (the last tile column
                                     # in 2 K pieces, finalised to e4m3), split-K GEMM2
                                     (4352, 2048, 8192)])
def test_mlp_fwd_fp8_delayed_integer_exact(M, D, F):
    # integer operands, ReLU: H is exact, H * fp32(1 / s_H) exact for s_H =
    # 1/16, so the e4m3 codes (saturating above 448) and the amax are bit-exact
    T = 2
    Ft = F // T
    x, wu, wd = si.small_ints((M, D), 121), si.small_ints((D, Ft), 122), si.small_ints((Ft, D), 123)
    X = si.to_e4m3_exact(x).cuda()
    WU = si.to_e4m3_exact(np.ascontiguousarray(wu.T)).cuda()        # K-major [Ft, D]
    WD = si.to_e4m3_exact(np.ascontiguousarray(wd.T)).cuda()        # K-major [D, Ft]
    scales = dev_f32(np.array([1.0, 1.0, 1.0], np.float32))
    hs = dev_f32(np.array([0.0625], np.float32))
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    H = torch.empty(M, Ft, dtype=torch.uint8, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_FP8_DELAYED_MLP_FWD, M, D, F, T, 1, _abi.FP8_E4M3)
    tpm.tp_mlp_fwd_delayed(X, WU, WD, H, P, T=T, rank=0, scales=scales, h_scale=hs, h_amax_out=amax,
                           act=_abi.ACT_RELU, workspace=ws)
    sync()
    ref = ops.tp_mlp_fwd_fp8_delayed(x.astype(np.float64), 1.0, wu.astype(np.float64), 1.0, wd.astype(np.float64),
                                     1.0, 0.0625, ops.ACT_RELU)
    assert np.any(np.abs(ref["H"]) * 16 > 464)                  # some codes saturate
    assert np.array_equal(H.cpu().numpy(), ref["Hq_codes"])
    assert amax.item() == ref["amax"]
    assert nerr(P, ref["P"]) <= TOL["bf16"]


def test_mlp_fwd_fp8_delayed_steps():
    """Two steps of delayed scaling on float inputs: step 1 with the initial
    scale 1, then the scale from the amax history (the oracle's, given to
    both sides); the library's scale update of the history is checked
    against the same rule."""
    M, D, F, T, C = 512, 512, 2048, 4, 8
    Ft = F // T
    x = si.normal_f32((M, D), 1)
    wu = si.normal_f32((D, Ft), 2, 0.02)
    wd = si.normal_f32((Ft, D), 3, 0.02)
    xq, sx = si.to_e4m3_current(x)
    wuq, su = si.to_e4m3_current(np.ascontiguousarray(wu.T))
    wdq, sd = si.to_e4m3_current(np.ascontiguousarray(wd.T))
    X, WU, WD = xq.cuda(), wuq.cuda(), wdq.cuda()
    scales = dev_f32(np.array([sx, su, sd], np.float32))
    hist = torch.zeros(4, dtype=torch.float32, device="cuda")
    H = torch.empty(M, Ft, dtype=torch.uint8, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    flags = torch.full((C,), 2, dtype=torch.int32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_FP8_DELAYED_MLP_FWD, M, D, F, T, C, _abi.FP8_E4M3)
    xd, wud, wdd = f64(xq), f64(wuq).T, f64(wdq).T
    s_h = 1.0
    for step in range(2):
        hs = dev_f32(np.array([s_h], np.float32))
        tpm.tp_mlp_fwd_delayed(X, WU, WD, H, P, T=T, rank=1, scales=scales, h_scale=hs, h_amax_out=hist[step:step + 1],
                               act=_abi.ACT_GELU_ERF, num_chunks=C, chunk_ready=flags, epoch=2, workspace=ws)
        sync()
        assert tpm.poll_device_error(ws) == 0
        ref = ops.tp_mlp_fwd_fp8_delayed(xd, sx, wud, su, wdd, sd, s_h, ops.ACT_GELU_ERF)
        hc = H.cpu().numpy().astype(int)
        rc = ref["Hq_codes"].astype(int)
        diff = hc != rc
        assert np.mean(diff) < 1e-2
        # a differing code is a neighbour (fp32 vs fp64 evaluation across a rounding boundary)
        assert np.all(((hc[diff] & 0x80) == (rc[diff] & 0x80)) & (np.abs((hc[diff] & 0x7F) - (rc[diff] & 0x7F)) == 1)
                      | (((hc[diff] & 0x7F) <= 1) & ((rc[diff] & 0x7F) <= 1)))
        assert abs(hist[step].item() - ref["amax"]) <= 1e-5 * ref["amax"]
        assert nerr(P, ref["P"]) <= TOL["fp8"]
        s_next = ops.fp8_delayed_scale([ref["amax"]] + ([] if step == 0 else [amax_prev]))
        amax_prev = ref["amax"]
        out = torch.empty(1, dtype=torch.float32, device="cuda")
        tpm.fp8_delayed_scale(hist, out)
        sync()
        # the update is fp32(max(history) / 448) of the history it read, and
        # that history holds amaxes within fp32 evaluation error of the oracle's
        h32 = hist.cpu().numpy()
        assert out.item() == float(np.float32(np.max(h32) / np.float32(448.0)))
        assert abs(out.item() - s_next) <= 1e-5 * s_next
        s_h = s_next


def test_mlp_fwd_fp8_small():
    M, D, F, T, C = 512, 512, 2048, 4, 8
    Ft = F // T
    x = si.normal_f32((M, D), 1)
    wu = si.normal_f32((D, Ft), 2, 0.02)
    wd = si.normal_f32((Ft, D), 3, 0.02)
    xq, sx = si.to_e4m3_current(x)
    wuq, su = si.to_e4m3_current(np.ascontiguousarray(wu.T))   # K-major copies of the weights
    wdq, sd = si.to_e4m3_current(np.ascontiguousarray(wd.T))
    scales = dev_f32(np.array([sx, su, sd], dtype=np.float32))
    H = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    sH = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, C, _abi.FP8_E4M3)
    tpm.tp_mlp_fwd(xq.cuda(), wuq.cuda(), wdq.cuda(), H, P, T=T, rank=0, act=_abi.ACT_GELU_ERF, scales=scales,
                   h_scale_out=sH, num_chunks=C, workspace=ws)
    sync()
    r = ops.tp_mlp_fwd_fp8(f64(xq), sx, f64(wuq).T, su, f64(wdq).T, sd, ops.ACT_GELU_ERF)
    assert nerr(H, r["H"]) <= TOL["bf16"]                 # H is stored in bf16
    assert nerr(P, r["P"]) <= TOL["fp8"]
    hq = ws[2048:2048 + M * Ft].cpu().numpy().reshape(M, Ft)
    _util.assert_fp8_h_consistent(f64(H), hq, sH.item(), r)


# --------------------------------------------- chunk arrival on a side stream
def test_chunks_arrive_from_side_stream():
    M, N, K, C = 2048, 1024, 512, 8
    x = si.normal_f32((M, K), 61)
    w = si.normal_f32((K, N), 62, 0.05)
    Xsrc, W = dev_bf16(x), dev_bf16(w)
    ref = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, num_chunks=C)
    # same workspace, hence the same split-K plan: the gated result must be bitwise equal
    tpm.seq_chunk_gemm(Xsrc, W, ref, act=_abi.ACT_GELU_ERF, num_chunks=C, workspace=ws)
    sync()
    Xdst = torch.zeros_like(Xsrc)
    flags = torch.zeros(C, dtype=torch.int32, device="cuda")
    Y = torch.empty_like(ref)
    order = si.ring_chunk_order(4, C, 2)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    rows = M // C
    epoch = 1
    tpm.seq_chunk_gemm(Xdst, W, Y, act=_abi.ACT_GELU_ERF, num_chunks=C, chunk_order=order, chunk_ready=flags,
                       epoch=epoch, workspace=ws, stream=main)
    with torch.cuda.stream(side):
        for c in order:
            Xdst[c * rows:(c + 1) * rows].copy_(Xsrc[c * rows:(c + 1) * rows])
            tpm.signal_chunk(flags, c, epoch, stream=side)
    sync()
    assert tpm.poll_device_error(ws) == 0
    assert torch.equal(Y, ref)


def test_chunks_arrive_on_cu_masked_streams_full_chip():
    # enough tiles for one waiting work-group on every CU of the compute
    # stream; the producer's copy and signal kernels run on CUs of their own
    M, N, K, C = 4096, 4096, 1024, 8
    x = si.normal_f32((M, K), 63)
    w = si.normal_f32((K, N), 64, 0.05)
    Xsrc, W = dev_bf16(x), dev_bf16(w)
    ref = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, num_chunks=C)
    tpm.seq_chunk_gemm(Xsrc, W, ref, act=_abi.ACT_RELU, num_chunks=C, workspace=ws)
    sync()
    compute, producer = tpm.masked_streams(producer_cus=8)
    Xdst = torch.zeros_like(Xsrc)
    flags = torch.zeros(C, dtype=torch.int32, device="cuda")
    Y = torch.empty_like(ref)
    order = si.ring_chunk_order(8, C, 3)
    rows = M // C
    sync()
    for epoch in (1, 2):
        tpm.seq_chunk_gemm(Xdst, W, Y, act=_abi.ACT_RELU, num_chunks=C, chunk_order=order, chunk_ready=flags,
                           epoch=epoch, workspace=ws, stream=compute)
        with torch.cuda.stream(producer):
            for c in order:
                Xdst[c * rows:(c + 1) * rows].copy_(Xsrc[c * rows:(c + 1) * rows])
                tpm.signal_chunk(flags, c, epoch, stream=producer)
        sync()
        assert tpm.poll_device_error(ws) == 0
        assert torch.equal(Y, ref)
        Xdst.zero_()
        sync()


@pytest.mark.parametrize("masked", [False, True])
def test_write_chunks_copies_in_order_and_flags(masked):
    C, rows, cols = 8, 97, 1000          # 194000-byte chunks: 12125 vectors, a ragged share per work-group
    g = torch.Generator().manual_seed(5)
    src = torch.randint(-2**31, 2**31 - 1, (C * rows, cols // 2), generator=g, dtype=torch.int32).cuda()
    dst = torch.zeros_like(src)
    keep = torch.randint(-5, 5, (rows, cols // 2), generator=g, dtype=torch.int32).cuda()
    dst[3 * rows:4 * rows] = keep                         # chunk 3 is already in place: not copied
    ready = torch.zeros(C, dtype=torch.int32, device="cuda")
    counters = torch.zeros(C, dtype=torch.int32, device="cuda")
    order = si.ring_chunk_order(4, C, 1)
    copy = [c != 3 for c in range(C)]
    stream = tpm.masked_streams(producer_cus=8)[1] if masked else torch.cuda.current_stream()
    sync()
    for epoch in (7, 8):
        tpm.write_chunks(dst, src, C, order, ready, epoch, counters, copy=copy, stream=stream)
        sync()
        for c in range(C):
            want = keep if c == 3 else src[c * rows:(c + 1) * rows]
            assert torch.equal(dst[c * rows:(c + 1) * rows], want), c
        assert torch.all(ready == epoch)
        assert torch.count_nonzero(counters).item() == 0


def test_write_chunks_feeds_gated_gemm_full_chip():
    M, N, K, C = 4096, 4096, 1024, 8
    Xsrc = dev_bf16(si.normal_f32((M, K), 65))
    W = dev_bf16(si.normal_f32((K, N), 66, 0.05))
    ref = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, num_chunks=C)
    tpm.seq_chunk_gemm(Xsrc, W, ref, act=_abi.ACT_GELU_TANH, num_chunks=C, workspace=ws)
    compute, producer = tpm.masked_streams(producer_cus=8)
    X = torch.zeros_like(Xsrc)
    ready = torch.zeros(C, dtype=torch.int32, device="cuda")
    counters = torch.zeros(C, dtype=torch.int32, device="cuda")
    Y = torch.empty_like(ref)
    order = si.ring_chunk_order(8, C, 5)
    sync()
    for epoch in (1, 2):
        tpm.seq_chunk_gemm(X, W, Y, act=_abi.ACT_GELU_TANH, num_chunks=C, chunk_order=order, chunk_ready=ready,
                           epoch=epoch, workspace=ws, stream=compute)
        tpm.write_chunks(X, Xsrc, C, order, ready, epoch, counters, stream=producer)
        sync()
        assert tpm.poll_device_error(ws) == 0
        assert torch.equal(Y, ref)
        X.zero_()
        sync()


def test_watchdog_reports_timeout_and_kernel_exits():
    M, N, K, C = 512, 256, 128, 2
    X = dev_bf16(si.normal_f32((M, K), 71))
    W = dev_bf16(si.normal_f32((K, N), 72))
    flags = torch.zeros(C, dtype=torch.int32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.set_wait_limit(2000)
    try:
        # chunk 1 is never signalled; chunk 0 is
        tpm.signal_chunk(flags, 0, 5)
        tpm.seq_chunk_gemm(X, W, Y, num_chunks=C, chunk_ready=flags, epoch=5, workspace=ws)
        sync()
        assert tpm.poll_device_error(ws) == _abi.ETIMEOUT
    finally:
        tpm.set_wait_limit(1 << 22)
    # the next gated call clears the error word
    flags.fill_(5)
    tpm.seq_chunk_gemm(X, W, Y, num_chunks=C, chunk_ready=flags, epoch=5, workspace=ws)
    sync()
    assert tpm.poll_device_error(ws) == 0


# ------------------------------------------------------------ split-K path
def test_split_k_narrow_gemm():
    # 2 output tiles, K = 4096: the plan cuts K into pieces whose fp32 partial
    # sums a second kernel adds in a fixed order
    M, N, K = 512, 264, 4096
    assert tpm.workspace_bytes(_abi.OP_SEQ_CHUNK_GEMM, M, N, K) > 2048      # split planned
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    a = si.small_ints((M, K), 81)
    b = si.small_ints((K, N), 82)
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(dev_bf16(a), dev_bf16(b), Y, workspace=ws)
    sync()
    assert np.array_equal(f64(Y), a.astype(np.float64) @ b.astype(np.float64))   # exact
    # float inputs, GeLU + Z save, chunk-gated (flags already set), amax
    x = dev_bf16(si.normal_f32((M, K), 83))
    w = dev_bf16(si.normal_f32((K, N), 84, 0.02))
    Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty_like(Yb)
    flags = torch.full((4,), 9, dtype=torch.int32, device="cuda")
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(x, w, Yb, act=_abi.ACT_GELU_ERF, aux=Z, num_chunks=4, chunk_order=[2, 0, 3, 1],
                       chunk_ready=flags, epoch=9, amax_out=amax, workspace=ws)
    sync()
    y, z = ops.seq_chunk_gemm(f64(x), f64(w), act=_abi.ACT_GELU_ERF)
    assert nerr(Yb, y) <= TOL["bf16"] and nerr(Z, z) <= TOL["bf16"]
    assert amax.item() == float(np.max(np.abs(f64(Yb))))
    assert tpm.poll_device_error(ws) == 0
    # DACT epilogue through the split path, K-major B
    wt = dev_bf16(si.normal_f32((N, K), 85, 0.02))
    zin = dev_bf16(si.normal_f32((M, N), 86))
    Yd = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(x, wt, Yd, trans_b=True, epilogue=_abi.EPI_DACT, act=_abi.ACT_GELU_ERF, aux=zin,
                       workspace=ws)
    sync()
    yd, _ = ops.seq_chunk_gemm(f64(x), f64(wt), trans_b=True, act=_abi.ACT_GELU_ERF, dact_z=f64(zin))
    assert nerr(Yd, yd) <= TOL["bf16"]


def test_split_k_sum_is_deterministic():
    # The fp32 partial sums of the K splits are added in ascending split
    # order, so repeated calls agree bit for bit; an ungated call does not
    # read the control words at the head of the workspace (filled here with
    # a byte pattern first).
    M, N, K = 1000, 520, 8192             # ragged row and column tiles, 8 splits
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    assert ws.numel() > 2048
    ws[:2048].fill_(0x13)
    x = dev_bf16(si.normal_f32((M, K), 87))
    w = dev_bf16(si.normal_f32((K, N), 88, 0.02))
    outs = []
    for _ in range(3):
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        tpm.seq_chunk_gemm(x, w, Y, act=_abi.ACT_GELU_TANH, workspace=ws)
        sync()
        outs.append(Y.clone())
    y, _ = ops.seq_chunk_gemm(f64(x), f64(w), act=_abi.ACT_GELU_TANH)
    assert nerr(outs[0], y) <= TOL["bf16"]
    assert all(torch.equal(o, outs[0]) for o in outs[1:])


def test_tail_split_bf16():
    # 17 x 16 = 272 output tiles: the whole tiles of the first 15 tile
    # columns fill one round; the last (ragged) column's 17 tiles, the ragged
    # last row tile among them, are cut into 2 K ranges whose fp32 partials a
    # second kernel sums in piece order before the epilogue
    M, N, K = 4312, 4072, 1024
    piece = 256 * 256 * 4
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    assert ws.numel() == 2048 + 17 * 2 * piece
    a = si.small_ints((M, K), 91)
    b = si.small_ints((K, N), 92)
    A, B = dev_bf16(a), dev_bf16(b)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Y0 = torch.empty_like(Y)
    tpm.seq_chunk_gemm(A, B, Y, workspace=ws)
    tpm.seq_chunk_gemm(A, B, Y0)                     # no scratch: whole tiles only
    sync()
    assert np.array_equal(f64(Y), exact) and np.array_equal(f64(Y0), exact)
    # float inputs: GeLU + Z save + amax through the finalisation, repeatable
    x = dev_bf16(si.normal_f32((M, K), 93))
    w = dev_bf16(si.normal_f32((K, N), 94, 0.02))
    outs = []
    for _ in range(2):
        Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        Z = torch.empty_like(Yb)
        amax = torch.empty(1, dtype=torch.float32, device="cuda")
        tpm.seq_chunk_gemm(x, w, Yb, act=_abi.ACT_GELU_ERF, aux=Z, amax_out=amax, workspace=ws)
        sync()
        outs.append((Yb, Z, amax))
    y, z = ops.seq_chunk_gemm(f64(x), f64(w), act=_abi.ACT_GELU_ERF)
    Yb, Z, amax = outs[0]
    assert nerr(Yb, y) <= TOL["bf16"] and nerr(Z, z) <= TOL["bf16"]
    assert amax.item() == float(np.max(np.abs(f64(Yb))))
    assert torch.equal(outs[1][0], Yb) and torch.equal(outs[1][1], Z) and torch.equal(outs[1][2], amax)
    # DACT epilogue through the tail path, K-major B
    wt = dev_bf16(si.normal_f32((N, K), 95, 0.02))
    zin = dev_bf16(si.normal_f32((M, N), 96))
    Yd = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(x, wt, Yd, trans_b=True, epilogue=_abi.EPI_DACT, act=_abi.ACT_GELU_ERF, aux=zin,
                       workspace=ws)
    sync()
    yd, _ = ops.seq_chunk_gemm(f64(x), f64(wt), trans_b=True, act=_abi.ACT_GELU_ERF, dact_z=f64(zin))
    assert nerr(Yd, yd) <= TOL["bf16"]


def test_tail_split_bits_independent_of_chunking():
    # The tail split cuts the last tile column whatever the chunking, so a
    # chunk-gated call (2 chunks of 2156 rows fed in the order [1, 0], flags
    # already set, one CU per XCD left to a producer), the same call
    # resident, and an unchunked call give the same bits.
    M, N, K = 4312, 4072, 1024
    ws2 = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, num_chunks=2)
    ws1 = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    assert ws2.numel() == 2048 + 18 * 2 * 256 * 256 * 4     # 9 row tiles per chunk
    x = dev_bf16(si.normal_f32((M, K), 97))
    w = dev_bf16(si.normal_f32((K, N), 98, 0.02))
    flags = torch.full((2,), 5, dtype=torch.int32, device="cuda")
    Yg = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Yr, Y1 = torch.empty_like(Yg), torch.empty_like(Yg)
    tpm.seq_chunk_gemm(x, w, Yg, act=_abi.ACT_RELU, num_chunks=2, chunk_order=[1, 0], chunk_ready=flags,
                       epoch=5, workspace=ws2)
    sync()
    assert tpm.poll_device_error(ws2) == 0
    tpm.seq_chunk_gemm(x, w, Yr, act=_abi.ACT_RELU, num_chunks=2, chunk_order=[1, 0], workspace=ws2)
    tpm.seq_chunk_gemm(x, w, Y1, act=_abi.ACT_RELU, workspace=ws1)
    sync()
    assert torch.equal(Yg, Yr) and torch.equal(Yr, Y1)
    y, _ = ops.seq_chunk_gemm(f64(x), f64(w), act=_abi.ACT_RELU)
    assert nerr(Yr, y) <= TOL["bf16"]


def test_tail_split_fp8():
    # e4m3, K = 2048 (16 steps of 128): 17 x 16 tiles, the last column's 17
    # cut in 2
    M, N, K = 4352, 4096, 2048
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, dtype=_abi.FP8_E4M3)
    assert ws.numel() == 2048 + 17 * 2 * 256 * 256 * 4
    a = si.small_ints((M, K), 99, -4, 4)
    bt = si.small_ints((N, K), 100, -4, 4)
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(si.to_e4m3_exact(a).cuda(), si.to_e4m3_exact(bt).cuda(), Y, trans_b=True, workspace=ws)
    sync()
    assert np.array_equal(f64(Y), a.astype(np.float64) @ bt.astype(np.float64).T)
    x = si.normal_f32((M, K), 101)
    wv = si.normal_f32((N, K), 102, 0.02)
    xq, sx = si.to_e4m3_current(x)
    wq, sw = si.to_e4m3_current(wv)
    scales = dev_f32(np.array([sx, sw], dtype=np.float32))
    Yb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty_like(Yb)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(xq.cuda(), wq.cuda(), Yb, trans_b=True, a_scale=scales[0:1], b_scale=scales[1:2],
                       act=_abi.ACT_GELU_ERF, aux=Z, amax_out=amax, workspace=ws)
    sync()
    y, z = ops.seq_chunk_gemm(f64(xq), f64(wq), trans_b=True, a_scale=sx, b_scale=sw, act=_abi.ACT_GELU_ERF)
    assert nerr(Yb, y) <= TOL["fp8"] and nerr(Z, z) <= TOL["fp8"]
    assert amax.item() == float(np.max(np.abs(f64(Yb))))


def test_chunk_gating_reads_fresh_data_after_stale_reads():
    # The consumer GEMM first reads X while it holds zeros (so caches may hold
    # those lines), then the chunks are rewritten with real data on a side
    # stream while the gated GEMM waits: the result must use the new data.
    M, N, K, C = 2048, 512, 1024, 8
    Xsrc = dev_bf16(si.normal_f32((M, K), 91))
    W = dev_bf16(si.normal_f32((K, N), 92, 0.05))
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, num_chunks=C)
    ref = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(Xsrc, W, ref, num_chunks=C, workspace=ws)
    X = torch.zeros_like(Xsrc)
    Y0 = torch.empty_like(ref)
    tpm.seq_chunk_gemm(X, W, Y0, num_chunks=C, workspace=ws)      # caches see zeros
    sync()
    assert torch.count_nonzero(Y0).item() == 0
    flags = torch.zeros(C, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    rows = M // C
    Y = torch.empty_like(ref)
    ev = torch.cuda.Event()
    ev.record()
    tpm.seq_chunk_gemm(X, W, Y, num_chunks=C, chunk_order=list(range(C)), chunk_ready=flags, epoch=3,
                       workspace=ws)
    side.wait_event(ev)
    with torch.cuda.stream(side):
        for c in range(C):
            X[c * rows:(c + 1) * rows].copy_(Xsrc[c * rows:(c + 1) * rows])
            tpm.signal_chunk(flags, c, 3, stream=side)
    sync()
    assert tpm.poll_device_error(ws) == 0
    assert torch.equal(Y, ref)


# ------------------------------------------------ HIP graph capture / replay
def test_graph_replays_match_eager():
    # bf16 MLP forward, an fp8 forward (control-word init, amax, quantiser),
    # a split-K GEMM (fp32 partials + finalisation), a reduction and a paired
    # linear backward (ticket counters zeroed by a kernel), captured
    # once and replayed three times with eager work and synchronisation in
    # between; every replay must equal the eager result bit for bit
    M, D, F, T = 512, 512, 2048, 4
    Ft = F // T
    X = dev_bf16(si.normal_f32((M, D), 111))
    Wu = dev_bf16(si.normal_f32((D, Ft), 112, 0.05))
    Wd = dev_bf16(si.normal_f32((Ft, D), 113, 0.05))
    H = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    stack = dev_bf16(si.normal_f32((T, M, D), 114))
    out = torch.empty(M // T, D, dtype=torch.bfloat16, device="cuda")
    ws_f = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, 4, _abi.BF16)
    xq, sx = si.to_e4m3_current(si.normal_f32((M, D), 115))
    wuq, su = si.to_e4m3_current(si.normal_f32((Ft, D), 116, 0.05))
    wdq, sd = si.to_e4m3_current(si.normal_f32((D, Ft), 117, 0.05))
    xq, wuq, wdq = xq.cuda(), wuq.cuda(), wdq.cuda()
    scales = dev_f32(np.array([sx, su, sd], dtype=np.float32))
    H8 = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    P8 = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    sH = torch.empty(1, dtype=torch.float32, device="cuda")
    ws_8 = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, 4, _abi.FP8_E4M3)
    a = dev_bf16(si.normal_f32((M, 4096), 118))
    b = dev_bf16(si.normal_f32((4096, 264), 119, 0.02))
    Yk = torch.empty(M, 264, dtype=torch.bfloat16, device="cuda")
    ws_k = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, 264, 4096)
    assert ws_k.numel() > 2048                                   # split-K planned
    # a paired linear backward (ticket counters zeroed by a kernel, dW split)
    lx = dev_bf16(si.normal_f32((2048, 512), 120))
    lw = dev_bf16(si.normal_f32((512, 256), 121, 0.05))
    ldy = dev_bf16(si.normal_f32((2048, 256), 122))
    ldW = torch.empty(512, 256, dtype=torch.bfloat16, device="cuda")
    ldX = torch.empty(2048, 512, dtype=torch.bfloat16, device="cuda")
    ws_l = tpm.alloc_workspace(_abi.OP_LINEAR_BWD, 2048, 256, 512)
    assert ws_l.numel() > 2048                                   # dW's contraction split

    def run():
        tpm.tp_mlp_fwd(X, Wu, Wd, H, stack[1], T=T, rank=1, act=_abi.ACT_GELU_TANH, num_chunks=4, workspace=ws_f)
        tpm.partial_reduce_seqshard(stack, out, T=T, rank=1)
        tpm.tp_mlp_fwd(xq, wuq, wdq, H8, P8, T=T, rank=0, act=_abi.ACT_RELU, scales=scales, h_scale_out=sH,
                       num_chunks=4, workspace=ws_8)
        tpm.seq_chunk_gemm(a, b, Yk, workspace=ws_k)
        tpm.tp_linear_bwd(lx, lw, ldy, ldW, ldX, workspace=ws_l)

    run()
    sync()
    ref = [t.clone() for t in (H, stack, out, H8, P8, sH, Yk, ldW, ldX)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    sync()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        for t in (H, out, H8, P8, sH, Yk, ldW, ldX):
            t.zero_()
        stack[1].zero_()
        sync()
        g.replay()
        sync()
        for got, want in zip((H, stack, out, H8, P8, sH, Yk, ldW, ldX), ref):
            assert torch.equal(got, want), rep


# ------------------------------------------------------- linear backward pair
LINEAR_SHAPES = [(296, 264, 520),     # ragged tiles, no split
                 (4096, 256, 1024),   # dW's contraction (4096 tokens) split 8 ways
                 (520, 4096, 264)]    # dX's contraction (4096) split 8 ways, dW first


@pytest.mark.parametrize("M,N,K", LINEAR_SHAPES)
def test_linear_bwd_integer_exact(M, N, K):
    # dW = X^T dY and dX = dY W^T in one launch; small integers make every
    # fp32 sum exact, so dW (fp32) must equal the oracle bit for bit and dX
    # (bf16) its single rounding, whatever split or work-group took a tile
    x = si.small_ints((M, K), 91)
    w = si.small_ints((K, N), 92)
    dy = si.small_ints((M, N), 93)
    dW = torch.empty(K, N, dtype=torch.float32, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_LINEAR_BWD, M, N, K)
    tpm.tp_linear_bwd(dev_bf16(x), dev_bf16(w), dev_bf16(dy), dW, dX, workspace=ws)
    sync()
    ref = ops.linear_bwd(x, w, dy)
    assert np.array_equal(f64(dW), ref["dW"])
    assert np.array_equal(f64(dX), formats.round_bf16(ref["dX"]))


def test_linear_bwd_float_repeatable_and_fp32():
    # float inputs: both products within the bf16 bound of the oracle, and
    # three calls bit-identical (which work-group takes which tile varies)
    M, N, K = 1000, 1280, 2056
    x = dev_bf16(si.normal_f32((M, K), 94))
    w = dev_bf16(si.normal_f32((K, N), 95, 0.02))
    dy = dev_bf16(si.normal_f32((M, N), 96))
    ws = tpm.alloc_workspace(_abi.OP_LINEAR_BWD, M, N, K)
    outs = []
    for _ in range(3):
        dW = torch.empty(K, N, dtype=torch.bfloat16, device="cuda")
        dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
        tpm.tp_linear_bwd(x, w, dy, dW, dX, workspace=ws)
        sync()
        outs.append((dW.clone(), dX.clone()))
    ref = ops.linear_bwd(f64(x), f64(w), f64(dy))
    assert nerr(outs[0][0], ref["dW"]) <= TOL["bf16"] and nerr(outs[0][1], ref["dX"]) <= TOL["bf16"]
    assert all(torch.equal(a, outs[0][0]) and torch.equal(b, outs[0][1]) for a, b in outs[1:])
    # fp32 inputs take the fp32 kernel for both products (1e-4 bound)
    xs, ws_, dys = (torch.from_numpy(si.uniform_f32(s, seed)).cuda()
                    for s, seed in (((40, 24), 97), ((24, 36), 98), ((40, 36), 99)))
    dW32 = torch.empty(24, 36, dtype=torch.float32, device="cuda")
    dX32 = torch.empty(40, 24, dtype=torch.float32, device="cuda")
    tpm.tp_linear_bwd(xs, ws_, dys, dW32, dX32)
    sync()
    r32 = ops.linear_bwd(f64(xs), f64(ws_), f64(dys))
    assert nerr(dW32, r32["dW"]) <= TOL["f32"] and nerr(dX32, r32["dX"]) <= TOL["f32"]


def test_linear_bwd_rejects_bad_arguments():
    x = torch.zeros(64, 32, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(32, 48, dtype=torch.bfloat16, device="cuda")
    dy = torch.zeros(64, 48, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(32, 48, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(64, 32, dtype=torch.bfloat16, device="cuda")
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tpm.TpmError):
        tpm.tp_linear_bwd(x, w, dy, dW, dX, workspace=small)        # workspace too small
    # an operand off 16-byte alignment runs on the predicated kernel: the
    # same (integer, exact) result as the aligned call
    xi, wi, dyi = si.small_ints((64, 32), 451), si.small_ints((32, 48), 452), si.small_ints((64, 48), 453)
    xa, wa, dya = dev_bf16(xi), dev_bf16(wi), dev_bf16(dyi)
    xm = torch.zeros(64 * 32 + 1, dtype=torch.bfloat16, device="cuda")[1:].view(64, 32)
    xm.copy_(xa)
    dW2, dX2 = torch.empty_like(dW), torch.empty_like(dX)
    tpm.tp_linear_bwd(xa, wa, dya, dW, dX)
    tpm.tp_linear_bwd(xm, wa, dya, dW2, dX2)
    sync()
    assert torch.equal(dW, dW2) and torch.equal(dX, dX2)
    assert np.array_equal(f64(dW2), formats.round_bf16(xi.T.astype(np.float64) @ dyi))
    with pytest.raises(ValueError):
        tpm.tp_linear_bwd(x, w, dy, dW, dX.float())                 # dX is written in the inputs' dtype
    with pytest.raises(ValueError):
        tpm.tp_linear_bwd(x, w, dy[:, :40].contiguous(), dW, dX)    # dY is [M, N]


def test_linear_bwd_empty_contractions():
    # M = 0 tokens: dW = X^T dY contracts over nothing and must be zeros, dX
    # is empty; N = 0: dX contracts over nothing (zeros), dW is empty
    ws = tpm.alloc_workspace(_abi.OP_LINEAR_BWD, 0, 64, 40)
    e = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    dW = torch.full((40, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    tpm.tp_linear_bwd(e(0, 40), e(40, 64), e(0, 64), dW, e(0, 40), workspace=ws)
    dX = torch.full((48, 40), 7.0, dtype=torch.bfloat16, device="cuda")
    ws2 = tpm.alloc_workspace(_abi.OP_LINEAR_BWD, 48, 0, 40)
    tpm.tp_linear_bwd(e(48, 40), e(40, 0), e(48, 0), e(40, 0), dX, workspace=ws2)
    sync()
    assert torch.count_nonzero(dW).item() == 0
    assert torch.count_nonzero(dX).item() == 0


@pytest.mark.parametrize("act", [_abi.ACT_GELU_ERF, _abi.ACT_GELU_TANH, _abi.ACT_SILU, _abi.ACT_RELU]
                         if torch.cuda.is_available() else [])
def test_epilogue_activation_accuracy(act):
    # the epilogue's activation and derivative on exact inputs: a rank-one
    # product puts every bf16 value z of [-12, 12] through the forward
    # epilogue (Y = act(z)) and, with Z = z saved and a product of 1, the
    # DACT epilogue (Y = act'(z)), fp32 outputs, against the oracle's float64
    # functions: within 1e-5 relative + 3e-7 absolute (the hardware exp / rcp
    # and, for GeLU-erf, Abramowitz & Stegun 7.1.26 with its 1.5e-7 bound)
    z = np.unique(formats.round_bf16(np.linspace(-12.0, 12.0, 20001)))
    z = np.concatenate([z, np.zeros((-len(z)) % 8)])
    M, K, N = len(z), 16, 8
    a = np.zeros((M, K), np.float32)
    a[:, 0] = z
    b = np.zeros((K, N), np.float32)
    b[0, :] = 1.0
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(dev_bf16(a), dev_bf16(b), Y, act=act)
    ones = np.zeros((M, K), np.float32)
    ones[:, 0] = 1.0
    Z = dev_f32(np.repeat(z[:, None], N, axis=1))
    G = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(dev_bf16(ones), dev_bf16(b), G, epilogue=_abi.EPI_DACT, act=act, aux=Z)
    sync()
    for got, ref in ((f64(Y)[:, 0], ops.act_fwd(z, act)), (f64(G)[:, 0], ops.act_grad(z, act))):
        assert np.all(np.isfinite(got))
        assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 3e-7), float(np.max(np.abs(got - ref)))


def test_bf16_output_rounding_ties_and_subnormals():
    # the epilogue's fp32 -> bf16 rounding on exact fp32 inputs: Y = x + y
    # with x, y bf16 whose exponents differ by at most 16 (so x + y is exact
    # in fp32 but has bits below bf16 precision), exact ties (y = half an
    # ulp of x, both parities), signs, and subnormal magnitudes; the bf16
    # output must equal the oracle's nearest-even rounding bit for bit
    g = np.random.default_rng(131)
    n = 1 << 14
    x = formats.round_bf16(g.standard_normal(n) * np.exp2(g.integers(-20, 20, n)))
    y = formats.round_bf16(x * np.exp2(-g.integers(0, 17, n).astype(np.float64)) * g.choice([-1.0, 1.0], n)
                           * (1 + g.integers(0, 128, n) / 128.0))
    ties_x = formats.round_bf16(np.abs(g.standard_normal(1024)) + 1.0)
    ties_y = np.exp2(np.floor(np.log2(ties_x)) - 8)                  # half an ulp of x
    sub_x = formats.round_bf16(g.standard_normal(1024) * 2.0 ** -130)
    sub_y = formats.round_bf16(g.standard_normal(1024) * 2.0 ** -133)
    X = np.concatenate([x, ties_x, sub_x])
    Yv = np.concatenate([y, ties_y, sub_y])
    ok = np.isfinite(X) & np.isfinite(Yv)
    X, Yv = X[ok], Yv[ok]
    assert np.all((X + Yv).astype(np.float32).astype(np.float64) == X + Yv)   # exact in fp32
    M = (len(X) + 7) // 8 * 8
    a = np.zeros((M, 8), np.float64)
    a[:len(X), 0], a[:len(X), 1] = X, Yv
    b = np.zeros((8, 8), np.float64)
    b[0, :] = b[1, :] = 1.0
    out = torch.empty(M, 8, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(si.to_bf16(a.astype(np.float32)).cuda(), si.to_bf16(b.astype(np.float32)).cuda(), out)
    sync()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)[:len(X), 0]
    # the accumulator starts at +0, so -0 + -0 gives +0 there
    want = formats.f32_to_bf16_bits((0.0 + X + Yv).astype(np.float32))
    assert np.array_equal(got, want)


def test_dact_epilogue_integer_exact_ragged_and_strided_z():
    # DACT with ReLU' in {0, 1} on integer products is exact: Y must equal
    # bf16(A.B * relu'(Z)) bit for bit.  Ragged rows and columns (300 =
    # 256 + 44, 264 = 256 + 8) exercise the masked loads of Z, and Z is a view
    # into a wider array (leading dimension N + 24)
    M, N, K = 300, 264, 200
    a = si.small_ints((M, K), 141)
    b = si.small_ints((N, K), 142)
    zfull = si.small_ints((M, N + 24), 143).astype(np.float32)            # includes exact zeros: the kink
    assert np.mean(zfull[:, :N] == 0) > 0.05
    Zd = dev_bf16(zfull)[:, :N]
    assert Zd.stride(0) == N + 24
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tpm.seq_chunk_gemm(dev_bf16(a), dev_bf16(b), Y, trans_b=True, epilogue=_abi.EPI_DACT, act=_abi.ACT_RELU, aux=Zd)
    sync()
    exact = (a.astype(np.float64) @ b.astype(np.float64).T) * (zfull[:, :N] > 0)
    assert np.array_equal(f64(Y), formats.round_bf16(exact))
    # ReLU'(0) = 0 ("Tensor parallelism", section "Code": 1 only where z > 0)
    kink = (zfull[:, :N] == 0) & ((a.astype(np.float64) @ b.astype(np.float64).T) != 0)
    assert kink.any() and not f64(Y)[kink].any()


# ------------------------------------------- predicated path (any shape / alignment)
def _placed(x, ld, off, dtype=torch.bfloat16):
    """A device view of host array x [rows, cols] at element offset `off` of a
    flat buffer, leading dimension ld (pointer alignment follows `off`)."""
    rows, cols = x.shape
    buf = torch.full((rows * ld + off + 8,), float("nan") if dtype != torch.uint8 else 0,
                     dtype=dtype if dtype != torch.uint8 else torch.uint8, device="cuda")
    v = torch.as_strided(buf, (rows, cols), (ld, 1), off)
    if dtype == torch.bfloat16:
        v.copy_(si.to_bf16(x).cuda())
    else:
        v.copy_(x.cuda())
    return v


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_gemm_ragged_n_k_integer_exact(ta, tb):
    """N = 1001, K = 999 (no whole 16-byte chunks), every operand layout:
    the predicated kernel, bit-exact on integer inputs; ReLU with its kink."""
    M, N, K = 300, 1001, 999
    a, b, A, B = _operands(M, N, K, ta, tb, lambda s, seed: si.small_ints(s, seed), 401)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, N, dtype=torch.float32, device="cuda")
    Yf = torch.empty(M, N, dtype=torch.float32, device="cuda")
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    tpm.seq_chunk_gemm(dev_bf16(A), dev_bf16(B), Yf, trans_a=ta, trans_b=tb, M=M, N=N, K=K, act=_abi.ACT_RELU,
                       aux=Z)
    tpm.seq_chunk_gemm(dev_bf16(A), dev_bf16(B), Y, trans_a=ta, trans_b=tb, M=M, N=N, K=K, act=_abi.ACT_RELU,
                       amax_out=amax, workspace=ws)
    sync()
    exact, _ = ops.seq_chunk_gemm(A, B, trans_a=ta, trans_b=tb)
    assert np.array_equal(f64(Z), exact)
    assert np.array_equal(f64(Yf), np.maximum(exact, 0))
    assert np.array_equal(f64(Y), formats.round_bf16(np.maximum(exact, 0)))
    assert amax.item() == float(np.max(formats.round_bf16(np.maximum(exact, 0))))


def test_gemm_unaligned_pointers_and_leading_dimensions():
    """Operands and output at odd element offsets (not 16-byte aligned) with
    odd leading dimensions, float inputs, GeLU and a saved Z: against the
    oracle, and integer inputs bit-exact; a DACT epilogue reading an
    unaligned Z."""
    M, N, K = 257, 136, 264
    x = si.normal_f32((M, K), 411)
    w = si.normal_f32((K, N), 412, 0.05)
    A = _placed(x, K + 3, 3)
    B = _placed(w, N + 5, 5)
    Y = _placed(np.zeros((M, N), np.float32), N + 1, 1)
    Z = _placed(np.zeros((M, N), np.float32), N + 7, 7)
    assert A.data_ptr() % 16 and B.data_ptr() % 16 and Y.data_ptr() % 16
    tpm.seq_chunk_gemm(A, B, Y, act=_abi.ACT_GELU_ERF, aux=Z)
    sync()
    y, z = ops.seq_chunk_gemm(f64(A), f64(B), act=_abi.ACT_GELU_ERF)
    assert nerr(Y, y) <= TOL["bf16"] and nerr(Z, z) <= TOL["bf16"]
    xi, wi = si.small_ints((M, K), 413), si.small_ints((K, N), 414)
    A2, B2 = _placed(xi, K + 3, 3), _placed(wi, N + 5, 5)
    tpm.seq_chunk_gemm(A2, B2, Y)
    Zd = _placed(si.small_ints((M, N), 415).astype(np.float32), N + 7, 7)
    D = _placed(np.zeros((M, N), np.float32), N + 1, 1)
    tpm.seq_chunk_gemm(A2, B2, D, epilogue=_abi.EPI_DACT, act=_abi.ACT_RELU, aux=Zd)
    sync()
    exact = xi.astype(np.float64) @ wi.astype(np.float64)
    assert np.array_equal(f64(Y), formats.round_bf16(exact))
    assert np.array_equal(f64(D), formats.round_bf16(exact * (f64(Zd) > 0)))


def test_gemm_fp8_mn_major_on_the_predicated_path():
    """e4m3 operands in the pages' layout (B = W [K, N], not K-major) with
    scales: integer codes, exact."""
    M, N, K = 192, 200, 160
    xi, wi = si.small_ints((M, K), 421), si.small_ints((K, N), 422)
    X = si.to_e4m3_exact(xi).cuda()
    W = si.to_e4m3_exact(wi).cuda()
    sa = dev_f32(np.array([0.5], np.float32))
    sb = dev_f32(np.array([0.25], np.float32))
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    tpm.seq_chunk_gemm(X, W, Y, a_scale=sa, b_scale=sb)
    sync()
    assert np.array_equal(f64(Y), (xi.astype(np.float64) @ wi.astype(np.float64)) * 0.125)


def test_linear_bwd_and_mlp_on_ragged_shapes():
    """tp_linear_bwd with M, N, K not multiples of 8, and one rank's MLP
    share whose F/T (250) and D (200) leave no whole 16-byte chunks: every
    GEMM on the predicated kernel, checked against the oracle with the
    GPU's saved Z, H and dZ as the inputs of the later products."""
    M, N, K = 300, 100, 52
    x, w, dy = si.normal_f32((M, K), 431), si.normal_f32((K, N), 432, 0.1), si.normal_f32((M, N), 433)
    X, W, DY = dev_bf16(x), dev_bf16(w), dev_bf16(dy)
    dW = torch.empty(K, N, dtype=torch.bfloat16, device="cuda")
    dX = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(tpm.workspace_bytes(_abi.OP_LINEAR_BWD, M, N, K), dtype=torch.uint8, device="cuda")
    tpm.tp_linear_bwd(X, W, DY, dW, dX, workspace=ws)
    sync()
    r = ops.linear_bwd(f64(X), f64(W), f64(DY))
    assert nerr(dW, r["dW"]) <= TOL["bf16"] and nerr(dX, r["dX"]) <= TOL["bf16"]

    M, D, F, T, C = 260, 200, 1000, 4, 4
    Ft = F // T
    x = dev_bf16(si.normal_f32((M, D), 441))
    wu, wd = dev_bf16(si.normal_f32((D, Ft), 442, 0.05)), dev_bf16(si.normal_f32((Ft, D), 443, 0.05))
    dy = dev_bf16(si.normal_f32((M, D), 444))
    e = lambda *sh: torch.empty(*sh, dtype=torch.bfloat16, device="cuda")
    Z, H, P, dWu, dWd, dXo = e(M, Ft), e(M, Ft), e(M, D), e(D, Ft), e(Ft, D), e(M, D)
    wsb = tpm.alloc_workspace(_abi.OP_MLP_BWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_mlp_fwd(x, wu, wd, H, P, T=T, rank=0, act=_abi.ACT_GELU_ERF, Z_t=Z, num_chunks=C)
    tpm.tp_mlp_bwd(x, wu, wd, Z, H, dy, dWu, dWd, dXo, T=T, rank=0, act=_abi.ACT_GELU_ERF, num_chunks=C,
                   workspace=wsb)
    sync()
    X64, WU, WD, DY = f64(x), f64(wu), f64(wd), f64(dy)
    fw = ops.tp_mlp_fwd(X64, WU, WD, ops.ACT_GELU_ERF)
    assert nerr(Z, fw["Z"]) <= TOL["bf16"] and nerr(H, fw["H"]) <= TOL["bf16"]
    assert nerr(P, ops.gemm(f64(H), WD)) <= TOL["bf16"]
    dz = wsb[2048:2048 + 2 * M * Ft].view(torch.bfloat16).view(M, Ft)
    bw = ops.tp_mlp_bwd(X64, WU, WD, f64(Z), f64(H), DY, ops.ACT_GELU_ERF, dz_stored=f64(dz))
    assert nerr(dz, bw["dZ"]) <= TOL["bf16"]
    for got, k in ((dWu, "dW_up"), (dWd, "dW_down"), (dXo, "dX")):
        assert nerr(got, bw[k]) <= TOL["bf16"], k

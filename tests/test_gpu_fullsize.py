"""Parity at the workloads' full sizes, in the launch configuration bench.py
uses (same shapes, chunk counts and orders, dtypes and workspaces), checked
on sampled outputs that the fp64 oracle computes one by one: a GEMM output
row needs only the matching rows of its left operand, a column only the
matching column of its right operand, so the oracle runs on those slices.
Where a quantity depends on the whole tensor (the fp8 amax of H), the check
at full size is a property that holds at any size, and a reduced-token run
at the full hidden / FFN sizes is compared end to end."""
import numpy as np
import pytest
import torch

import sequence_transformer_gemms_amd as tpm
from sequence_transformer_gemms_amd import _abi
import synthetic_inputs as si
from oracle import formats, ops
from tests import _util
from tests._util import TOL, assert_mx_close, f64, nerr

pytestmark = pytest.mark.gpu


def sync():
    torch.cuda.synchronize()


def pick(n, k, seed):
    """k distinct sorted indices in [0, n), always including the first and last."""
    g = np.random.default_rng(seed)
    idx = set(g.choice(n, size=k - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(idx))


def host64(t):
    """fp64 values of a (CPU or device) tensor's rows/cols already selected."""
    return f64(t.cpu() if t.is_cuda else t)


# ------------------------------------------------------------------ C2
def test_c2_projection_full_size_resident_and_arriving():
    """Single column-parallel projection: X [8192, 8192] bf16, rank shard
    t = 0 of W [8192, 32768] (columns 0..8191), 4 chunks of 2048 tokens in
    ring order [0, 3, 2, 1]; resident, then with the chunks written by the
    side-stream writer on disjoint CUs (bitwise equal)."""
    M, K, Nfull, T, C = 8192, 8192, 32768, 4, 4
    N = Nfull // T
    x = si.to_bf16(si.normal_f32((M, K), 1))
    w = si.to_bf16(np.ascontiguousarray(si.normal_f32((K, Nfull), 2, 1.0 / np.sqrt(8192.0))[:, :N]))
    X, W = x.cuda(), w.cuda()
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    order = si.ring_chunk_order(T, C, 0)
    assert order == [0, 3, 2, 1]
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K, num_chunks=C)
    tpm.seq_chunk_gemm(X, W, Y, num_chunks=C, chunk_order=order, workspace=ws)
    sync()
    ref, _ = ops.seq_chunk_gemm(f64(x), f64(w))             # the whole output
    assert nerr(Y, ref) <= TOL["bf16"]
    del ref

    compute, producer = tpm.masked_streams(producer_cus=8)
    Xa = torch.zeros_like(X)
    flags = torch.zeros(C, dtype=torch.int32, device="cuda")
    counters = torch.zeros(C, dtype=torch.int32, device="cuda")
    Y2 = torch.empty_like(Y)
    sync()
    tpm.seq_chunk_gemm(Xa, W, Y2, num_chunks=C, chunk_order=order, chunk_ready=flags, epoch=1, workspace=ws,
                       stream=compute)
    tpm.write_chunks(Xa, X, C, order, flags, 1, counters, stream=producer)
    sync()
    assert tpm.poll_device_error(ws) == 0
    assert torch.equal(Y2, Y)


# ------------------------------------------------------------------ C3
def test_c3_mlp_forward_full_size_and_reduction():
    """Llama3-70B-shaped MLP share of rank 0 of TP = 8, bf16: 8192 tokens,
    D = 8192, F = 28672 (F/T = 3584), GeLU, 8 chunks in ring order, the
    second GEMM producing destination ranges in order r+1, ..., r; then the
    sequence-sharded reduction of 8 seeded partials [8192, 8192]."""
    M, D, F, T, C, r = 8192, 8192, 28672, 8, 8, 0
    Ft = F // T
    x = si.to_bf16(si.normal_f32((M, D), 1))
    wu = si.to_bf16(si.normal_f32((D, Ft), 2, 0.02))
    wd = si.to_bf16(si.normal_f32((Ft, D), 3, 0.02))
    X, Wu, Wd = x.cuda(), wu.cuda(), wd.cuda()
    H = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty_like(H)
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    done = torch.zeros(T, dtype=torch.int32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_mlp_fwd(X, Wu, Wd, H, P, T=T, rank=r, act=_abi.ACT_GELU_ERF, Z_t=Z, num_chunks=C,
                   chunk_order=si.ring_chunk_order(T, C, r), range_order=si.dest_range_order(T, r),
                   range_done=done, epoch=3, workspace=ws)
    sync()
    assert torch.all(done == 3)
    # whole outputs: Z and H against the exact product, P against the exact
    # product of the H the GPU stored
    ref = ops.tp_mlp_fwd(f64(x), f64(wu), f64(wd), ops.ACT_GELU_ERF)
    assert nerr(Z, ref["Z"]) <= TOL["bf16"]
    assert nerr(H, ref["H"]) <= TOL["bf16"]
    assert nerr(P, ops.gemm(f64(H), f64(wd))) <= TOL["bf16"]
    del ref
    del X, Wu, Wd, H, Z, P, ws
    torch.cuda.empty_cache()

    # reduction: partials [8, 8192, 8192] N(0,1) seeds 100..107 -> rank 5's [1024, 8192] slice
    stack = torch.empty(T, M, D, dtype=torch.bfloat16, device="cuda")
    host = []
    for t in range(T):
        pt = si.to_bf16(si.normal_f32((M, D), 100 + t))
        host.append(pt)
        stack[t] = pt.cuda()
    out = torch.empty(M // T, D, dtype=torch.bfloat16, device="cuda")
    rank = 5
    tpm.partial_reduce_seqshard(stack, out, T=T, rank=rank)
    sync()
    lrows, cols = pick(M // T, 64, 32), pick(D, 64, 33)
    grows = rank * (M // T) + lrows
    parts = np.stack([f64(h[grows][:, cols]) for h in host])          # [T, rows, cols]
    ref_red = ops.partial_reduce_seqshard(parts, -1)
    got = host64(out[lrows][:, cols])
    # one rounding of the fp32 sum to bf16: within half a bf16 ulp plus fp32 summation error
    assert nerr(got, ref_red) <= TOL["bf16"]
    assert np.array_equal(got, formats.round_bf16(ref_red)) or \
        np.mean(got != formats.round_bf16(ref_red)) < 1e-3


# ------------------------------------------------------------------ C4
def _c4_inputs(M, D, F, T):
    Ft = F // T
    xq, sx = si.to_e4m3_current(si.normal_f32((M, D), 1))
    wu = si.normal_f32((D, Ft), 2, 0.02)
    wd = si.normal_f32((Ft, D), 3, 0.02)
    wuq, su = si.to_e4m3_current(np.ascontiguousarray(wu.T))    # K-major copies: [Ft, D]
    wdq, sd = si.to_e4m3_current(np.ascontiguousarray(wd.T))    # [D, Ft]
    return xq, sx, wuq, su, wdq, sd


def _c4_run(xq, sx, wuq, su, wdq, sd, M, D, F, T, C):
    Ft = F // T
    scales = torch.tensor([sx, su, sd], dtype=torch.float32, device="cuda")
    H = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    sH = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, C, _abi.FP8_E4M3)
    tpm.tp_mlp_fwd(xq.cuda(), wuq.cuda(), wdq.cuda(), H, P, T=T, rank=0, act=_abi.ACT_GELU_ERF, scales=scales,
                   h_scale_out=sH, num_chunks=C, chunk_order=si.ring_chunk_order(T, C, 0), workspace=ws)
    sync()
    return H, P, sH, ws


def test_c4_fp8_mlp_forward_full_size():
    """Llama3-405B-shaped MLP share, fp8 e4m3 with per-tensor current scales:
    8192 tokens, D = 16384, F/T = 6656, 16 chunks of 512, against the
    oracle's whole fp8 chain (H, its amax and e4m3 codes, P) at full size.
    H is stored in bf16 (bf16 tolerance); the codes and scale are exactly
    the quantisation of the GPU's own H, and differ from the oracle's codes
    only where the GPU's bf16 H does (tests/_util.assert_fp8_h_consistent)."""
    M, D, F, T, C = 8192, 16384, 53248, 8, 16
    Ft = F // T
    xq, sx, wuq, su, wdq, sd = _c4_inputs(M, D, F, T)
    H, P, sH, ws = _c4_run(xq, sx, wuq, su, wdq, sd, M, D, F, T, C)
    hq = ws[2048:2048 + M * Ft].cpu().numpy().reshape(M, Ft)
    h_gpu, p_gpu, s_gpu = f64(H), f64(P), sH.item()
    del H, P, ws
    torch.cuda.empty_cache()
    ref = ops.tp_mlp_fwd_fp8(f64(xq), sx, f64(wuq).T, su, f64(wdq).T, sd, ops.ACT_GELU_ERF)
    assert nerr(h_gpu, ref["H"]) <= TOL["bf16"]
    hb_diff, flips = _util.assert_fp8_h_consistent(h_gpu, hq, s_gpu, ref)
    # GEMM2 against the exact product of the codes and scale the GPU gave it;
    # the whole chain (the oracle's own codes) is reported beside it: its
    # largest normalised difference comes from the code differences above
    # (about seven per 6656-term output row)
    wd_dec = f64(wdq).T * float(np.float32(sd))
    p_own = ops.gemm(formats.e4m3_to_f64(hq), wd_dec) * s_gpu
    assert nerr(p_gpu, p_own) <= TOL["fp8"]
    print(f"C4 full size: bf16 H differs from the oracle's rounding at {hb_diff:.2e}, e4m3 codes at {flips:.2e}; "
          f"P vs the GPU's codes {nerr(p_gpu, p_own):.2e}, vs the oracle's whole chain {nerr(p_gpu, ref['P']):.2e}")


def test_c4_fp8_mlp_forward_full_width_end_to_end():
    """The same hidden and FFN sizes and 16 chunks, 32 tokens: small enough
    for the oracle to compute the whole H (hence its amax) and compare H,
    the scale, the e4m3 codes of H and P end to end."""
    M, D, F, T, C = 32, 16384, 53248, 8, 16
    xq, sx, wuq, su, wdq, sd = _c4_inputs(M, D, F, T)
    H, P, sH, ws = _c4_run(xq, sx, wuq, su, wdq, sd, M, D, F, T, C)
    ref = ops.tp_mlp_fwd_fp8(f64(xq), sx, f64(wuq).T, su, f64(wdq).T, sd, ops.ACT_GELU_ERF)
    assert nerr(host64(H), ref["H"]) <= TOL["bf16"]
    assert nerr(host64(P), ref["P"]) <= TOL["fp8"]
    Ft = F // T
    hq = ws[2048:2048 + M * Ft].cpu().numpy().reshape(M, Ft)
    _util.assert_fp8_h_consistent(host64(H), hq, sH.item(), ref, max_flip=1e-2)


# ------------------------------------------------------------------ C5
def test_c5_layer_step_full_size_sampled():
    """The bench's Llama3-70B-shaped layer step of rank 0 (4096 tokens, bf16),
    call by call with the bench's shapes, orders and workspaces: QKV and O
    projections, MLP forward, MLP backward, O and QKV backward (as separate
    GEMMs, and as the paired tp_linear_bwd launches of the resident step).  Row-indexed
    outputs are checked on sampled token rows, weight gradients on sampled
    rows or columns."""
    M, D, F, T, C, r = 4096, 8192, 28672, 8, 8, 0
    Ft, Nq, Da = F // T, 1280, 1024
    bf = lambda a: si.to_bf16(a)
    x = bf(si.normal_f32((M, D), 1))
    wu = bf(si.normal_f32((D, Ft), 2, 0.02))
    wd = bf(si.normal_f32((Ft, D), 3, 0.02))
    dy = bf(si.normal_f32((M, D), 4))
    wq = bf(si.normal_f32((D, Nq), 5, 0.02))
    wo = bf(si.normal_f32((Da, D), 6, 0.02))
    a = bf(si.normal_f32((M, Da), 7))
    dq = bf(si.normal_f32((M, Nq), 8))
    dyo = bf(si.normal_f32((M, D), 9))
    dev = {k: v.cuda() for k, v in dict(x=x, wu=wu, wd=wd, dy=dy, wq=wq, wo=wo, a=a, dq=dq, dyo=dyo).items()}
    e = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    shapes = [(M, Nq, D, T), (M, D, Da, T), (M, Da, D, T), (Da, D, M, 1), (D, Nq, M, 1), (M, D, Nq, 1)]
    wsg = torch.zeros(max(tpm.workspace_bytes(_abi.OP_SEQ_CHUNK_GEMM, m, n, k, 1, c) for m, n, k, c in shapes),
                      dtype=torch.uint8, device="cuda")
    order, dest = si.ring_chunk_order(T, C, r), si.dest_range_order(T, r)
    qkv, o_part, z, h, p = e(M, Nq), e(M, D), e(M, Ft), e(M, Ft), e(M, D)
    g_up, g_down, dx, d_attn, g_o, g_qkv, dx_q = e(D, Ft), e(Ft, D), e(M, D), e(M, Da), e(Da, D), e(D, Nq), e(M, D)
    tpm.seq_chunk_gemm(dev["x"], dev["wq"], qkv, num_chunks=C, chunk_order=order, workspace=wsg)
    tpm.seq_chunk_gemm(dev["a"], dev["wo"], o_part, num_chunks=T, chunk_order=dest, workspace=wsg)
    ws_f = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_mlp_fwd(dev["x"], dev["wu"], dev["wd"], h, p, T=T, rank=r, act=_abi.ACT_GELU_ERF, Z_t=z, num_chunks=C,
                   chunk_order=order, workspace=ws_f)
    ws_b = tpm.alloc_workspace(_abi.OP_MLP_BWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_mlp_bwd(dev["x"], dev["wu"], dev["wd"], z, h, dev["dy"], g_up, g_down, dx, T=T, rank=r,
                   act=_abi.ACT_GELU_ERF, num_chunks=C, dy_chunk_order=order, workspace=ws_b)
    tpm.seq_chunk_gemm(dev["dyo"], dev["wo"], d_attn, trans_b=True, num_chunks=C, chunk_order=order, workspace=wsg)
    tpm.seq_chunk_gemm(dev["a"], dev["dyo"], g_o, trans_a=True, workspace=wsg)
    tpm.seq_chunk_gemm(dev["x"], dev["dq"], g_qkv, trans_a=True, workspace=wsg)
    tpm.seq_chunk_gemm(dev["dq"], dev["wq"], dx_q, trans_b=True, workspace=wsg)
    # the same two backward pairs as the resident step runs them: one launch each
    ws_l = torch.zeros(max(tpm.workspace_bytes(_abi.OP_LINEAR_BWD, M, n, k) for n, k in ((D, Da), (Nq, D))),
                       dtype=torch.uint8, device="cuda")
    g_o2, d_attn2, g_qkv2, dx_q2 = e(Da, D), e(M, Da), e(D, Nq), e(M, D)
    tpm.tp_linear_bwd(dev["a"], dev["wo"], dev["dyo"], g_o2, d_attn2, workspace=ws_l)
    tpm.tp_linear_bwd(dev["x"], dev["wq"], dev["dq"], g_qkv2, dx_q2, workspace=ws_l)
    sync()
    B = TOL["bf16"]
    X, WU, WD, DY = f64(x), f64(wu), f64(wd), f64(dy)
    WQ, WO, A_, DQ, DYO = f64(wq), f64(wo), f64(a), f64(dq), f64(dyo)
    # every output in full, each GEMM against the exact product of the inputs
    # the GPU gave it: the saved Z and H of the forward and the dZ the
    # backward stored (its workspace, after the control block) are the GPU's
    # own, so no bf16 rounding of an intermediate is re-derived here
    assert nerr(qkv, X @ WQ) <= B
    assert nerr(o_part, A_ @ WO) <= B
    Zx = X @ WU
    assert nerr(z, Zx) <= B
    assert nerr(h, ops.act_fwd(Zx, ops.ACT_GELU_ERF)) <= B
    Zg, Hg = f64(z), f64(h)
    assert nerr(p, Hg @ WD) <= B
    dz = f64(ws_b[2048:2048 + 2 * M * Ft].view(torch.bfloat16).view(M, Ft))
    bw = ops.tp_mlp_bwd(X, WU, WD, Zg, Hg, DY, ops.ACT_GELU_ERF, dz_stored=dz)
    assert nerr(dz, bw["dZ"]) <= B
    assert nerr(g_down, bw["dW_down"]) <= B
    assert nerr(g_up, bw["dW_up"]) <= B
    assert nerr(dx, bw["dX"]) <= B
    ref_da, ref_go = DYO @ WO.T, A_.T @ DYO
    ref_gq, ref_dxq = X.T @ DQ, DQ @ WQ.T
    assert nerr(d_attn, ref_da) <= B and nerr(g_o, ref_go) <= B
    assert nerr(g_qkv, ref_gq) <= B and nerr(dx_q, ref_dxq) <= B
    # the paired launches of the resident step
    assert nerr(d_attn2, ref_da) <= B and nerr(g_o2, ref_go) <= B
    assert nerr(g_qkv2, ref_gq) <= B and nerr(dx_q2, ref_dxq) <= B


# ------------------------------------------------- tensor-parallel degree sweep
@pytest.mark.parametrize("T", [1, 2, 4])
def test_tp_degree_sweep_shapes_sampled_and_chunk_invariant(T):
    """The Llama3-70B MLP share (8192 tokens, D = 8192, F = 28672) at the
    other tensor-parallel degrees bench.py --sweep times (T = 8 is C3):
    rank 0's F/T = 28672 / T columns, chunk-gated with the flags already set.
    Sampled rows of Z, H and P against the oracle with C = T chunks in ring
    order; then C = 4T chunks give bitwise the same forward and backward
    results (the chunk count only changes the tile order)."""
    M, D, F = 8192, 8192, 28672
    Ft = F // T
    x = si.to_bf16(si.normal_f32((M, D), 1))
    wu = si.to_bf16(si.normal_f32((D, Ft), 2, 0.02))
    wd = si.to_bf16(si.normal_f32((Ft, D), 3, 0.02))
    X, Wu, Wd = x.cuda(), wu.cuda(), wd.cuda()
    dY = si.to_bf16(si.normal_f32((M, D), 4)).cuda()
    outs = []
    for C in (T, 4 * T):
        Z = torch.empty(M, Ft, dtype=torch.bfloat16, device="cuda")
        H, P = torch.empty_like(Z), torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
        dWu, dWd, dX = torch.empty_like(Wu), torch.empty_like(Wd), torch.empty_like(X)
        flags = torch.full((C,), 2, dtype=torch.int32, device="cuda")
        order = si.ring_chunk_order(T, C, 0)
        ws = tpm.alloc_workspace(_abi.OP_MLP_FWD, M, D, F, T, C, _abi.BF16)
        tpm.tp_mlp_fwd(X, Wu, Wd, H, P, T=T, rank=0, act=_abi.ACT_GELU_ERF, Z_t=Z, num_chunks=C,
                       chunk_order=order, chunk_ready=flags, epoch=2, workspace=ws)
        wsb = tpm.alloc_workspace(_abi.OP_MLP_BWD, M, D, F, T, C, _abi.BF16)
        tpm.tp_mlp_bwd(X, Wu, Wd, Z, H, dY, dWu, dWd, dX, T=T, rank=0, act=_abi.ACT_GELU_ERF, num_chunks=C,
                       dy_chunk_order=order, dy_ready=flags, epoch=2, workspace=wsb)
        sync()
        assert tpm.poll_device_error(ws) == 0 and tpm.poll_device_error(wsb) == 0
        outs.append((Z, H, P, dWu, dWd, dX))
        del ws, wsb
    rows = pick(M, 12, 60 + T)
    ref = ops.tp_mlp_fwd(f64(x[rows]), f64(wu), f64(wd), ops.ACT_GELU_ERF, store="bf16")
    Z, H, P = outs[0][:3]
    assert nerr(host64(Z[rows]), ref["Z"]) <= TOL["bf16"]
    assert nerr(host64(H[rows]), ref["H"]) <= TOL["bf16"]
    assert nerr(host64(P[rows]), ref["P"]) <= TOL["bf16"]
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


# ------------------------------------------------ gated MLP (worked example)
def test_gated_mlp_worked_example_full_size_sampled():
    """The worked example's MLP pair ("Tensor and sequence parallelism",
    "Worked example: Partitioning an MLP pair") at its full size, rank 0 of
    T = 4: X [8192, 4096], gate and up shards [4096, 4096] each (side by side
    in one [4096, 8192] buffer), SwiGLU, contraction shard [4096, 4096], 4
    chunks in ring order; forward and backward as bench.py runs them.  Rows
    of G, U, H, P and dX; columns of dW_gate, dW_up and rows of dW_down, with
    the bf16-rounding ambiguity of the stored intermediates added to the bound
    (as for the layer step's weight gradients)."""
    M, D, F, T, C, r = 8192, 4096, 16384, 4, 4, 0
    Ft, act = F // T, ops.ACT_SILU
    x = si.to_bf16(si.normal_f32((M, D), 1))
    wg, wu = si.to_bf16(si.normal_f32((D, Ft), 2, 0.02)), si.to_bf16(si.normal_f32((D, Ft), 5, 0.02))
    wd = si.to_bf16(si.normal_f32((Ft, D), 3, 0.02))
    dy = si.to_bf16(si.normal_f32((M, D), 4))
    X, WGU, WD, DYd = x.cuda(), torch.cat([wg, wu], dim=1).cuda(), wd.cuda(), dy.cuda()
    e = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device="cuda")
    GU, H, P = e(M, 2 * Ft), e(M, Ft), e(M, D)
    dWgu, dWd, dX = e(D, 2 * Ft), e(Ft, D), e(M, D)
    flags = torch.full((C,), 1, dtype=torch.int32, device="cuda")
    order = si.ring_chunk_order(T, C, r)
    wsf = tpm.alloc_workspace(_abi.OP_GATED_MLP_FWD, M, D, F, T, C, _abi.BF16)
    wsb = tpm.alloc_workspace(_abi.OP_GATED_MLP_BWD, M, D, F, T, C, _abi.BF16)
    tpm.tp_gated_mlp_fwd(X, WGU, WD, H, P, T=T, rank=r, act=act, GU_t=GU, num_chunks=C, chunk_order=order,
                         chunk_ready=flags, epoch=1, workspace=wsf)
    tpm.tp_gated_mlp_bwd(X, WGU, WD, GU, H, DYd, dWgu, dWd, dX, T=T, rank=r, act=act, num_chunks=C,
                         dy_chunk_order=order, dy_ready=flags, epoch=1, workspace=wsb)
    sync()
    assert tpm.poll_device_error(wsf) == 0 and tpm.poll_device_error(wsb) == 0
    B = TOL["bf16"]
    Xf, WG, WU, WDf, DY = f64(x), f64(wg), f64(wu), f64(wd), f64(dy)
    # whole outputs; each GEMM against the exact product of the inputs the
    # GPU gave it (its saved [G | U] and H, and the [dG | dU] the backward
    # stored in its workspace after the control block)
    G_ex, U_ex = Xf @ WG, Xf @ WU
    GUg, Hg = f64(GU), f64(H)
    assert nerr(GUg[:, :Ft], G_ex) <= B and nerr(GUg[:, Ft:], U_ex) <= B
    assert nerr(Hg, ops.act_fwd(G_ex, act) * U_ex) <= B
    assert nerr(P, Hg @ WDf) <= B
    dgu = f64(wsb[2048:2048 + 2 * M * 2 * Ft].view(torch.bfloat16).view(M, 2 * Ft))
    dh = DY @ WDf.T
    g, u = GUg[:, :Ft], GUg[:, Ft:]
    assert nerr(dgu[:, :Ft], dh * u * ops.act_grad(g, act)) <= B
    assert nerr(dgu[:, Ft:], dh * ops.act_fwd(g, act)) <= B
    assert nerr(dWd, Hg.T @ DY) <= B
    assert nerr(dWgu, Xf.T @ dgu) <= B
    assert nerr(dX, dgu @ np.concatenate([WG, WU], axis=1).T) <= B


# ------------------------------------------------------------ MXFP8 (C4 shape)
def test_c4_mxfp8_mlp_forward_full_size_sampled():
    """The fp8 configuration's shapes (8192 tokens, D = 16384, F = 53248,
    T = 8, 16 chunks in ring order) under MXFP8 block scaling: every operand
    in 32-element blocks along its contraction axis, H requantised to MXFP8
    in GEMM1's epilogue.  MX blocks are local to a row, so the oracle
    computes sampled token rows of Z, H (codes and block exponents) and P
    exactly; H is compared under the fp32-evaluation bound of its values."""
    M, D, F, T, C = 8192, 16384, 53248, 8, 16
    Ft = F // T
    xc, xe = (t.numpy() for t in si.to_mxfp8(si.normal_f32((M, D), 1)))
    uc, ue = (t.numpy() for t in si.to_mxfp8(si.normal_f32((Ft, D), 2, 0.02)))   # W_up,t K-major [Ft, D]
    dc, de = (t.numpy() for t in si.to_mxfp8(si.normal_f32((D, Ft), 3, 0.02)))   # W_down,t K-major [D, Ft]
    dev = lambda c, e, k: (torch.from_numpy(c).cuda(), tpm.mx_swizzle_scales(torch.from_numpy(e).cuda(), k))
    X, Xs = dev(xc, xe, D)
    WU, WUs = dev(uc, ue, D)
    WD, WDs = dev(dc, de, Ft)
    H = torch.empty(M, Ft, dtype=torch.uint8, device="cuda")
    Hs = torch.zeros(tpm.mx_scales_bytes(M, Ft), dtype=torch.uint8, device="cuda")
    P = torch.empty(M, D, dtype=torch.bfloat16, device="cuda")
    flags = torch.full((C,), 1, dtype=torch.int32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_MX_MLP_FWD, M, D, F, T, C, _abi.FP8_E4M3)
    tpm.tp_mlp_fwd_mx(X, Xs, WU, WUs, WD, WDs, H, Hs, P, T=T, rank=0, act=_abi.ACT_GELU_ERF, num_chunks=C,
                      chunk_order=si.ring_chunk_order(T, C, 0), chunk_ready=flags, epoch=1, workspace=ws)
    sync()
    assert tpm.poll_device_error(ws) == 0
    rows = pick(M, 10, 71)
    Xd = formats.mx_e4m3_decode(xc[rows], xe[rows])
    Ud = formats.mx_e4m3_decode(uc, ue)
    z = Xd @ Ud.T
    h = ops.act_fwd(z, ops.ACT_GELU_ERF)
    off = (((rows[:, None] // 32) * (Ft // 128) + np.arange(Ft // 32)[None, :] // 4) * 32 + rows[:, None] % 32) * 4 + \
        np.arange(Ft // 32)[None, :] % 4
    hc, he = H[rows].cpu().numpy(), Hs.cpu().numpy()[off]
    delta = D * 2.0 ** -24 * (np.abs(Xd) @ np.abs(Ud).T) * np.abs(ops.act_grad(z, ops.ACT_GELU_ERF)) + \
        2.0 ** -20 * np.abs(h) + 1e-30
    assert_mx_close(hc, he, h, delta)
    del Ud
    hq, hs = formats.mx_e4m3_quantize(h)
    p_ref = formats.mx_e4m3_decode(hq, hs) @ formats.mx_e4m3_decode(dc, de).T
    assert nerr(host64(P[rows]), p_ref) <= TOL["fp8"]

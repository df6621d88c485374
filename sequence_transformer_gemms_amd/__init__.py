"""One tensor-parallel rank's MLP hot path on AMD MI355X (gfx950).

Python face of libtpmlp: the four operations of include/tpmlp.h under the same
names, taking torch tensors for device memory and torch's current stream.
Arguments are marshalled to the C ABI; nothing is computed here.

    seq_chunk_gemm          chunk-fed local GEMM with fused epilogue
    tp_mlp_fwd              Z = X W_up,t; H = act(Z); P = H W_down,t (partial)
    tp_mlp_bwd              dZ, dW_down,t, dW_up,t, dX_t (partial)
    tp_gated_mlp_fwd        G, U = X [W_gate,t | W_up,t]; H = act(G) * U; P = H W_down,t
    tp_gated_mlp_bwd        [dG | dU], dW_down,t, [dW_gate,t | dW_up,t], dX_t (partial)
    seq_chunk_gemm_mx       the local GEMM with MXFP8 operands (and optionally output)
    tp_mlp_fwd_mx           the MLP forward under MXFP8 block scaling
    tp_mlp_fwd_delayed      the fp8 MLP forward under delayed scaling (+ fp8_delayed_scale)
    tp_mlp_bwd_fp8          the MLP backward in fp8 (e5m2 gradients); cast_fp8 the current-scaling cast
    partial_reduce_seqshard sum of T partials over this rank's token slice
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import (ACT_GELU_ERF, ACT_GELU_TANH, ACT_NONE, ACT_RELU, ACT_SILU, BF16, EPI_DACT,  # noqa: F401
                   EPI_DGATED, EPI_FWD, EPI_GATED, F32, FP8_E4M3, FP8_E5M2, OP_CAST_FP8, OP_FP8_DELAYED_MLP_FWD, OP_LINEAR_BWD,
                   OP_GATED_MLP_BWD, OP_GATED_MLP_FWD, OP_MLP_BWD, OP_MLP_BWD_FP8, OP_MLP_FWD, OP_MX_MLP_FWD,
                   OP_SEQ_CHUNK_GEMM, TpmError, check, lib)
from .streams import masked_streams  # noqa: F401

__all__ = ["seq_chunk_gemm", "seq_chunk_gemm_noalloc", "tp_mlp_fwd", "tp_mlp_bwd", "tp_linear_bwd", "tp_gated_mlp_fwd", "tp_gated_mlp_bwd",
           "seq_chunk_gemm_mx", "tp_mlp_fwd_mx", "mx_scales_bytes", "mx_swizzle_scales",
           "tp_mlp_fwd_delayed", "fp8_delayed_scale", "cast_fp8", "tp_mlp_bwd_fp8",
           "partial_reduce_seqshard",
           "workspace_bytes", "alloc_workspace", "signal_chunk", "write_chunks", "poll_device_error",
           "set_wait_limit", "dtype_code", "masked_streams", "TpmError", "lib"]


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    if t == torch.float8_e5m2:
        return FP8_E5M2
    raise TypeError(f"unsupported dtype {t}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ld(t: torch.Tensor) -> int:
    assert t.dim() == 2 and t.stride(1) == 1, "row-major 2-D tensors with unit inner stride"
    return t.stride(0)


def workspace_bytes(op: int, M: int, N: int, K: int, T: int = 1, num_chunks: int = 1, dtype: int = BF16) -> int:
    return int(lib.tpm_workspace_bytes(op, M, N, K, T, num_chunks, dtype))


def alloc_workspace(op: int, M: int, N: int, K: int, T: int = 1, num_chunks: int = 1, dtype: int = BF16,
                    device="cuda") -> torch.Tensor:
    # zero-filled: the error word reads TPM_OK until a chunk-gated call sets it
    return torch.zeros(max(workspace_bytes(op, M, N, K, T, num_chunks, dtype), 1), dtype=torch.uint8, device=device)


def seq_chunk_gemm(A, B, Y, *, trans_a=False, trans_b=False, a_scale=None, b_scale=None,
                   epilogue=EPI_FWD, act=ACT_NONE, aux=None, amax_out=None, num_chunks=1,
                   chunk_order=None, chunk_ready=None, epoch=0, workspace=None, stream=None,
                   M=None, N=None, K=None):
    """Y = epilogue(op(A) . op(B)); shapes are taken from the tensors (with
    EPI_GATED, B is [W_gate | W_up] and N is half its width)."""
    if M is None:
        M = A.shape[1] if trans_a else A.shape[0]
    if K is None:
        K = A.shape[0] if trans_a else A.shape[1]
    if N is None:
        N = B.shape[0] if trans_b else B.shape[1]
        if epilogue == EPI_GATED:
            N //= 2
    order = _abi.int_array(chunk_order)
    rc = lib.seq_chunk_gemm(M, N, K,
                            _ptr(A), _ld(A), int(trans_a), dtype_code(A.dtype), _ptr(a_scale),
                            _ptr(B), _ld(B), int(trans_b), dtype_code(B.dtype), _ptr(b_scale),
                            _ptr(Y), _ld(Y), dtype_code(Y.dtype),
                            epilogue, act, _ptr(aux), _ld(aux) if aux is not None else 0, _ptr(amax_out),
                            num_chunks, order, _ptr(chunk_ready), epoch,
                            _ptr(workspace), workspace.numel() if workspace is not None else 0,
                            _stream(stream))
    return check(rc)


def seq_chunk_gemm_noalloc(A, B, Y, *, trans_a=False, trans_b=False, a_scale=None, b_scale=None,
                           epilogue=EPI_FWD, act=ACT_NONE, aux=None, amax_out=None, num_chunks=1,
                           chunk_order=None, stream=None, M=None, N=None, K=None):
    """seq_chunk_gemm without a workspace: control words and split-K partial
    sums in the library's own per-GPU device array (no allocation; calls that
    overlap on one GPU race).  No chunk flags."""
    if M is None:
        M = A.shape[1] if trans_a else A.shape[0]
    if K is None:
        K = A.shape[0] if trans_a else A.shape[1]
    if N is None:
        N = B.shape[0] if trans_b else B.shape[1]
    rc = lib.seq_chunk_gemm_noalloc(M, N, K,
                                    _ptr(A), _ld(A), int(trans_a), dtype_code(A.dtype), _ptr(a_scale),
                                    _ptr(B), _ld(B), int(trans_b), dtype_code(B.dtype), _ptr(b_scale),
                                    _ptr(Y), _ld(Y), dtype_code(Y.dtype),
                                    epilogue, act, _ptr(aux), _ld(aux) if aux is not None else 0, _ptr(amax_out),
                                    num_chunks, _abi.int_array(chunk_order), _stream(stream))
    return check(rc)


def tp_mlp_fwd(X, W_up_t, W_down_t, H_t, P_t, *, T, rank, act=ACT_GELU_ERF, Z_t=None, scales=None,
               h_scale_out=None, num_chunks=1, chunk_order=None, chunk_ready=None, epoch=0,
               range_order=None, range_done=None, workspace=None, stream=None):
    """One rank's forward.  Dense tensors: X [M,D], W_up_t [D,F/T], W_down_t
    [F/T,D] (fp8: stored transposed, [F/T,D] and [D,F/T]), H_t/Z_t [M,F/T],
    P_t [M,D]."""
    M, D = X.shape
    Ft = H_t.shape[1]
    dt = dtype_code(X.dtype)
    rc = lib.tp_mlp_fwd(M, D, Ft * T, T, rank,
                        _ptr(X), _ptr(W_up_t), _ptr(W_down_t),
                        dt, _ptr(scales), act,
                        _ptr(Z_t), _ptr(H_t), _ptr(P_t), _ptr(h_scale_out),
                        num_chunks, _abi.int_array(chunk_order), _ptr(chunk_ready), epoch,
                        _abi.int_array(range_order), _ptr(range_done),
                        _ptr(workspace), workspace.numel() if workspace is not None else 0,
                        _stream(stream))
    return check(rc)


def tp_mlp_bwd(X, W_up_t, W_down_t, Z_t, H_t, dY, dW_up_t, dW_down_t, dX_t, *, T, rank,
               act=ACT_GELU_ERF, num_chunks=1, dy_chunk_order=None, dy_ready=None, epoch=0,
               workspace=None, stream=None):
    M, D = X.shape
    Ft = H_t.shape[1]
    rc = lib.tp_mlp_bwd(M, D, Ft * T, T, rank,
                        _ptr(X), _ptr(W_up_t), _ptr(W_down_t),
                        _ptr(Z_t), _ptr(H_t), _ptr(dY),
                        dtype_code(X.dtype), act,
                        _ptr(dW_up_t), _ptr(dW_down_t), _ptr(dX_t), dtype_code(dW_up_t.dtype),
                        num_chunks, _abi.int_array(dy_chunk_order), _ptr(dy_ready), epoch,
                        _ptr(workspace), workspace.numel() if workspace is not None else 0,
                        _stream(stream))
    return check(rc)


def tp_linear_bwd(X, W, dY, dW, dX, *, workspace=None, stream=None):
    """dW = X^T . dY and dX = dY . W^T of a linear layer Y = X . W (X [M, K],
    W [K, N], dY [M, N]) in one call; the workspace defaults to a fresh one."""
    M, K = X.shape
    N = W.shape[1]
    if tuple(W.shape) != (K, N) or tuple(dY.shape) != (M, N) or tuple(dW.shape) != (K, N) or tuple(dX.shape) != (M, K):
        raise ValueError(f"tp_linear_bwd: shapes X {tuple(X.shape)}, W {tuple(W.shape)}, dY {tuple(dY.shape)}, "
                         f"dW {tuple(dW.shape)}, dX {tuple(dX.shape)}")
    if not (W.dtype == dY.dtype == dX.dtype == X.dtype):
        raise ValueError("tp_linear_bwd: X, W, dY and dX share one dtype (dW may be fp32)")
    for t in (X, W, dY, dW, dX):
        if t.numel() and (t.stride(1) != 1 or t.stride(0) != t.shape[1]):
            raise ValueError("tp_linear_bwd: dense row-major tensors")
    if workspace is None:
        workspace = alloc_workspace(OP_LINEAR_BWD, M, N, K, 1, 1, dtype_code(X.dtype), device=X.device)
    rc = lib.tp_linear_bwd(M, N, K, _ptr(X), _ptr(W), _ptr(dY), dtype_code(X.dtype),
                           _ptr(dW), _ptr(dX), dtype_code(dW.dtype),
                           _ptr(workspace), workspace.numel(), _stream(stream))
    return check(rc)


def tp_gated_mlp_fwd(X, W_gu_t, W_down_t, H_t, P_t, *, T, rank, act=ACT_SILU, GU_t=None, num_chunks=1,
                     chunk_order=None, chunk_ready=None, epoch=0, range_order=None, range_done=None,
                     workspace=None, stream=None):
    """One rank's gated-MLP forward (bf16).  X [M,D], W_gu_t [D, 2F/T] =
    [W_gate,t | W_up,t], W_down_t [F/T, D], H_t [M, F/T], P_t [M, D], GU_t
    [M, 2F/T] or None."""
    M, D = X.shape
    Ft = H_t.shape[1]
    rc = lib.tp_gated_mlp_fwd(M, D, Ft * T, T, rank, _ptr(X), _ptr(W_gu_t), _ptr(W_down_t),
                              dtype_code(X.dtype), act, _ptr(GU_t), _ptr(H_t), _ptr(P_t),
                              num_chunks, _abi.int_array(chunk_order), _ptr(chunk_ready), epoch,
                              _abi.int_array(range_order), _ptr(range_done),
                              _ptr(workspace), workspace.numel() if workspace is not None else 0,
                              _stream(stream))
    return check(rc)


def tp_gated_mlp_bwd(X, W_gu_t, W_down_t, GU_t, H_t, dY, dW_gu_t, dW_down_t, dX_t, *, T, rank, act=ACT_SILU,
                     num_chunks=1, dy_chunk_order=None, dy_ready=None, epoch=0, workspace=None, stream=None):
    M, D = X.shape
    Ft = H_t.shape[1]
    rc = lib.tp_gated_mlp_bwd(M, D, Ft * T, T, rank, _ptr(X), _ptr(W_gu_t), _ptr(W_down_t),
                              _ptr(GU_t), _ptr(H_t), _ptr(dY), dtype_code(X.dtype), act,
                              _ptr(dW_gu_t), _ptr(dW_down_t), _ptr(dX_t), dtype_code(dW_gu_t.dtype),
                              num_chunks, _abi.int_array(dy_chunk_order), _ptr(dy_ready), epoch,
                              _ptr(workspace), workspace.numel() if workspace is not None else 0,
                              _stream(stream))
    return check(rc)


def mx_scales_bytes(rows: int, k: int) -> int:
    return int(lib.tpm_mx_scales_bytes(rows, k))


def mx_swizzle_scales(scales, k: int, out=None, stream=None):
    """Row-major E8M0 scales [rows, K/32] (uint8, device) -> a new (or the
    given) uint8 device tensor in the scaled-MFMA layout."""
    rows = scales.shape[0]
    if out is None:
        out = torch.empty(max(mx_scales_bytes(rows, k), 1), dtype=torch.uint8, device=scales.device)
    check(lib.tpm_mx_swizzle_scales(rows, k, _ptr(scales), _ld(scales), _ptr(out), _stream(stream)))
    return out


def seq_chunk_gemm_mx(A, a_scales, B, b_scales, Y, *, y_scales=None, act=ACT_NONE, aux=None, num_chunks=1,
                      chunk_order=None, chunk_ready=None, epoch=0, workspace=None, stream=None):
    """Y = act(A . B^T) with MXFP8 operands: A [M, K], B stored [N, K] (codes,
    uint8) and their swizzled scales; Y bf16 / fp32, or uint8 codes with
    y_scales (MXFP8 output)."""
    M, K = A.shape
    N = B.shape[0]
    ydt = FP8_E4M3 if Y.dtype == torch.uint8 else dtype_code(Y.dtype)
    rc = lib.seq_chunk_gemm_mx(M, N, K, _ptr(A), _ld(A), _ptr(a_scales), _ptr(B), _ld(B), _ptr(b_scales),
                               _ptr(Y), _ld(Y), ydt, _ptr(y_scales), act, _ptr(aux), _ld(aux) if aux is not None else 0,
                               num_chunks, _abi.int_array(chunk_order), _ptr(chunk_ready), epoch,
                               _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    return check(rc)


def tp_mlp_fwd_mx(X, x_scales, W_up_t, w_up_scales, W_down_t, w_down_scales, H_t, h_scales, P_t, *, T, rank,
                  act=ACT_GELU_ERF, Z_t=None, num_chunks=1, chunk_order=None, chunk_ready=None, epoch=0,
                  range_order=None, range_done=None, workspace=None, stream=None):
    """MXFP8 forward: X [M,D] codes; W_up_t [F/T, D] and W_down_t [D, F/T]
    codes stored K-major; all scales swizzled; H_t [M, F/T] uint8 codes with
    h_scales; P_t [M, D] bf16."""
    M, D = X.shape
    Ft = H_t.shape[1]
    rc = lib.tp_mlp_fwd_mx(M, D, Ft * T, T, rank, _ptr(X), _ptr(x_scales), _ptr(W_up_t), _ptr(w_up_scales),
                           _ptr(W_down_t), _ptr(w_down_scales), act, _ptr(Z_t), _ptr(H_t), _ptr(h_scales), _ptr(P_t),
                           num_chunks, _abi.int_array(chunk_order), _ptr(chunk_ready), epoch,
                           _abi.int_array(range_order), _ptr(range_done),
                           _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    return check(rc)


def tp_mlp_fwd_delayed(X, W_up_t, W_down_t, H_t, P_t, *, T, rank, scales, h_scale, h_amax_out=None,
                       act=ACT_GELU_ERF, Z_t=None, num_chunks=1, chunk_order=None, chunk_ready=None, epoch=0,
                       range_order=None, range_done=None, workspace=None, stream=None):
    """fp8 forward under delayed scaling: X [M,D] codes, W_up_t [F/T, D] and
    W_down_t [D, F/T] codes stored K-major, scales = device fp32 {sX, sWup,
    sWdown}, h_scale = device fp32 scale of H fixed before the step; H_t
    [M, F/T] uint8 codes, P_t [M, D] bf16; h_amax_out (device fp32) gets
    max|H|."""
    M, D = X.shape
    Ft = H_t.shape[1]
    rc = lib.tp_mlp_fwd_delayed(M, D, Ft * T, T, rank, _ptr(X), _ptr(W_up_t), _ptr(W_down_t), _ptr(scales),
                                _ptr(h_scale), _ptr(h_amax_out), act, _ptr(Z_t), _ptr(H_t), _ptr(P_t),
                                num_chunks, _abi.int_array(chunk_order), _ptr(chunk_ready), epoch,
                                _abi.int_array(range_order), _ptr(range_done),
                                _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(stream))
    return check(rc)


def fp8_delayed_scale(amax_history, scale_out, stream=None):
    """scale_out[0] = max(amax_history) / 448 (1 when all are 0), on the device."""
    return check(lib.tpm_fp8_delayed_scale(_ptr(amax_history), amax_history.numel(), _ptr(scale_out),
                                           _stream(stream)))


def cast_fp8(x, dtype, q=None, qt=None, scale_out=None, workspace=None, stream=None):
    """Current-scaling cast of a bf16 [rows, cols] tensor to fp8 codes (dtype
    FP8_E4M3 or FP8_E5M2): q [rows, cols] and / or qt [cols, rows] (uint8),
    scale_out (device fp32) = amax / fmax."""
    rows, cols = x.shape
    if workspace is None:
        workspace = torch.zeros(max(workspace_bytes(OP_CAST_FP8, 0, 0, 0), 1), dtype=torch.uint8, device=x.device)
    rc = lib.tpm_cast_fp8(rows, cols, _ptr(x), _ld(x), dtype, _ptr(q), _ld(q) if q is not None else 0,
                          _ptr(qt), _ld(qt) if qt is not None else 0, _ptr(scale_out),
                          _ptr(workspace), workspace.numel(), _stream(stream))
    return check(rc)


def tp_mlp_bwd_fp8(X, W_up_t, W_down_t, Z_t, H_t, dY, dW_up_t, dW_down_t, dX_t, *, T, rank, scales,
                   act=ACT_GELU_ERF, dy_scale=None, num_chunks=1, dy_chunk_order=None, dy_ready=None, epoch=0,
                   workspace=None, stream=None):
    """fp8 backward: X [M, D] e4m3 codes, W_up_t [D, F/T] and W_down_t [F/T, D]
    e4m3 codes (the pages' layouts), scales = device fp32 {sX, sWup, sWdown};
    Z_t, H_t [M, F/T] bf16; dY [M, D] bf16 (cast here with current scaling,
    all rows resident) or uint8 e5m2 codes with dy_scale (device fp32), whose
    rows may arrive in chunks (dy_ready); dW_up_t, dW_down_t (bf16 / fp32),
    dX_t bf16."""
    M, D = X.shape
    Ft = H_t.shape[1]
    codes = dY.dtype == torch.uint8
    rc = lib.tp_mlp_bwd_fp8(M, D, Ft * T, T, rank, _ptr(X), _ptr(W_up_t), _ptr(W_down_t), _ptr(scales),
                            _ptr(Z_t), _ptr(H_t), _ptr(dY), FP8_E5M2 if codes else BF16, _ptr(dy_scale), act,
                            _ptr(dW_up_t), _ptr(dW_down_t), _ptr(dX_t), dtype_code(dW_up_t.dtype),
                            num_chunks, _abi.int_array(dy_chunk_order), _ptr(dy_ready), epoch, _ptr(workspace),
                            workspace.numel() if workspace is not None else 0, _stream(stream))
    return check(rc)


def partial_reduce_seqshard(partials, out, *, T, rank, M=None, stream=None):
    """partials: [T, M, D] (or [T, M/T, D] with rank=-1); out: [M/T, D]."""
    assert partials.dim() == 3 and partials.stride(2) == 1
    Tn, rows, D = partials.shape
    assert Tn == T
    if M is None:
        M = rows if rank >= 0 else rows * T
    rc = lib.partial_reduce_seqshard(T, M, D, rank, _ptr(partials), partials.stride(0), partials.stride(1),
                                     dtype_code(partials.dtype), _ptr(out), _ld(out), dtype_code(out.dtype),
                                     _stream(stream))
    return check(rc)


def signal_chunk(flag_tensor, index: int, value: int, stream=None):
    """Release-store `value` into flag_tensor[index] (device uint32/int32) on `stream`."""
    ptr = flag_tensor.data_ptr() + 4 * index
    return check(lib.tpm_signal_chunk(_stream(stream), ptr, value))


def write_chunks(dst, src, num_chunks: int, order, ready, epoch: int, counters, copy=None, stream=None):
    """Side-stream chunk writer: for c in `order`, copy rows chunk c of `src`
    into `dst` (skipped where copy[c] is false) and then set ready[c] = epoch.
    dst/src: contiguous device tensors of equal size, split into num_chunks
    equal chunks; ready/counters: device int32/uint32 tensors of num_chunks
    words (counters zero before the first call)."""
    nbytes = dst.numel() * dst.element_size()
    if src.numel() * src.element_size() != nbytes or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("write_chunks: dst and src must be contiguous and of equal size")
    if nbytes % num_chunks != 0:
        raise ValueError("write_chunks: size not divisible by num_chunks")
    order_arr = (ctypes.c_int32 * num_chunks)(*[int(c) for c in order])
    copy_arr = None if copy is None else (ctypes.c_uint8 * num_chunks)(*[1 if b else 0 for b in copy])
    return check(lib.tpm_write_chunks(_ptr(dst), _ptr(src), nbytes // num_chunks, num_chunks, order_arr, copy_arr,
                                      _ptr(ready), epoch, _ptr(counters), _stream(stream)))


def poll_device_error(workspace) -> int:
    return int(lib.tpm_poll_device_error(_ptr(workspace)))


def set_wait_limit(polls: int) -> None:
    check(lib.tpm_set_wait_limit(ctypes.c_uint32(polls).value))

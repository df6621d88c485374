"""The allocation-free entry point against seq_chunk_gemm with a workspace:
two calls in a row (the second smaller, both planning split-K, so the
second reuses the per-GPU scratch the first left behind), bit for bit; the
amax is zeroed by each call.  A shape with a tail split (its last tile
column in K pieces) takes the same scratch."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from tests._util import f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import sequence_transformer_gemms_amd as tpm
    from sequence_transformer_gemms_amd import _abi


def _run_pair(M, N, K, seed, act, trans_b):
    a = si.normal_f32((M, K), seed)
    b = si.normal_f32((N, K) if trans_b else (K, N), seed + 1, 0.05)
    A, B = si.to_bf16(a).cuda(), si.to_bf16(b).cuda()
    Y0 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    Y1 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Z0, Z1 = torch.empty_like(Y0), torch.empty_like(Y0)
    m0 = torch.empty(1, dtype=torch.float32, device="cuda")
    m1 = torch.full((1,), 1e30, dtype=torch.float32, device="cuda")
    ws = tpm.alloc_workspace(_abi.OP_SEQ_CHUNK_GEMM, M, N, K)
    assert ws.numel() > 2048                                   # the plan splits K
    tpm.seq_chunk_gemm(A, B, Y0, trans_b=trans_b, act=act, aux=Z0, amax_out=m0, workspace=ws)
    tpm.seq_chunk_gemm_noalloc(A, B, Y1, trans_b=trans_b, act=act, aux=Z1, amax_out=m1)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1) and torch.equal(Z0, Z1) and torch.equal(m0, m1)
    return f64(Y1)


def test_noalloc_matches_workspace_call_twice_then_smaller():
    # 8 output tiles, K cut in 8: 16.8 MB of partial sums
    _run_pair(1024, 512, 4096, 501, _abi.ACT_GELU_ERF, False)
    # smaller: one tile, K = 2048 in 8 pieces (2 MB of the same scratch)
    y = _run_pair(256, 200, 2048, 503, _abi.ACT_RELU, True)
    assert np.all(y >= 0)


def test_noalloc_integer_exact_and_repeatable():
    M, N, K = 512, 256, 1024
    a, b = si.small_ints((M, K), 505), si.small_ints((K, N), 506)
    A, B = si.to_bf16(a).cuda(), si.to_bf16(b).cuda()
    Y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    for _ in range(2):
        tpm.seq_chunk_gemm_noalloc(A, B, Y)
        torch.cuda.synchronize()
        assert np.array_equal(f64(Y), a.astype(np.float64) @ b.astype(np.float64))


def test_noalloc_tail_split_matches_workspace_call():
    # 17 x 16 tiles: the last tile column's 17 tiles in 2 K pieces (8.9 MB of
    # partials in the per-GPU scratch), then a smaller split-K call reusing it
    M, N, K = 4312, 4072, 1024
    assert tpm.workspace_bytes(_abi.OP_SEQ_CHUNK_GEMM, M, N, K) == 2048 + 17 * 2 * 256 * 256 * 4
    _run_pair(M, N, K, 507, _abi.ACT_GELU_TANH, False)
    _run_pair(256, 200, 2048, 509, _abi.ACT_NONE, True)

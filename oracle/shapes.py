"""Local shapes and payloads of column- and row-parallel layers.

"Tensor and sequence parallelism", sections "Derive column-parallel linear
algebra", "Derive row-parallel linear algebra", "Calculate local shapes and
communication" and "Worked example: Partitioning an MLP pair"; "Tensor
parallelism", section "Complexity and constants" (all-reduce payload of
2*b*s*h bytes in bf16).
"""
from __future__ import annotations


def column_parallel(M: int, K: int, N: int, T: int) -> dict:
    assert N % T == 0
    return dict(W_t=(K, N // T), Y_t=(M, N // T), dW_t=(K, N // T), dX_t=(M, K),
                forward_collective=None, backward_collective="sum of dX_t partials")


def row_parallel(M: int, K: int, N: int, T: int) -> dict:
    assert K % T == 0
    return dict(X_t=(M, K // T), W_t=(K // T, N), Y_t=(M, N), dW_t=(K // T, N),
                dX_t=(M, K // T), forward_collective="sum of Y_t partials",
                backward_collective=None)


def partial_payload_bytes(M: int, N: int, elem_bytes: int = 2) -> int:
    """Bytes of one [M,N] partial output (bf16 by default)."""
    return M * N * elem_bytes


def seq_slice_rows(M: int, T: int) -> int:
    """Rows each rank owns after a reduce-scatter along tokens."""
    assert M % T == 0
    return M // T

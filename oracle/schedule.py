"""Unit-cost timeline of a layer boundary, with and without chunked overlap.

Reading of "Collective GEMMs in Tensor Sequence Parallelism", Figure 3 and
section "Collective GEMMs (CGEMM)": the tensor is cut into n sequence chunks;
each chunk costs `c` units of GEMM and `m` units of transfer; the blocking
collective moves the whole tensor (n transfers) before or after the whole
GEMM.

  all-gather + GEMM: the own chunk is present at time 0; remote chunks land
  back to back (chunk i at i*m); chunk i's GEMM starts when it has landed and
  the previous chunk's GEMM is done.  No tail: the boundary is n*c when m <= c.

  GEMM + reduce-scatter: range i can be sent once its GEMM is done and the
  previous send has finished; the first GEMM and the last send are exposed.

The figure's numbers (n = 4, c = m = 1): all-gather end 8 -> 4 units,
reduce-scatter end 8 -> 5 units.
"""
from __future__ import annotations


def serial(n: int, c: float = 1.0, m: float = 1.0) -> float:
    return n * m + n * c


def allgather_gemm(n: int, c: float = 1.0, m: float = 1.0) -> float:
    t = 0.0
    for i in range(n):
        arrival = 0.0 if i == 0 else i * m
        t = max(t, arrival) + c
    return t


def gemm_reducescatter(n: int, c: float = 1.0, m: float = 1.0) -> float:
    send_done = 0.0
    for i in range(n):
        computed = (i + 1) * c
        send_done = max(send_done, computed) + m
    return send_done

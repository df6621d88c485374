"""fp64 CPU oracle for one tensor-parallel rank's MLP hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package; only tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py use it.  It shares no code with the HIP library.

What it computes is exact dense linear algebra (the sharded layer equals the
unsharded one, "Tensor parallelism" algorithm page, section "How it works";
"Tensor and sequence parallelism", sections "Derive column-parallel linear
algebra" and "Derive row-parallel linear algebra"), so the oracle is that
definition written out in float64, plus a mirror of the fp8 current-scaling
quantisation of the intermediate activation (the "FP8 with current scaling"
recipe of "Collective GEMMs in Tensor Sequence Parallelism").

Modules:
  formats  -- bf16 / OCP e4m3fn decode and round-to-nearest-even encode
  ops      -- activations, GEMM, the four operations and their backward
  brute    -- pure-Python math.fsum brute force for tiny shapes
  schedule -- unit-cost timeline model of chunked all-gather+GEMM and
              GEMM+reduce-scatter (Figure 3 of the collective-GEMM blog)
  shapes   -- local shapes and payload bytes of column/row-parallel layers

Parity unpinned: GeLU evaluated by the GPU in fp32 against fp64 erf (checked
by tolerance only); fp8 code flips of the intermediate activation at rounding
boundaries (counted, tolerance only).
"""

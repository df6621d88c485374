/*
 * tpmlp -- one tensor-parallel rank's share of a transformer MLP under
 * tensor-sequence parallelism, on one AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; no framework types.  All matrices are
 * row-major with an explicit leading dimension (elements between consecutive
 * rows), as the pages write them: X[M,K], W[K,N] ("Tensor and sequence
 * parallelism", section "Derive column-parallel linear algebra").
 *
 * Ownership: the caller owns every buffer (device memory unless marked host)
 * and every stream.  The library never allocates, frees or synchronises a
 * stream; it only enqueues kernels on the `stream` argument (a hipStream_t;
 * NULL is the default stream).  Calls are asynchronous.
 *
 * Errors: every argument check runs on the host before anything is
 * enqueued; on failure the call returns a negative tpm_status, enqueues
 * nothing, and tpm_last_error() describes the problem (thread-local).  A
 * launch failure returns TPM_EHIP.  A device-side wait that gives up
 * (watchdog) is reported by tpm_poll_device_error() after the stream has
 * been synchronised.
 *
 * Shapes and alignment: any M, N, K >= 0 and any leading dimensions are
 * accepted ("Tensor parallelism", section "Implementation notes", asks only
 * that the sharded dimensions divide by T).  The matrix-core kernel takes a
 * GEMM whose rows are whole 16-byte chunks: N % 8 == 0; K and the operands'
 * leading dimensions multiples of 8 (bf16) or 16 (fp8); ldy, ldaux % 4 == 0;
 * A, B, Y, aux 16-byte aligned; with trans_a, M % 8 == 0; fp8 operands
 * stored K-major; each operand under 4 GiB.  Any other GEMM runs on a
 * predicated LDS-tiled FMA kernel (same results up to fp32 summation order,
 * far slower), which takes the FWD / DACT epilogues, scales and amax but not
 * chunk gating, range signalling, the gated epilogues or MXFP8 / fp8
 * outputs: those return TPM_EUNSUPPORTED unless the fast-path conditions hold.
 */
#ifndef TPMLP_H
#define TPMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  TPM_FP8_E4M3 is OCP e4m3fn (bias 7, max 448, no inf);
 * TPM_FP8_E5M2 is OCP e5m2 (bias 15, max 57344; the gradient format of the
 * hybrid fp8 recipe).  An fp8 GEMM may mix the two (not e5m2 x e5m2). */
typedef enum { TPM_F32 = 0, TPM_BF16 = 1, TPM_FP8_E4M3 = 2, TPM_FP8_E5M2 = 3 } tpm_dtype;

/* Activations.  GELU_ERF: 0.5 z (1 + erf(z / sqrt 2)); GELU_TANH: the tanh
 * approximation; RELU: max(z, 0) with derivative 1 only where z > 0
 * ("Tensor parallelism" algorithm page, section "Code"); SILU: z sigma(z),
 * sigma the logistic function (the gate of SwiGLU).  Evaluated in fp32 in
 * the GEMM epilogues on the hardware exp2 / reciprocal units; erf through
 * Hastings' approximation (Abramowitz & Stegun eq. 7.1.26, absolute error
 * below 1.5e-7): each activation and its derivative are within 1e-5
 * relative + 3e-7 absolute of the exact function. */
typedef enum {
  TPM_ACT_NONE = 0, TPM_ACT_RELU = 1, TPM_ACT_GELU_ERF = 2, TPM_ACT_GELU_TANH = 3, TPM_ACT_SILU = 4
} tpm_act;

/* Epilogue of seq_chunk_gemm.  The gated forms serve the gated MLP of the
 * worked example in "Tensor and sequence parallelism" ("Worked example:
 * Partitioning an MLP pair"), H = act(X W_gate) * (X W_up), with the gate
 * and up shards side by side: W_gu = [W_gate | W_up], [K, 2N]. */
typedef enum {
  TPM_EPI_FWD = 0,   /* Y = act(acc * sa * sb); aux (optional) receives the pre-activation */
  TPM_EPI_DACT = 1,  /* Y = acc * sa * sb * act'(aux): aux is the saved pre-activation Z */
  TPM_EPI_GATED = 2, /* B is W_gu [K, ldb >= 2N] (trans_b = 0): G = op(A) . B[:, 0:N],
                        U = op(A) . B[:, N:2N]; Y[M,N] = act(G) * U; aux (optional,
                        [M, ldaux >= 2N]) receives [G | U].  bf16 operands, trans_a = 0,
                        no amax. */
  TPM_EPI_DGATED = 3 /* acc is dH [M,N]; aux is the saved [G | U] ([M, ldaux >= 2N]);
                        Y [M, ldy >= 2N] receives [dG | dU] with dG = dH * U * act'(G),
                        dU = dH * act(G).  bf16 operands, no amax. */
} tpm_epilogue;

typedef enum {
  TPM_OK = 0,
  TPM_EINVAL = -1,       /* bad pointer, size, leading dimension or order */
  TPM_EUNSUPPORTED = -2, /* valid but not implemented (dtype / layout / alignment combination) */
  TPM_EHIP = -3,         /* a HIP launch failed */
  TPM_ETIMEOUT = -4,     /* a device-side wait for a chunk gave up (watchdog) */
  TPM_EWORKSPACE = -5    /* workspace missing or smaller than tpm_workspace_bytes() */
} tpm_status;

/* Operation ids for tpm_workspace_bytes(). */
typedef enum {
  TPM_OP_SEQ_CHUNK_GEMM = 0, TPM_OP_MLP_FWD = 1, TPM_OP_MLP_BWD = 2,
  TPM_OP_GATED_MLP_FWD = 3, TPM_OP_GATED_MLP_BWD = 4, TPM_OP_MX_MLP_FWD = 5, TPM_OP_FP8_DELAYED_MLP_FWD = 6,
  TPM_OP_MLP_BWD_FP8 = 7, TPM_OP_CAST_FP8 = 8, TPM_OP_LINEAR_BWD = 9
} tpm_op;

#define TPM_MAX_CHUNKS 256

/*
 * seq_chunk_gemm -- one local GEMM of a tensor-parallel rank, fed by
 * sequence chunks in arrival order ("Collective GEMMs in Tensor Sequence
 * Parallelism", section "Collective GEMMs (CGEMM)", all-gather + GEMM: each
 * chunk of tokens yields distinct output rows, written in place with no
 * accumulation).
 *
 *   Y[M,N] = epilogue( op(A)[M,K] . op(B)[K,N] )
 *
 * A: trans_a = 0 -> A is [M, lda >= K] (K contiguous, e.g. the activation
 *    X[tokens, K]); trans_a = 1 -> A is stored [K, lda >= M] and op(A) = A^T
 *    (e.g. X^T in a weight gradient).
 * B: trans_b = 0 -> B is [K, ldb >= N] (the pages' W[K,N]); trans_b = 1 ->
 *    B is stored [N, ldb >= K] and op(B) = B^T (e.g. W^T in dX = dY W^T).
 * a_dtype == b_dtype in {F32, BF16}, or both fp8 (E4M3 / E5M2, not both
 *    E5M2); fp32 accumulation always.  fp8 operands stored K-major
 *    (trans_a = 0, trans_b = 1) run on the matrix cores.
 * a_scale, b_scale: device fp32 dequantisation factors (value = code *
 *    scale), or NULL for 1.
 * Y: [M, ldy >= N], y_dtype F32 or BF16 (round to nearest even).
 * epilogue/act/aux: see tpm_epilogue; aux is [M, ldaux >= N] of y_dtype
 *    (FWD: written if non-NULL; DACT: required, read; the gated forms use
 *    [M, 2N] aux and, for DGATED, a [M, 2N] Y).
 * amax_out: device fp32 or NULL; set to max |Y| as stored (zeroed by the
 *    call first).
 * Chunks: the M rows of Y are cut into num_chunks equal chunks (M %
 *    num_chunks == 0, 1 <= num_chunks <= TPM_MAX_CHUNKS).  chunk_order
 *    (HOST, num_chunks entries, a permutation) is the arrival order, or NULL
 *    for ascending.  chunk_ready (DEVICE, num_chunks uint32) or NULL: when
 *    given, no row of chunk c is read before chunk_ready[c] >= epoch
 *    (wrap-around compare); the flags are written by the producer of the
 *    chunk (tpm_signal_chunk).  The result does not depend on the order.
 *    The producer must be able to run while the call waits: on CUs the
 *    gated kernel does not hold (a CU-masked pair of streams), and not
 *    ordered behind it -- e.g. not enqueued on a blocking stream after the
 *    null stream was made to wait for the gated call (HIP's null stream
 *    orders itself against blocking streams, and streams created with a CU
 *    mask are blocking).  A wait that cannot end gives up after the
 *    watchdog limit with TPM_ETIMEOUT in the workspace's error word.
 *    A chunk-gated A must be stored token-major (trans_a = 0) with its
 *    base and every chunk boundary ((M / num_chunks) * lda * element size)
 *    on a 128-byte line, so no cache line of a chunk is fetched before its
 *    flag is seen (else TPM_EUNSUPPORTED).
 * workspace: device, >= tpm_workspace_bytes(TPM_OP_SEQ_CHUNK_GEMM, ...);
 *    required when chunk_ready or amax_out is given, else may be NULL
 *    (then no split-K: a GEMM with few output tiles runs on fewer CUs).
 *    Its head holds control words and its tail the fp32 partial sums of
 *    split-K; calls that share a workspace must not overlap in time.
 */
int seq_chunk_gemm(int64_t M, int64_t N, int64_t K,
                   const void* A, int64_t lda, int trans_a, int a_dtype, const float* a_scale,
                   const void* B, int64_t ldb, int trans_b, int b_dtype, const float* b_scale,
                   void* Y, int64_t ldy, int y_dtype,
                   int epilogue, int act, void* aux, int64_t ldaux, float* amax_out,
                   int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * seq_chunk_gemm_noalloc -- seq_chunk_gemm for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * device allocation): the same arguments without the workspace and without
 * chunk flags (its watchdog word would not be visible to the caller), the
 * same kernels and split-K plan, hence the same results.  Control words and
 * the fp32 split-K partial sums live in a library-owned device array of
 * TPM_NOALLOC_SCRATCH_BYTES per GPU (2 KiB + 64 MiB), set up on the first
 * call on a device and held until the process ends; the call allocates and
 * frees nothing.  A GEMM whose split-K plan needs more scratch returns
 * TPM_EUNSUPPORTED (nothing enqueued): use seq_chunk_gemm with a workspace.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (different streams, or the same call replayed concurrently)
 * race and give wrong results.  amax_out (device, optional) is zeroed by
 * the call as in seq_chunk_gemm.
 */
#define TPM_NOALLOC_SCRATCH_BYTES ((size_t)2048 + ((size_t)64 << 20))
int seq_chunk_gemm_noalloc(int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, int trans_a, int a_dtype, const float* a_scale,
                           const void* B, int64_t ldb, int trans_b, int b_dtype, const float* b_scale,
                           void* Y, int64_t ldy, int y_dtype,
                           int epilogue, int act, void* aux, int64_t ldaux, float* amax_out,
                           int num_chunks, const int32_t* chunk_order, void* stream);

/*
 * tp_mlp_fwd -- rank `rank` of a T-way tensor-parallel MLP ("Tensor
 * parallelism" algorithm page, section "How it works"; "Tensor and sequence
 * parallelism", section "Pair adjacent transformer projections"):
 *
 *   Z_t = X . W_up,t            column-parallel, [M, F/T], chunk-fed
 *   H_t = act(Z_t)              local activation
 *   P_t = H_t . W_down,t        row-parallel partial [M, D]
 *
 * X: [M, D] (the all-gathered token rows), dtype BF16, F32 or FP8_E4M3;
 * all arrays dense (leading dimension = row width).  BF16 / F32 weights in
 * the pages' layout: W_up_t [D, F/T], W_down_t [F/T, D].  FP8_E4M3 weights
 * stored K-major (the transposed copies fp8 recipes keep): W_up_t [F/T, D],
 * W_down_t [D, F/T]; the leading dimensions are taken from D and F/T, so a
 * weight in the other layout is not detected.  Z_t (optional), H_t:
 * [M, F/T]; P_t: [M, D]; stored as BF16 (F32 when dtype is F32).
 * FP8 (current scaling, "Supported quantization recipes"): scales = device
 * fp32[3] = {s_X, s_Wup, s_Wdown}; H is stored bf16, its amax taken over the
 * stored values, and GEMM2 reads H quantised to e4m3 with inv = 448/amax;
 * s_H = amax/448 is written to h_scale_out (device fp32) when non-NULL.
 * F % T == 0, M % T == 0, M % num_chunks == 0.
 * Chunk arguments as in seq_chunk_gemm, for GEMM1's rows (tokens);
 * chunk_order NULL means the ring all-gather arrival order at `rank`: own
 * chunks first, then those of ranks rank-1, rank-2, ... (needs
 * num_chunks % T == 0; else ascending).
 * GEMM2 produces destination token ranges (T ranges of M/T rows) in
 * range_order (HOST, T entries) or, when NULL, rank+1, rank+2, ..., rank
 * (own range last), so finished ranges could leave first ("Collective
 * GEMMs", GEMM + reduce-scatter); range_done (DEVICE, T uint32, or NULL) is
 * set to epoch when a range is fully stored.
 * workspace >= tpm_workspace_bytes(TPM_OP_MLP_FWD, M, D, F, T, ...).
 */
int tp_mlp_fwd(int64_t M, int64_t D, int64_t F, int T, int rank,
               const void* X, const void* W_up_t, const void* W_down_t,
               int dtype, const float* scales, int act,
               void* Z_t, void* H_t, void* P_t, float* h_scale_out,
               int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
               const int32_t* range_order, uint32_t* range_done,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_mlp_bwd -- backward of tp_mlp_fwd ("Tensor and sequence parallelism",
 * sections "Derive column-parallel linear algebra" and "Derive row-parallel
 * linear algebra"; "Tensor parallelism", section "Code"):
 *
 *   dZ_t      = (dY . W_down,t^T) * act'(Z_t)    chunk-fed by dY rows
 *   dW_down,t = H_t^T . dY                       [F/T, D]
 *   dW_up,t   = X^T . dZ_t                       [D, F/T]
 *   dX_t      = dZ_t . W_up,t^T                  [M, D] partial (to be summed
 *                                                across ranks)
 * Inputs as in tp_mlp_fwd plus Z_t, H_t (saved forward values) and dY
 * [M, D]; dtype BF16 or F32.  dW outputs in dw_dtype (BF16 or F32; F32 only
 * with dtype F32), dX_t in dtype.  dZ_t lives in the workspace.
 * dy_chunk_order / dy_ready / epoch gate the rows of dY as in seq_chunk_gemm.
 * workspace >= tpm_workspace_bytes(TPM_OP_MLP_BWD, M, D, F, T, ...).
 */
int tp_mlp_bwd(int64_t M, int64_t D, int64_t F, int T, int rank,
               const void* X, const void* W_up_t, const void* W_down_t,
               const void* Z_t, const void* H_t, const void* dY,
               int dtype, int act,
               void* dW_up_t, void* dW_down_t, void* dX_t, int dw_dtype,
               int num_chunks, const int32_t* dy_chunk_order, const uint32_t* dy_ready, uint32_t epoch,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_linear_bwd -- backward of one sharded linear layer Y = X . W ("Tensor
 * and sequence parallelism", sections "Derive column-parallel linear
 * algebra" and "Derive row-parallel linear algebra"; the attention
 * projections of section "Pair adjacent transformer projections" are such
 * layers: W_qkv,t column-parallel, W_o,t row-parallel):
 *
 *   dW = X^T . dY     [K, N]   (the rank's weight gradient, W's shape)
 *   dX = dY . W^T     [M, K]   (column-parallel W: a full partial summed
 *                              across ranks; row-parallel W: the rank's
 *                              shard of the input gradient)
 *
 * X [M, K], W [K, N] (the shard as the rank stores it), dY [M, N]: dense
 * row-major device arrays, dtype BF16 or F32 (shapes the matrix-core kernel
 * does not take run both products on the predicated kernel).  dW in
 * dw_dtype (BF16 or F32; F32 only with dtype F32), dX in dtype.  The two
 * products read the same dY and are independent; for BF16 they run as one
 * launch whose work-groups take tiles of either product from per-XCD
 * queues, so that narrow shards (few output tiles each) fill the chip
 * together, and split-K is used only where one product's tiles are much
 * longer than the other's.  Results do not depend on which work-group
 * computes a tile.  Caller-owned device workspace of
 * >= tpm_workspace_bytes(TPM_OP_LINEAR_BWD, M, N, K, 1, 1, dtype) bytes
 * (control words and split-K partial sums).  M == 0 writes zeros to dW,
 * N == 0 zeros to dX (empty arrays may be null).  Errors: TPM_EINVAL (null
 * pointer to a non-empty array, negative size, bad dtype), TPM_EWORKSPACE (workspace too small),
 * nothing is enqueued on error.  Asynchronous on `stream`.
 */
int tp_linear_bwd(int64_t M, int64_t N, int64_t K,
                  const void* X, const void* W, const void* dY, int dtype,
                  void* dW, void* dX, int dw_dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * partial_reduce_seqshard -- the arithmetic a rank performs in the
 * reduce-scatter that follows a row-parallel GEMM ("Collective GEMMs in
 * Tensor Sequence Parallelism", section "Collective GEMMs (CGEMM)"; "Tensor
 * and sequence parallelism", section "Derive row-parallel linear algebra"):
 *
 *   out[i, j] = sum_{t=0}^{T-1} P_t[row0 + i, j],   0 <= i < M/T,
 *
 * with row0 = rank * M/T, or row0 = 0 when rank == -1 (each P_t then holds
 * only this rank's M/T rows, e.g. a receive buffer [T, M/T, D]).
 * P_t starts at partials + t * partial_stride elements and has leading
 * dimension ld >= D; out is [M/T, ldo >= D].  Sum in fp32 in ascending t,
 * one rounding at the end.  in_dtype/out_dtype: BF16 or F32.  M % T == 0.
 */
int partial_reduce_seqshard(int T, int64_t M, int64_t D, int rank,
                            const void* partials, int64_t partial_stride, int64_t ld, int in_dtype,
                            void* out, int64_t ldo, int out_dtype, void* stream);

/*
 * tp_gated_mlp_fwd -- rank `rank` of a T-way tensor-parallel gated MLP
 * ("Tensor and sequence parallelism", "Worked example: Partitioning an MLP
 * pair": the expansion and gate weights column-partitioned, the gated
 * activation applied locally, the contraction row-partitioned):
 *
 *   G_t = X . W_gate,t,  U_t = X . W_up,t      [M, F/T] each
 *   H_t = act(G_t) * U_t                        [M, F/T]  (act gates)
 *   P_t = H_t . W_down,t                        [M, D] partial
 *
 * X [M, D] bf16; W_gu_t [D, 2F/T] bf16 = [W_gate,t | W_up,t] (the rank's two
 * column shards side by side); W_down_t [F/T, D] bf16.  GU_t [M, 2F/T] bf16
 * or NULL receives [G_t | U_t] (saved for the backward); H_t [M, F/T] and
 * P_t [M, D] bf16.  Chunks, orders, flags and range_done as in tp_mlp_fwd.
 * dtype must be TPM_BF16.  All leading dimensions are the row widths.
 * workspace >= tpm_workspace_bytes(TPM_OP_GATED_MLP_FWD, M, D, F, T, ...)
 * (may be NULL when no flags are given: then no split-K).
 */
int tp_gated_mlp_fwd(int64_t M, int64_t D, int64_t F, int T, int rank,
                     const void* X, const void* W_gu_t, const void* W_down_t, int dtype, int act,
                     void* GU_t, void* H_t, void* P_t,
                     int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                     const int32_t* range_order, uint32_t* range_done,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_gated_mlp_bwd -- backward of tp_gated_mlp_fwd (chain rule through the
 * gate; column- and row-parallel layouts as in tp_mlp_bwd):
 *
 *   dH_t = dY . W_down,t^T;  dG_t = dH_t * U_t * act'(G_t);  dU_t = dH_t * act(G_t)
 *   dW_down,t = H_t^T . dY                      [F/T, D]
 *   dW_gu,t   = X^T . [dG_t | dU_t]             [D, 2F/T] = [dW_gate,t | dW_up,t]
 *   dX_t      = [dG_t | dU_t] . W_gu,t^T        [M, D] partial
 *
 * GU_t and H_t are the forward's saved values; dY [M, D] arrives in chunks
 * (dy_ready as in tp_mlp_bwd).  [dG_t | dU_t] is stored in bf16 in the
 * workspace before the two GEMMs that read it.  dw_dtype BF16 or F32.
 * workspace >= tpm_workspace_bytes(TPM_OP_GATED_MLP_BWD, M, D, F, T, ...).
 */
int tp_gated_mlp_bwd(int64_t M, int64_t D, int64_t F, int T, int rank,
                     const void* X, const void* W_gu_t, const void* W_down_t,
                     const void* GU_t, const void* H_t, const void* dY, int dtype, int act,
                     void* dW_gu_t, void* dW_down_t, void* dX_t, int dw_dtype,
                     int num_chunks, const int32_t* dy_chunk_order, const uint32_t* dy_ready, uint32_t epoch,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * MXFP8 block scaling ("Collective GEMMs in Tensor Sequence Parallelism",
 * section "Supported quantization recipes", MXFP8; the format is the OCP
 * Microscaling v1.0 one): an operand stored K-major ([rows, K], K contiguous)
 * as e4m3fn codes, each 32-element block of a row along K with one E8M0
 * scale 2^(E - 127).  The scales are passed in the layout gfx950's scaled
 * MFMA reads them: rows in groups of 32, each group one 128-byte record per
 * 128 elements of K holding 4 bytes (blocks 4s .. 4s+3) for each of its 32
 * rows.  tpm_mx_scales_bytes(rows, K) is the size of such an array (rows
 * padded to a multiple of 32); tpm_mx_swizzle_scales converts row-major
 * [rows, ld >= K/32] E8M0 bytes into it (padding rows get E = 0).  K must
 * be a multiple of 128.
 */
size_t tpm_mx_scales_bytes(int64_t rows, int64_t k);
int tpm_mx_swizzle_scales(int64_t rows, int64_t k, const uint8_t* src, int64_t ld, uint8_t* dst, void* stream);

/*
 * seq_chunk_gemm_mx -- seq_chunk_gemm with MXFP8 operands: A [M, lda >= K]
 * and B stored [N, ldb >= K] (op(B) = B^T), both e4m3 codes with their
 * block scales (layout above); fp32 accumulation on the scaled MFMA.
 * y_dtype BF16 or F32: Y = act(A . B^T); y_dtype FP8_E4M3: Y is written as
 * MXFP8 (codes [M, ldy >= N], y_scales in the layout above for K = N, blocks
 * of 32 output columns; N % 128 == 0), each block's scale exponent the
 * exponent field of its fp32 amax minus 8 (0 for a zero block) and each code
 * e4m3(v * 2^(127 - E)), nearest-even, saturating.  aux (optional, bf16
 * [M, ldaux >= N]) receives the pre-activation.  Chunks as seq_chunk_gemm.
 */
int seq_chunk_gemm_mx(int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, const uint8_t* a_scales,
                      const void* B, int64_t ldb, const uint8_t* b_scales,
                      void* Y, int64_t ldy, int y_dtype, uint8_t* y_scales,
                      int act, void* aux, int64_t ldaux,
                      int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_mlp_fwd_mx -- tp_mlp_fwd under MXFP8 block scaling: X [M, D] codes with
 * x_scales; W_up,t stored K-major [F/T, D] with w_up_scales; W_down,t stored
 * K-major [D, F/T] with w_down_scales.  GEMM1's epilogue writes H straight
 * to MXFP8 (H_t codes [M, F/T], h_scales of tpm_mx_scales_bytes(M, F/T)
 * bytes) from its fp32 result: the blocks are local, so there is no
 * tensor-wide amax and no separate quantisation pass.  Z_t (bf16, optional)
 * receives the pre-activation; P_t [M, D] bf16.  D and F/T multiples of 128.
 * Chunks, orders, flags and range_done as in tp_mlp_fwd.  workspace >=
 * tpm_workspace_bytes(TPM_OP_MX_MLP_FWD, M, D, F, T, ...) when flags are
 * given (else may be NULL).
 */
int tp_mlp_fwd_mx(int64_t M, int64_t D, int64_t F, int T, int rank,
                  const void* X, const uint8_t* x_scales, const void* W_up_t, const uint8_t* w_up_scales,
                  const void* W_down_t, const uint8_t* w_down_scales, int act,
                  void* Z_t, void* H_t, uint8_t* h_scales, void* P_t,
                  int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                  const int32_t* range_order, uint32_t* range_done,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_mlp_fwd_delayed -- the fp8 MLP forward under delayed scaling
 * ("Collective GEMMs in Tensor Sequence Parallelism", section "Supported
 * quantization recipes", FP8 with delayed scaling): X, W_up,t, W_down,t as
 * in tp_mlp_fwd's fp8 form (codes, weights stored K-major, scales =
 * device {sX, sWup, sWdown}); h_scale (device fp32) is H's dequantisation
 * factor fixed before the step.  GEMM1's epilogue writes H_t [M, F/T] as
 * e4m3 codes e4m3(act(Z) * fp32(1 / h_scale)), nearest-even, saturating, and
 * records max|act(Z)| (fp32 values) into h_amax_out (device, zeroed by the
 * call; NULL to skip); GEMM2 reads the codes with h_scale.  Z_t (bf16,
 * optional) receives the pre-activation.  Chunks, orders, flags and
 * range_done as in tp_mlp_fwd.  workspace >= tpm_workspace_bytes(
 * TPM_OP_FP8_DELAYED_MLP_FWD, M, D, F, T, ...) when flags or h_amax_out are
 * given.
 */
int tp_mlp_fwd_delayed(int64_t M, int64_t D, int64_t F, int T, int rank,
                       const void* X, const void* W_up_t, const void* W_down_t, const float* scales,
                       const float* h_scale, float* h_amax_out, int act,
                       void* Z_t, void* H_t, void* P_t,
                       int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                       const int32_t* range_order, uint32_t* range_done,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Delayed scaling's scale update: *scale_out = fp32(max(amax_history[0..n)) /
 * 448), or 1 when every entry is 0 (device pointers, one small kernel on
 * `stream`).  With h_amax_out of step k pointing at history[k % n], this
 * gives the h_scale of step k + 1. */
int tpm_fp8_delayed_scale(const float* amax_history, int n, float* scale_out, void* stream);

/*
 * tpm_cast_fp8 -- current-scaling cast of a bf16 matrix x [rows, ld >= cols]
 * to fp8 (dtype TPM_FP8_E4M3 or TPM_FP8_E5M2, largest value fmax 448 or
 * 57344): amax = max|x|, inv = fp32(fmax / amax), code = fp8(fp32(x * inv)),
 * nearest-even and saturating; *scale_out = fp32(amax / fmax) (device; both
 * factors 1 when amax = 0).  q [rows, ldq] and / or qt [cols, ldqt] (the
 * transpose) receive the codes (either may be NULL).  rows and cols
 * multiples of 16, ld % 8, ldq and ldqt % 16 == 0.  workspace >=
 * tpm_workspace_bytes(TPM_OP_CAST_FP8, ...) holds the amax.
 */
int tpm_cast_fp8(int64_t rows, int64_t cols, const void* x, int64_t ld, int dtype,
                 void* q, int64_t ldq, void* qt, int64_t ldqt, float* scale_out,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_mlp_bwd_fp8 -- tp_mlp_bwd in fp8 (hybrid recipe of "Collective GEMMs in
 * Tensor Sequence Parallelism", section "Supported quantization recipes":
 * activations and weights e4m3 with their forward scales, gradients e5m2
 * with current scaling):
 *   H_t [M, F/T] bf16 (the forward's) -> e4m3 transposed (current scaling,
 *     the codes the forward's GEMM2 read); X's codes transposed;
 *   dZ_t = (dYq . W_down,t^T) * act'(Z_t), chunk-fed by dY's rows, stored
 *     bf16, -> e5m2 (current scaling) and its transpose;
 *   dW_down,t = H_t^T . dYq,  dW_up,t = X^T . dZ_t,  dX_t = dZ_t . W_up,t^T.
 * dY [M, D]: dy_dtype TPM_BF16 -> cast here to e5m2 with current scaling
 * (every row must be resident: dy_ready must be NULL); TPM_FP8_E5M2 -> dY
 * holds e5m2 codes already quantised by their producers with the
 * dequantisation factor *dy_scale (device fp32), as an all-gather of
 * quantised gradients delivers them; its rows may then arrive in chunks:
 * num_chunks / dy_chunk_order / dy_ready / epoch as in seq_chunk_gemm (the
 * dZ GEMM waits per chunk; dY's transposed copy for dW_down is made after it).
 * X [M, D] e4m3 codes; W_up_t [D, F/T] and W_down_t [F/T, D] e4m3 codes in
 * the pages' layouts (the transposes of the forward's K-major copies);
 * scales = device fp32 {sX, sWup, sWdown}; Z_t bf16 (pre-activation).
 * dW_up_t [D, F/T], dW_down_t [F/T, D] in dw_dtype (BF16 or F32), dX_t
 * [M, D] bf16.  M, D and F/T multiples of 16.  workspace >=
 * tpm_workspace_bytes(TPM_OP_MLP_BWD_FP8, M, D, F, T, ...) holds the casts.
 */
int tp_mlp_bwd_fp8(int64_t M, int64_t D, int64_t F, int T, int rank,
                   const void* X, const void* W_up_t, const void* W_down_t, const float* scales,
                   const void* Z_t, const void* H_t, const void* dY, int dy_dtype, const float* dy_scale, int act,
                   void* dW_up_t, void* dW_down_t, void* dX_t, int dw_dtype,
                   int num_chunks, const int32_t* dy_chunk_order, const uint32_t* dy_ready, uint32_t epoch,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace needed by an operation (bytes).  For TPM_OP_MLP_FWD /
 * TPM_OP_MLP_BWD and the gated forms pass (M, N = D, K = F, T); for
 * TPM_OP_SEQ_CHUNK_GEMM and TPM_OP_LINEAR_BWD the sizes are (M, N, K)
 * and T is ignored. */
size_t tpm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int T, int num_chunks, int dtype);

/* Enqueue on `stream` a release store of `value` into the device word
 * `flag` (marks a chunk as landed after the copies enqueued before it). */
int tpm_signal_chunk(void* stream, uint32_t* flag, uint32_t value);

/*
 * tpm_write_chunks -- the side-stream writer of sequence-chunk arrival.  In
 * tensor-sequence parallelism the input of a column-parallel GEMM reaches a
 * rank as token chunks from its peers (the all-gather in front of the GEMM,
 * "Collective GEMMs in Tensor Sequence Parallelism", section "Collective
 * GEMMs (CGEMM)"); on one GPU a copy from a staging buffer stands in for the
 * peers' writes.  One kernel launch writes, for i = 0 .. num_chunks-1 and
 * chunk c = order[i], the bytes [c*chunk_bytes, (c+1)*chunk_bytes) of src
 * into the same range of dst (skipped when copy != NULL and copy[c] == 0:
 * a chunk already in place), and as soon as the whole chunk is written sets
 * ready[c] = epoch with a release store, so a chunk-gated GEMM can start on
 * chunk c while later chunks are still being written.
 *   dst, src   device, 16-byte aligned; chunk_bytes a multiple of 16.
 *   order      host, a permutation of 0 .. num_chunks-1 (<= TPM_MAX_CHUNKS).
 *   copy       host, num_chunks bytes indexed by chunk id, or NULL (copy all).
 *   ready      device, num_chunks words.
 *   counters   device, num_chunks words, zero before the first call; every
 *              call leaves them zero.  Calls that share counters must not
 *              overlap.
 * Work-groups: one per compute unit of the stream's CU mask (at most 64), or
 * 8 on a stream that may use every CU.  Run it on a stream whose CU mask is
 * disjoint from that of the consuming GEMM's stream: a writer work-group
 * dispatched to a CU held by a waiting GEMM work-group cannot start, and the
 * GEMM then ends with TPM_ETIMEOUT.
 * Errors: TPM_EINVAL (arguments), TPM_EHIP (launch).
 */
int tpm_write_chunks(void* dst, const void* src, int64_t chunk_bytes, int num_chunks, const int32_t* order,
                     const uint8_t* copy, uint32_t* ready, uint32_t epoch, uint32_t* counters, void* stream);

/* After synchronising the stream: TPM_OK, or TPM_ETIMEOUT if a chunk wait
 * of the last chunk-gated call on this workspace gave up (its error word
 * then holds one specific 32-bit value, which every chunk-gated call clears
 * before its kernels run; any other content reads as TPM_OK).  workspace:
 * device, at least its 2 KiB control block.  Blocking copy of one device
 * word; TPM_EWORKSPACE for NULL. */
int tpm_poll_device_error(const void* workspace);

/* Number of polls a device-side chunk wait makes before it gives up and
 * flags TPM_ETIMEOUT (default 1 << 22, a few seconds).  Process-wide. */
int tpm_set_wait_limit(uint32_t polls);

/* Thread-local description of the last error; never NULL. */
const char* tpm_last_error(void);

const char* tpm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPMLP_H */

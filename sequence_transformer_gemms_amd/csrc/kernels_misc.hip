// Bandwidth-bound kernels of the path and the fp32 correctness GEMM:
//   * sequence-sharded partial reduction (local arithmetic of the
//     reduce-scatter after a row-parallel GEMM: "Collective GEMMs in Tensor
//     Sequence Parallelism", section "Collective GEMMs (CGEMM)", GEMM +
//     reduce-scatter; "Tensor and sequence parallelism", section "Derive
//     row-parallel linear algebra": Y = sum_t Y_t)
//   * fp8 current scaling of the intermediate activation (FP8 current-scaling
//     recipe, "Supported quantization recipes")
//   * control-word initialisation and chunk-ready signalling
//   * an LDS-tiled FMA GEMM with predicated loads: the fp32 configuration,
//     and shapes, layouts or alignments the matrix-core kernel does not take.
#include "tpm_device.hpp"
#include "tpm_internal.hpp"

namespace tpm {

namespace {

// ------------------------------------------------------------- reduction
// out[i, :] = sum_{t=0}^{T-1} P_t[i, :] for i < rows, with the partials at
// partials + t * pstride.  One lane owns 8 bf16 (16 bytes) of one row: T
// sixteen-byte nontemporal loads, one in flight at a time (more per lane
// measured slower: many waves each with one load keep HBM busier than few
// waves with eight), fp32 sum in ascending t, one rounding to bf16, one
// 16-byte store.  1024-thread blocks, grid-stride over (row, 8-column
// group).
__global__ void __launch_bounds__(1024) reduce_bf16_vec(int T, int64_t rows, int64_t D8, const uint16_t* __restrict__ P,
                                                       int64_t pstride, int64_t ld, uint16_t* __restrict__ out,
                                                       int64_t ldo) {
  const int64_t total = rows * D8;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / D8;
    const int64_t c = (v - r * D8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const uint16_t* src = P + r * ld + c;
    for (int t = 0; t < T; ++t) {
      const i32x4 w = __builtin_nontemporal_load((const i32x4*)(src + (int64_t)t * pstride));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = (uint32_t)w[e];
        s[2 * e] += bf16_to_f32((uint16_t)(u & 0xFFFFu));
        s[2 * e + 1] += bf16_to_f32((uint16_t)(u >> 16));
      }
    }
    i32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (int)pack_bf16x2(s[2 * e], s[2 * e + 1]);
    __builtin_nontemporal_store(o, (i32x4*)(out + r * ldo + c));
  }
}

// General element-wise form: any D, any leading dimensions, fp32 or bf16 on
// either side (fp32 partials for the fp32 configuration).
__global__ void __launch_bounds__(256) reduce_scalar(int T, int64_t rows, int64_t D, const void* __restrict__ P,
                                                     int64_t pstride, int64_t ld, int in_f32, void* __restrict__ out,
                                                     int64_t ldo, int out_f32) {
  const int64_t total = rows * D;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / D;
    const int64_t c = v - r * D;
    float s = 0.f;
    for (int t = 0; t < T; ++t) {
      const int64_t off = (int64_t)t * pstride + r * ld + c;
      s += in_f32 ? ((const float*)P)[off] : bf16_to_f32(((const uint16_t*)P)[off]);
    }
    if (out_f32) ((float*)out)[r * ldo + c] = s;
    else ((uint16_t*)out)[r * ldo + c] = f32_to_bf16_rne(s);
  }
}

// --------------------------------------------------------- fp8 quantiser
// amax (fp32 bits, from the producing GEMM's epilogue) -> inv = 448/amax,
// s = amax/448 (both 1 when amax == 0); q = e4m3(fp32(h * inv)).
__global__ void __launch_bounds__(256) quant_e4m3(const uint16_t* __restrict__ h, int64_t M, int64_t N8, int64_t ldh,
                                                  const float* __restrict__ amax_p, uint8_t* __restrict__ q,
                                                  int64_t ldq, float* __restrict__ s_out) {
  const float amax = *amax_p;
  const float inv = amax > 0.f ? 448.0f / amax : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0 && s_out) *s_out = amax > 0.f ? amax / 448.0f : 1.0f;
  const int64_t total = M * N8;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total; v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / N8;
    const int64_t c = (v - r * N8) * 8;
    const i32x4 w = __builtin_nontemporal_load((const i32x4*)(h + r * ldh + c));
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)w[e];
      f[2 * e] = bf16_to_f32((uint16_t)(u & 0xFFFFu)) * inv;
      f[2 * e + 1] = bf16_to_f32((uint16_t)(u >> 16)) * inv;
    }
    *(uint2*)(q + r * ldq + c) = make_uint2(fp8x4<false>(f[0], f[1], f[2], f[3]), fp8x4<false>(f[4], f[5], f[6], f[7]));
  }
}

// ------------------------------------------- fp8 backward: amax, casts
// max |x| of a bf16 [rows, cols] matrix into *out (fp32 bits as uint32,
// non-negative floats order as integers; *out zeroed beforehand).  A lane
// keeps four 16-byte loads in flight: over the flat array when rows are
// contiguous (DENSE: ld = cols), else along whole rows.  Each work-group
// folds its 256 lanes' maxima through LDS and issues one atomic: atomics on
// the one word, one per wave of a grid sized to the matrix, had serialised
// into most of the kernel's time.
__device__ inline float absmax_bf16x8(float m, const i32x4& w) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)((uint32_t)w[e] & 0xFFFFu))));
    m = fmaxf(m, fabsf(bf16_to_f32((uint16_t)((uint32_t)w[e] >> 16))));
  }
  return m;
}

template <bool DENSE>
__global__ void __launch_bounds__(256) amax_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t c8, int64_t ld,
                                                 uint32_t* out) {
  __shared__ float wmax[4];
  float m = 0.f;
  if (DENSE) {
    const int64_t total = rows * c8;   // 16-byte groups
    for (int64_t v0 = (int64_t)blockIdx.x * 1024 + threadIdx.x; v0 < total; v0 += (int64_t)gridDim.x * 1024) {
      i32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t v = v0 + 256 * u;
        w[u] = v < total ? *(const i32x4*)(x + v * 8) : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) m = absmax_bf16x8(m, w[u]);
    }
  } else {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const uint16_t* xr = x + r * ld;
      for (int64_t c0 = threadIdx.x; c0 < c8; c0 += 4 * 256) {
        i32x4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t c = c0 + 256 * u;
          w[u] = c < c8 ? *(const i32x4*)(xr + c * 8) : i32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) m = absmax_bf16x8(m, w[u]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

// Current-scaling cast of a bf16 [rows, cols] matrix to fp8 (e4m3 or e5m2,
// largest value fmax): inv = fp32(fmax / amax), s = fp32(amax / fmax) (both 1
// when amax = 0), code = fp8(fp32(x * inv)).  Writes the codes row-major (q)
// and / or transposed (qt, [cols, rows]), 64 x 64 tiles through LDS.
template <bool E5M2>
__global__ void __launch_bounds__(256) cast_fp8_t(const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                  const float* __restrict__ amax_p, float fmax, uint8_t* __restrict__ q,
                                                  int64_t ldq, uint8_t* __restrict__ qt, int64_t ldqt, float* s_out) {
  __shared__ uint8_t tile[64][64 + 16];
  const float amax = *amax_p;
  const float inv = amax > 0.f ? fmax / amax : 1.0f;
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && s_out) *s_out = amax > 0.f ? amax / fmax : 1.0f;
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  {
    const int r = t >> 2, cg = (t & 3) * 16;
    const int64_t row = r0 + r, col = c0 + cg;
    if (row < rows && col < cols) {
      float f[16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const i32x4 v = *(const i32x4*)(x + row * ld + col + 8 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t u = (uint32_t)v[e];
          f[8 * h + 2 * e] = bf16_to_f32((uint16_t)(u & 0xFFFFu)) * inv;
          f[8 * h + 2 * e + 1] = bf16_to_f32((uint16_t)(u >> 16)) * inv;
        }
      }
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = fp8x4<E5M2>(f[4 * k], f[4 * k + 1], f[4 * k + 2], f[4 * k + 3]);
      if (q) *(uint4*)(q + row * ldq + col) = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
      for (int i = 0; i < 16; ++i) tile[r][cg + i] = (uint8_t)(w[i / 4] >> (8 * (i % 4)));
    }
  }
  if (!qt) return;
  __syncthreads();
  const int oc = t >> 2, rg = (t & 3) * 16;      // source column oc, source rows rg .. rg+15
  const int64_t col = c0 + oc, row = r0 + rg;
  if (col < cols && row < rows) {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i / 4] |= (uint32_t)tile[rg + i][oc] << (8 * (i % 4));
    *(uint4*)(qt + col * ldqt + row) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Byte transpose [rows, cols] -> [cols, rows] (fp8 codes; rows and cols
// multiples of 16), 128 x 128 tiles through LDS held as 32-bit words (row
// pitch padded to 33 words): each thread loads 4 x 16 bytes of input rows,
// then reads 16 words down one column of words (4 input columns x 16 input
// rows), transposes the four 4 x 4 byte blocks in registers and stores 4
// output rows of 16 bytes, 8 threads covering 128 bytes of an output row.
constexpr int kTrTile = 128, kTrPitch = kTrTile / 4 + 1;
__global__ void __launch_bounds__(256) transpose_u8(const uint8_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                    uint8_t* __restrict__ y, int64_t ldy) {
  __shared__ uint32_t tile[kTrTile * kTrPitch];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kTrTile, c0 = (int64_t)blockIdx.x * kTrTile;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = j * 256 + t;
    const int r = idx >> 3, cg = (idx & 7) * 16;
    if (r0 + r < rows && c0 + cg < cols) {
      const uint4 v = *(const uint4*)(x + (r0 + r) * ld + c0 + cg);
      uint32_t* d = tile + r * kTrPitch + cg / 4;
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
  }
  __syncthreads();
  const int g = t & 7, wc = t >> 3;  // input rows 16g .. 16g+15, input columns 4wc .. 4wc+3
  if (r0 + 16 * g < rows) {
    uint32_t out[4][4];                // [output row b][input rows 16g+4k .. +3]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t* src = tile + (16 * g + 4 * k) * kTrPitch + wc;
      const uint32_t w0 = src[0], w1 = src[kTrPitch], w2 = src[2 * kTrPitch], w3 = src[3 * kTrPitch];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        out[b][k] = ((w0 >> (8 * b)) & 0xFFu) | (((w1 >> (8 * b)) & 0xFFu) << 8) |
                    (((w2 >> (8 * b)) & 0xFFu) << 16) | (((w3 >> (8 * b)) & 0xFFu) << 24);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t oc = c0 + 4 * wc + b;
      if (oc < cols) *(uint4*)(y + oc * ldy + r0 + 16 * g) = make_uint4(out[b][0], out[b][1], out[b][2], out[b][3]);
    }
  }
}

// ------------------------------------------------------ chunk writer
// Side-stream writer of sequence-chunk arrival: for each chunk of the list,
// in list order, every work-group copies its share of the chunk (16-byte
// vectors, kWriterDepth in flight per lane), makes it visible device-wide, and
// counts itself in counters[c]; the last of the G work-groups to finish the
// chunk publishes ready[c] = epoch with a release store and resets the
// counter for the next call.
#ifndef TPM_WRITER_THREADS
#define TPM_WRITER_THREADS 1024
#endif
#ifndef TPM_WRITER_DEPTH
#define TPM_WRITER_DEPTH 8
#endif
constexpr int kWriterThreads = TPM_WRITER_THREADS;  // per work-group
constexpr int kWriterDepth = TPM_WRITER_DEPTH;      // 16-byte loads in flight per lane

__global__ void __launch_bounds__(kWriterThreads) write_chunks(const WriterParams p) {
  constexpr int NT = kWriterThreads, U = kWriterDepth;
  const int G = gridDim.x;
  const int64_t n16 = p.chunk_bytes / 16;
  const int64_t share = (n16 + G - 1) / G;
  const int64_t lo = (int64_t)blockIdx.x * share;
  const int64_t hi = lo + share < n16 ? lo + share : n16;
  for (int i = 0; i < p.n; ++i) {
    const int c = p.order[i];
    if (p.copy[c]) {
      const i32x4* __restrict__ src = (const i32x4*)(p.src + (int64_t)c * p.chunk_bytes);
      i32x4* __restrict__ dst = (i32x4*)(p.dst + (int64_t)c * p.chunk_bytes);
      int64_t v = lo + threadIdx.x;
      for (; v + (U - 1) * NT < hi; v += U * NT) {
        i32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = __builtin_nontemporal_load(src + v + u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u) dst[v + u * NT] = w[u];
      }
      for (; v < hi; v += NT) dst[v] = src[v];
    }
    // every wave's stores of the share have completed (the barrier waits for
    // them); one release by thread 0 then writes this XCD's L2 back, so
    // the share is in memory before it is counted
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t prev = __hip_atomic_fetch_add(p.counters + c, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (prev == (uint32_t)G - 1u) {
        __hip_atomic_store(p.counters + c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ready + c, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
}

// MXFP8 scales: row-major [rows, kblocks] E8M0 bytes -> the layout the
// scaled MFMA reads (mx_scale_offset); rows padded to a multiple of 32 get
// exponent 0.  One thread per destination byte.
__global__ void __launch_bounds__(256) mx_swizzle(const uint8_t* __restrict__ src, int64_t ld, int rows, int kblocks,
                                                  int64_t total, uint8_t* __restrict__ dst) {
  const int ksteps = kblocks / 4;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(t / kblocks), kb = (int)(t - (int64_t)row * kblocks);
    dst[mx_scale_offset((uint32_t)row, (uint32_t)kb, (uint32_t)ksteps)] = row < rows ? src[(int64_t)row * ld + kb] : 0;
  }
}

// Delayed scaling: scale = fp32(max(history) / 448), 1 when all are 0.
__global__ void __launch_bounds__(256) delayed_scale(const float* __restrict__ hist, int n, float* out) {
  __shared__ float red[256];
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, hist[i]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0] > 0.f ? red[0] / 448.0f : 1.0f;
}

__global__ void ctrl_init(uint32_t* w, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

__global__ void signal_flag(uint32_t* flag, uint32_t value) {
  __hip_atomic_store(flag, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ------------------------------------------------------------ fp32 GEMM
// 16 x 16 output tile per 256-thread block, K staged through LDS in steps
// of 16; one output element per thread, fp32 FMA accumulation in ascending k.
// Element e of an operand of element type dt (TPM dtype codes: 0 fp32,
// 1 bf16, 2 e4m3fn, 3 e5m2), widened to fp32.
__device__ inline float load_elem(const void* base, int dt, int64_t e) {
  switch (dt) {
    case 0: return ((const float*)base)[e];
    case 1: return bf16_to_f32(((const uint16_t*)base)[e]);
    case 2: return e4m3_to_f32(((const uint8_t*)base)[e]);
    default: return e5m2_to_f32(((const uint8_t*)base)[e]);
  }
}

// Predicated GEMM for shapes and layouts the matrix-core kernel does not
// take (any M, N, K >= 0, any leading dimensions and alignments, any element
// type on either side, fp8 in either layout): 16 x 16 output tile per
// work-group staged through LDS, one output per thread, fp32 FMA in
// ascending k.  Same epilogues as the matrix-core kernel: scale, FWD (aux
// receives the pre-activation, then act) or DACT (times act'(aux)), amax of
// the stored values, fp32 or bf16 output (nearest even).
__global__ void __launch_bounds__(256) gemm_generic_kernel(const GemmParams p, int trans_a, int trans_b) {
  __shared__ float As[16][17];
  __shared__ float Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = blockIdx.y * 16 + ty;
  const int col = blockIdx.x * 16 + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    {  // As[ty][tx] = op(A)[blockIdx.y*16 + ty][k0 + tx]
      const int r = blockIdx.y * 16 + ty, k = k0 + tx;
      float v = 0.f;
      if (r < p.M && k < p.K) v = load_elem(p.A, p.a_dt, trans_a ? (int64_t)k * p.lda + r : (int64_t)r * p.lda + k);
      As[ty][tx] = v;
    }
    {  // Bs[ty][tx] = op(B)[k0 + ty][blockIdx.x*16 + tx]
      const int k = k0 + ty, c = blockIdx.x * 16 + tx;
      float v = 0.f;
      if (k < p.K && c < p.N) v = load_elem(p.B, p.b_dt, trans_b ? (int64_t)c * p.ldb + k : (int64_t)k * p.ldb + c);
      Bs[ty][tx] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc = fmaf(As[ty][kk], Bs[kk][tx], acc);
    __syncthreads();
  }
  float stored = 0.f;
  if (row < p.M && col < p.N) {
    float s = 1.f;
    if (p.a_scale) s *= *p.a_scale;
    if (p.b_scale) s *= *p.b_scale;
    float v = acc * s;
    if (p.epi == EPI_DACT) {
      const float z = p.aux_f32 ? ((const float*)p.aux)[(int64_t)row * p.ldaux + col]
                                : bf16_to_f32(((const uint16_t*)p.aux)[(int64_t)row * p.ldaux + col]);
      v *= act_grad(z, p.act);
    } else {
      if (p.aux) {
        if (p.aux_f32) ((float*)p.aux)[(int64_t)row * p.ldaux + col] = v;
        else ((uint16_t*)p.aux)[(int64_t)row * p.ldaux + col] = f32_to_bf16_rne(v);
      }
      v = act_fwd(v, p.act);
    }
    if (p.y_f32) {
      ((float*)p.Y)[(int64_t)row * p.ldy + col] = v;
      stored = v;
    } else {
      const uint16_t b = f32_to_bf16_rne(v);
      ((uint16_t*)p.Y)[(int64_t)row * p.ldy + col] = b;
      stored = bf16_to_f32(b);
    }
  }
  if (p.amax) {
    float m = fabsf(stored);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((threadIdx.x & 63) == 0) atomicMax((unsigned int*)p.amax, __builtin_bit_cast(unsigned int, m));
  }
}

int grid_for(int64_t work, int per_block) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > 8192) b = 8192;
  return (int)b;
}

}  // namespace

hipError_t launch_reduce(int T, int64_t rows, int64_t D, const void* partials, int64_t pstride, int64_t ld, int in_f32,
                         void* out, int64_t ldo, int out_f32, hipStream_t s) {
  if (rows <= 0 || D <= 0) return hipSuccess;
  const bool vec = !in_f32 && !out_f32 && (D % 8 == 0) && (ld % 8 == 0) && (ldo % 8 == 0) && (pstride % 8 == 0) &&
                   (((uintptr_t)partials & 15) == 0) && (((uintptr_t)out & 15) == 0);
  if (vec) {
    const int64_t work = rows * (D / 8);
    reduce_bf16_vec<<<grid_for(work, 1024), 1024, 0, s>>>(T, rows, D / 8, (const uint16_t*)partials, pstride, ld,
                                                          (uint16_t*)out, ldo);
  } else {
    reduce_scalar<<<grid_for(rows * D, 256), 256, 0, s>>>(T, rows, D, partials, pstride, ld, in_f32, out, ldo, out_f32);
  }
  return hipGetLastError();
}

hipError_t launch_quant_e4m3(const uint16_t* h, int64_t M, int64_t N, int64_t ldh, const float* amax, uint8_t* q,
                             int64_t ldq, float* s_out, hipStream_t s) {
  const int64_t work = M * (N / 8);
  quant_e4m3<<<grid_for(work, 256), 256, 0, s>>>(h, M, N / 8, ldh, amax, q, ldq, s_out);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint32_t* out, hipStream_t s) {
  // at most 8 work-groups per CU
  if (ld == cols) {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((rows * (cols / 8) + 1023) / 1024, 2048));
    amax_bf16<true><<<grid, 256, 0, s>>>(x, rows, cols / 8, ld, out);
  } else {
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(rows, 2048));
    amax_bf16<false><<<grid, 256, 0, s>>>(x, rows, cols / 8, ld, out);
  }
  return hipGetLastError();
}

hipError_t launch_cast_fp8_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* amax, bool e5m2,
                             uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s_out, hipStream_t s) {
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64));
  if (e5m2) cast_fp8_t<true><<<grid, 256, 0, s>>>(x, rows, cols, ld, amax, 57344.0f, q, ldq, qt, ldqt, s_out);
  else cast_fp8_t<false><<<grid, 256, 0, s>>>(x, rows, cols, ld, amax, 448.0f, q, ldq, qt, ldqt, s_out);
  return hipGetLastError();
}

hipError_t launch_transpose_u8(const uint8_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* y, int64_t ldy,
                               hipStream_t s) {
  const dim3 grid((unsigned)((cols + kTrTile - 1) / kTrTile), (unsigned)((rows + kTrTile - 1) / kTrTile));
  transpose_u8<<<grid, 256, 0, s>>>(x, rows, cols, ld, y, ldy);
  return hipGetLastError();
}

hipError_t launch_delayed_scale(const float* history, int n, float* scale_out, hipStream_t s) {
  delayed_scale<<<1, 256, 0, s>>>(history, n, scale_out);
  return hipGetLastError();
}

hipError_t launch_mx_swizzle(const uint8_t* src, int64_t ld, int rows, int kblocks, uint8_t* dst, hipStream_t s) {
  const int64_t total = (int64_t)((rows + 31) / 32) * 32 * kblocks;
  mx_swizzle<<<grid_for(total, 256), 256, 0, s>>>(src, ld, rows, kblocks, total, dst);
  return hipGetLastError();
}

hipError_t launch_write_chunks(const WriterParams& p, int groups, hipStream_t s) {
  write_chunks<<<groups, kWriterThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_ctrl_init(uint32_t* words, int n, hipStream_t s) {
  ctrl_init<<<1, 256, 0, s>>>(words, n);
  return hipGetLastError();
}

hipError_t launch_signal(uint32_t* flag, uint32_t value, hipStream_t s) {
  signal_flag<<<1, 1, 0, s>>>(flag, value);
  return hipGetLastError();
}

hipError_t launch_gemm_generic(const GemmParams& p, bool trans_a, bool trans_b, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  dim3 grid((p.N + 15) / 16, (p.M + 15) / 16);
  gemm_generic_kernel<<<grid, 256, 0, s>>>(p, trans_a ? 1 : 0, trans_b ? 1 : 0);
  return hipGetLastError();
}

}  // namespace tpm

// Persistent MFMA GEMM for gfx950 with a group-ordered tile scheduler.
//
// Work: Y[M,N] = epilogue(op(A) . op(B)), the local GEMMs of a tensor-parallel
// rank ("Tensor and sequence parallelism": column-parallel Y_t = X W_t,
// row-parallel partial Y_t = X_t W_t, and their backward products).  Rows of
// Y are tokens for the forward GEMMs; they are cut into groups (sequence
// chunks for the all-gather side, destination token ranges for the
// reduce-scatter side, "Collective GEMMs in Tensor Sequence Parallelism",
// section "Collective GEMMs (CGEMM)").  Tiles are visited group by group in
// the caller's order; a tile of group g may wait for ready[g] >= epoch, and
// the last finished tile of group g publishes done[g] = epoch.
//
// Tile: 256 x 256 per work-group of 4 waves (2 x 2), each wave 128 x 128
// with v_mfma_f32_32x32x16_bf16 (16 accumulators of 16 floats).  K steps of
// 64 bf16 are staged global -> LDS with buffer_load ... lds (no VGPR
// staging), double-buffered (2 x 64 KB).  Operands stored K-major are read
// with ds_read_b128; operands stored MN-major (the pages' W[K,N], or X^T in
// weight gradients) are read with ds_read_b64_tr_b16, which transposes 16-bit
// elements across each 16-lane group.  The MFMA is issued with the operands
// swapped (B fragment as the matrix-core "A"), so each lane ends up holding
// four consecutive output columns of one row: stores are 8 or 16 bytes wide.
// fp8 (OCP e4m3fn) operands take the same 128-byte-per-row K-major staging
// (128 K elements per step) and v_mfma_f32_32x32x64_f8f6f4.
#include <type_traits>

#include "tpm_device.hpp"
#include "tpm_internal.hpp"

namespace tpm {

namespace {

constexpr int BM = kTileM, BN = kTileN;
constexpr int THREADS = 256;
constexpr int TILE_BYTES = 32768;            // one operand stage: 256 rows x 128 bytes of K

// K-major tile: 256 rows x 8 chunks of 16 bytes; chunk c of row r is stored
// at slot c ^ swz_k(r), which spreads the 32 rows read by one ds_read_b128
// over distinct banks.
__device__ __forceinline__ uint32_t swz_k(uint32_t r) { return (r ^ (r >> 3)) & 7u; }
// MN-major tile (bf16): 64 rows of K x 32 chunks; the four K rows read by one
// transposed read land in distinct bank groups.
__device__ __forceinline__ uint32_t swz_mn(uint32_t k) { return ((k & 3u) << 2) ^ ((k & 3u) << 1); }

struct Tile {
  int g, m0, m_end, n0;
};

__device__ __forceinline__ Tile map_tile(const GemmParams& p, int t) {
  const int G = gridDim.x;
  int L = t;
  if ((G & 7) == 0) {
    const int r = t / G;
    if ((r + 1) * G <= p.total_tiles) {
      const int s = t - r * G;
      L = r * G + (s & 7) * (G >> 3) + (s >> 3);  // tiles of one XCD are contiguous in L
    }
  }
  const int pos = L / p.tiles_per_group;
  const int q = L - pos * p.tiles_per_group;
  const int g = p.order[pos];
  const int band = q / (p.band_m * p.nt);
  const int rem_m = p.mt_per_group - band * p.band_m;
  const int gm = rem_m < p.band_m ? rem_m : p.band_m;
  const int idx = q - band * p.band_m * p.nt;
  const int mt = band * p.band_m + idx % gm;
  const int ntile = idx / gm;
  Tile tl;
  tl.g = g;
  const int gstart = g * p.group_rows;
  tl.m0 = gstart + mt * BM;
  const int gend = gstart + p.group_rows;
  tl.m_end = (tl.m0 + BM < gend) ? tl.m0 + BM : gend;
  tl.n0 = ntile * BN;
  return tl;
}

// Issue this thread's 8 sixteen-byte loads of one operand tile (256 x 64 bf16).
// kmajor: rows are the M (or N) index, 128 bytes of K each.
// otherwise: rows are K, 512 bytes (256 elements) of M or N each.
template <bool KMAJ, int ESZ>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int mn0, int mn_end,
                                           int k0, int K, char* lds_tile) {
  static_assert(KMAJ || ESZ == 2, "MN-major staging is bf16 only");
  constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t P = (uint32_t)(j * 256 + tid);
    uint32_t voff;
    if (KMAJ) {
      const uint32_t row = P >> 3;
      const uint32_t c = (P & 7u) ^ swz_k(row);
      const int k = k0 + (int)c * EPC;
      const bool ok = (mn0 + (int)row < mn_end) && (k < K);
      voff = ok ? (uint32_t)((int64_t)(mn0 + (int)row) * ld_bytes + (int64_t)k * ESZ) : kOOB;
    } else {
      const uint32_t row = P >> 5;
      const uint32_t c = (P & 31u) ^ swz_mn(row);
      const int mn = mn0 + (int)c * 8;
      const bool ok = (k0 + (int)row < K) && (mn < mn_end);
      voff = ok ? (uint32_t)((int64_t)(k0 + (int)row) * ld_bytes + (int64_t)mn * 2) : kOOB;
    }
    load16_to_lds(rs, voff, lds_tile + (j * 256 + wave * 64) * 16);
  }
}

// One 32 (rows) x 16 (K) bf16 fragment for a 32x32x16 MFMA operand:
// lane l holds row rb + l%32, K elements 8*(l/32) .. +7 of substep kk.
template <bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const char* lds_tile, int rb, int kk) {
  const int lane = threadIdx.x & 63;
  if (KMAJ) {
    const uint32_t r = (uint32_t)(rb + (lane & 31));
    const uint32_t c = (uint32_t)(2 * kk + (lane >> 5));
    const uint32_t addr = r * 128u + ((c ^ swz_k(r)) << 4);
    i32x4 v = *(const lds_i32x4*)((lds_void*)(lds_tile + addr));
    return __builtin_bit_cast(bf16x8, v);
  } else {
    const int g = lane >> 4, j = lane & 15;
    const int mn = rb + 16 * (g & 1) + 4 * (j & 3);
    const uint32_t byte = (uint32_t)mn * 2u;
    i16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t k = (uint32_t)(16 * kk + 8 * (g >> 1) + 4 * hh + (j >> 2));
      const uint32_t addr = k * 512u + (((byte >> 4) ^ swz_mn(k)) << 4) + (byte & 15u);
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_void*)(lds_tile + addr)));
    }
    i16x4 lo = h[0], hi = h[1];
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
}

// One 32 (rows) x 64 (K) fp8 fragment for a 32x32x64 MFMA operand (K-major
// tile only): lane l holds row rb + l%32, K bytes 32*(l/32) .. +31 of substep kk.
__device__ __forceinline__ i32x8 read_frag_fp8(const char* lds_tile, int rb, int kk) {
  const int lane = threadIdx.x & 63;
  const uint32_t r = (uint32_t)(rb + (lane & 31));
  const uint32_t c0 = (uint32_t)(4 * kk + 2 * (lane >> 5));
  const uint32_t sw = swz_k(r);
  const i32x4 lo = *(const lds_i32x4*)((lds_void*)(lds_tile + r * 128u + ((c0 ^ sw) << 4)));
  const i32x4 hi = *(const lds_i32x4*)((lds_void*)(lds_tile + r * 128u + (((c0 + 1u) ^ sw) << 4)));
  i32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ bool wait_group(const GemmParams& p, int g) {
  __shared__ int timed_out;
  if (threadIdx.x == 0) {
    int bad = 0;
    uint32_t polls = 0;
    for (;;) {
      const uint32_t v = __hip_atomic_load(p.ready + g, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM);
      if ((int32_t)(v - p.epoch) >= 0) break;
      if (__hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || ++polls > p.wait_limit) {
        __hip_atomic_fetch_or(p.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bad = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(4);
    }
    timed_out = bad;
  }
  __syncthreads();
  return timed_out != 0;
}

template <int N>
struct IC {
  static constexpr int value = N;
};
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<N, I + 1>(f);
  }
}

// Epilogue of four consecutive output columns (row, col..col+3) of one lane.
__device__ __forceinline__ void epi_quad(const GemmParams& p, f32x4 v, int row, int col, float& lmax) {
  if (p.epi == EPI_DACT) {
    f32x4 z;
    if (p.aux_f32) {
      z = *(const f32x4*)((const float*)p.aux + (int64_t)row * p.ldaux + col);
    } else {
      const uint2 zz = *(const uint2*)((const uint16_t*)p.aux + (int64_t)row * p.ldaux + col);
      z[0] = bf16_to_f32((uint16_t)(zz.x & 0xFFFFu));
      z[1] = bf16_to_f32((uint16_t)(zz.x >> 16));
      z[2] = bf16_to_f32((uint16_t)(zz.y & 0xFFFFu));
      z[3] = bf16_to_f32((uint16_t)(zz.y >> 16));
    }
    v[0] *= act_grad(z[0], p.act);
    v[1] *= act_grad(z[1], p.act);
    v[2] *= act_grad(z[2], p.act);
    v[3] *= act_grad(z[3], p.act);
  } else {
    if (p.aux) {
      if (p.aux_f32) {
        *(f32x4*)((float*)p.aux + (int64_t)row * p.ldaux + col) = v;
      } else {
        uint2 zz;
        zz.x = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        zz.y = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *(uint2*)((uint16_t*)p.aux + (int64_t)row * p.ldaux + col) = zz;
      }
    }
    if (p.act != ACT_NONE) {
      v[0] = act_fwd(v[0], p.act);
      v[1] = act_fwd(v[1], p.act);
      v[2] = act_fwd(v[2], p.act);
      v[3] = act_fwd(v[3], p.act);
    }
  }
  if (p.y_f32) {
    *(f32x4*)((float*)p.Y + (int64_t)row * p.ldy + col) = v;
    if (p.amax) lmax = fmaxf(lmax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  } else {
    const uint32_t b0 = f32_to_bf16_rne(v[0]), b1 = f32_to_bf16_rne(v[1]);
    const uint32_t b2 = f32_to_bf16_rne(v[2]), b3 = f32_to_bf16_rne(v[3]);
    uint2 yy;
    yy.x = b0 | (b1 << 16);
    yy.y = b2 | (b3 << 16);
    *(uint2*)((uint16_t*)p.Y + (int64_t)row * p.ldy + col) = yy;
    if (p.amax) {
      const float m01 = fmaxf(fabsf(bf16_to_f32((uint16_t)b0)), fabsf(bf16_to_f32((uint16_t)b1)));
      const float m23 = fmaxf(fabsf(bf16_to_f32((uint16_t)b2)), fabsf(bf16_to_f32((uint16_t)b3)));
      lmax = fmaxf(lmax, fmaxf(m01, m23));
    }
  }
}

template <bool FP8, bool AK, bool BKM>
__global__ void __launch_bounds__(THREADS, 1) gemm_kernel(const GemmParams p) {
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = 128 / ESZ;  // K elements per staged step (128 bytes per row)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = (wave >> 1) * 128;
  const int wn = (wave & 1) * 128;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, p.b_bytes);
  const int64_t lda_b = p.lda * ESZ, ldb_b = p.ldb * ESZ;
  const int nk = (p.K + KSTEP - 1) / KSTEP;
  float scale = 1.f;
  if (p.a_scale) scale *= *p.a_scale;
  if (p.b_scale) scale *= *p.b_scale;

  for (int t = blockIdx.x; t < p.total_tiles; t += gridDim.x) {
    const Tile tl = map_tile(p, t);
    if (p.ready) wait_group(p, tl.g);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // K loop over two LDS stages (A and B tiles of 32 KB each per stage).
    auto issue = [&](char* As, char* Bs, int k0) {
      issue_tile<AK, ESZ>(ra, lda_b, tl.m0, tl.m_end, k0, p.K, As);
      issue_tile<BKM, ESZ>(rb, ldb_b, tl.n0, p.N, k0, p.K, Bs);
    };
    // One K step, software-pipelined: the fragments of substep kk+1 are read
    // from LDS before the MFMAs of substep kk are issued (sched_barrier keeps
    // the scheduler from sinking them), and the global loads of the next
    // stage go out right after the first fragment reads.
    using Frag = typename std::conditional<FP8, i32x8, bf16x8>::type;
    constexpr int KSUB = FP8 ? 2 : 4;
    auto read_set = [&](const char* As, const char* Bs, int kk, Frag (&af)[4], Frag (&bfr)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (FP8) af[i] = read_frag_fp8(As, wm + 32 * i, kk);
        else af[i] = read_frag<AK>(As, wm + 32 * i, kk);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FP8) bfr[j] = read_frag_fp8(Bs, wn + 32 * j, kk);
        else bfr[j] = read_frag<BKM>(Bs, wn + 32 * j, kk);
      }
    };
    auto mfma_set = [&](const Frag (&af)[4], const Frag (&bfr)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (FP8)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0, 0, 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
    };
    // The restrict qualifiers tell the compiler that the two stages do not
    // overlap, so the fragment reads do not wait for the loads just issued.
    auto iteration = [&](const char* __restrict__ cur, char* __restrict__ nxt, int k_next) {
      Frag fa[2][4], fb[2][4];
      read_set(cur, cur + TILE_BYTES, 0, fa[0], fb[0]);
      if (k_next >= 0) issue(nxt, nxt + TILE_BYTES, k_next);
      static_for<KSUB>([&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        if constexpr (kk + 1 < KSUB) read_set(cur, cur + TILE_BYTES, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_set(fa[kk & 1], fb[kk & 1]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    issue(smem, smem + TILE_BYTES, 0);
    wait_vmem();
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      char* cur = smem + (kt & 1) * (2 * TILE_BYTES);
      char* nxt = smem + ((kt + 1) & 1) * (2 * TILE_BYTES);
      iteration(cur, nxt, kt + 1 < nk ? (kt + 1) * KSTEP : -1);
      wait_vmem();
      __syncthreads();
    }

    // ---- epilogue: lane holds rows m0+wm+32i+lane%32, columns
    //      n0+wn+32j+8q+4*(lane/32)+{0..3} in acc[i][j][4q..4q+3].  Every
    //      index is a compile-time constant so the accumulators stay in
    //      registers.
    float lmax = 0.f;
    static_for<64>([&](auto ijq) {
      constexpr int i = decltype(ijq)::value / 16;
      constexpr int j = (decltype(ijq)::value / 4) % 4;
      constexpr int q = decltype(ijq)::value % 4;
      const int row = tl.m0 + wm + 32 * i + (lane & 31);
      const int col = tl.n0 + wn + 32 * j + 8 * q + 4 * (lane >> 5);
      if (row < tl.m_end && col < p.N) {
        f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        epi_quad(p, v * scale, row, col, lmax);
      }
    });
    if (p.amax) {
      lmax = wave_max(lmax);
      if (lane == 0) atomicMax((unsigned int*)p.amax, __builtin_bit_cast(unsigned int, lmax));
    }
    if (p.done) {
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const uint32_t prev = atomicAdd(p.group_cnt + tl.g, 1u);
        if (prev + 1u == (uint32_t)p.tiles_per_group)
          __hip_atomic_store(p.done + tl.g, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmParams& p, bool a_kmajor, bool b_kmajor, int grid, hipStream_t s) {
  if (a_kmajor && !b_kmajor) gemm_kernel<false, true, false><<<grid, THREADS, 0, s>>>(p);
  else if (a_kmajor && b_kmajor) gemm_kernel<false, true, true><<<grid, THREADS, 0, s>>>(p);
  else if (!a_kmajor && !b_kmajor) gemm_kernel<false, false, false><<<grid, THREADS, 0, s>>>(p);
  else gemm_kernel<false, false, true><<<grid, THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmParams& p, bool a_kmajor, bool b_kmajor, int grid, hipStream_t s) {
  if (!a_kmajor || !b_kmajor) return hipErrorInvalidValue;  // rejected on the host first
  gemm_kernel<true, true, true><<<grid, THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace tpm

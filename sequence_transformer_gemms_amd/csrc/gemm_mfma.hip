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
// Tile: 256 x 256 per work-group.  bf16: 8 waves (2 x 4, two per SIMD),
// each wave 128 x 64 with v_mfma_f32_32x32x16_bf16 (8 accumulators of 16
// floats); fp8: 4 waves (2 x 2), each 128 x 128.  K steps of 64 bf16 (128
// fp8) are staged global -> LDS with buffer_load ... lds (no VGPR staging)
// through a ring of five 32 KB operand tiles, A two steps and B one step
// ahead of the step being computed.  Operands stored K-major are read
// with ds_read_b128; operands stored MN-major (the pages' W[K,N], or X^T in
// weight gradients) are read with ds_read_b64_tr_b16, which transposes 16-bit
// elements across each 16-lane group.  The MFMA is issued with the operands
// swapped (B fragment as the matrix-core "A"), so each lane ends up holding
// four consecutive output columns of one row: stores are 8 or 16 bytes wide.
// fp8 (OCP e4m3fn) operands take the same 128-byte-per-row K-major staging
// (128 K elements per step) and v_mfma_f32_32x32x64_f8f6f4.
//
// A launch may cut K into ranges: every tile's (few tiles), or only the
// tiles of the last tile columns when whole tiles would leave the last round
// of work-groups mostly empty; those units store fp32 partials, and a
// finalisation kernel sums them in a fixed order and runs the epilogue.
// The epilogue's common shapes are fixed at compile time per unit.
#include <type_traits>

#include "tpm_device.hpp"
#include "tpm_internal.hpp"

namespace tpm {

namespace {

constexpr int BM = kTileM, BN = kTileN;
constexpr int ROW_BYTES = 128;                   // K bytes per staged row (64 bf16 / 128 fp8)
constexpr int TILE_BYTES = 256 * ROW_BYTES;      // one operand tile of one K step: 32 KB
// LDS ring of five operand tiles: A of step k in tile (2k) mod 5, B of step k
// in tile (2k+1) mod 5 (steps counted from the start of the work unit).
// While step k is read, steps k+1 and A of k+2 are held or landing, so the A
// tiles are loaded two steps ahead and the B tiles one step ahead: about 1.5
// steps (96 KB) in flight per CU, which the global -> LDS path needs to keep
// up with the matrix cores (one step in flight delivers ~24 bytes/clock/CU,
// the 256 x 256 tile consumes 32).  The ring takes the whole 160 KB.
constexpr int NHALF = 5;
constexpr int RING_BYTES = NHALF * TILE_BYTES;
// two control words in the ring's last bytes, used only between work units
// (no operand load in flight): the pair kernel's ticket and the chunk wait's
// outcome
constexpr int CTRL_TICKET = RING_BYTES - 16, CTRL_WAIT = RING_BYTES - 32;
static_assert(ROW_BYTES == kStepBytes, "host-side K step");
// Wave layouts of the 256 x 256 tile: NW = 4 waves as 2 x 2 (128 x 128 per
// wave, one wave per SIMD) or NW = 8 waves as 2 x 4 (128 x 64 per wave, two
// waves per SIMD so that one issues MFMAs while the other waits).
template <int NW>
struct Layout {
  static constexpr int THREADS = 64 * NW;
  static constexpr int WAVES_N = NW / 2;              // waves along N
  static constexpr int NF = 4 * 2 / WAVES_N;          // 32-wide N fragments per wave (4 or 2)
  static constexpr int WN = 32 * NF;                  // wave tile width (128 or 64)
  static constexpr int LOADS = TILE_BYTES / (THREADS * 16);  // loads per thread per operand tile
  // Epilogue staging: each pass moves EPI_ROWS x 64 fp32 of the wave tile
  // through LDS, so every row segment a wave stores is 128 bytes of bf16.
  static constexpr int EPI_COLS = 64;
  static constexpr int EPI_ROWS = NW == 4 ? 128 : 64;  // 8 waves x 64 rows keeps the staging within 139 KB
  static constexpr int EPI_LD = EPI_COLS + 4;          // padded staging row (floats)
  static constexpr int EPI_WAVE_FLOATS = EPI_ROWS * EPI_LD;
  static constexpr int COL_PASSES = WN / EPI_COLS;
  static constexpr int PASSES = (128 / EPI_ROWS) * COL_PASSES;
  static constexpr int SMEM = RING_BYTES;
  static_assert(NW * EPI_WAVE_FLOATS * 4 <= CTRL_WAIT, "epilogue staging stays clear of the control words");
};

// K-major tile: 256 rows x 128 bytes of K, one 128-byte LDS line per row.
// The 16-byte chunk c of row r sits at position c ^ swz_k(r): the 16
// consecutive rows that one LDS cycle serves for a ds_read_b128 (same chunk)
// then cover every bank once (odd and even rows fall in the two halves of the
// 64 banks, and swz_k takes 8 distinct values over each half).  Global loads
// fill whole rows, so every row segment fetched is 128 bytes.
__device__ __forceinline__ uint32_t swz_k(uint32_t row) { return (row ^ (row >> 3)) & 7u; }
__device__ __forceinline__ uint32_t kmaj_offset(uint32_t row, uint32_t c) {
  return row * 128u + ((c ^ swz_k(row)) * 16u);
}
// MN-major tile (bf16): 64 rows of K x 32 chunks; the four K rows read by one
// transposed read land in distinct bank groups.
__device__ __forceinline__ uint32_t swz_mn(uint32_t k) { return ((k & 3u) << 2) ^ ((k & 3u) << 1); }

struct Tile {
  int g, m0, m_end, n0;
};

struct Unit {
  Tile tl;
  int split;   // K range: split of every tile, or the piece of a tail tile
  int tail;    // tail slot of the tile (0 .. tail_tiles - 1), -1 for a whole-range unit
};

// Work unit u -> (split, tile).  Units of one XCD (work-group ids congruent
// mod 8, which the dispatcher places round-robin on the 8 XCDs) are made
// contiguous in the logical order, and the logical order walks the groups
// (chunks / destination ranges) in the caller's order, each group in bands
// of band_m row tiles, so the 32 tiles an XCD works on at once share few
// A row panels and B column panels in its L2.  Splits of the K range are the
// outermost index, except in a chunk-gated GEMM, where they come right
// after the group: every unit of a chunk precedes the next chunk's, so the
// work-groups' first units are the earliest chunks' and later chunks are
// only waited for by units of a later round.  A tail split takes the last
// tail_cols tile columns out of every group: the whole tiles of the other
// columns come first, then the pieces of the tail tiles, piece-major (the
// tiles an XCD works on at once read the same K range), each piece in the
// group order.
__device__ __forceinline__ int xcd_logical(const GemmParams& p, int u) {
  const int G = gridDim.x;
  const int total = p.units;
  int L = u;
  if ((G & 7) == 0) {
    const int r = u / G;
    if ((r + 1) * G <= total) {
      const int s = u - r * G;
      L = r * G + (s & 7) * (G >> 3) + (s >> 3);
    }
  }
  return L;
}

// Position pos in the group order and index q within the group's tiles of
// tile columns col0 .. col0 + ncols - 1 -> tile.
__device__ __forceinline__ Tile tile_of(const GemmParams& p, int pos, int q, int ncols, int col0) {
  const int g = p.order[pos];
  const int band = q / (p.band_m * ncols);
  const int rem_m = p.mt_per_group - band * p.band_m;
  const int gm = rem_m < p.band_m ? rem_m : p.band_m;
  const int idx = q - band * p.band_m * ncols;
  const int mt = band * p.band_m + idx % gm;
  const int ntile = col0 + idx / gm;
  Tile tl;
  tl.g = g;
  const int gstart = g * p.group_rows;
  tl.m0 = gstart + mt * BM;
  const int gend = gstart + p.group_rows;
  tl.m_end = (tl.m0 + BM < gend) ? tl.m0 + BM : gend;
  tl.n0 = ntile * p.bn_out;
  return tl;
}

// Tail tile t (0 .. tail_tiles - 1, in the group order) -> tile.
__device__ __forceinline__ Tile tail_tile(const GemmParams& p, int t) {
  const int per_group = p.mt_per_group * p.tail_cols;
  const int pos = t / per_group;
  return tile_of(p, pos, t - pos * per_group, p.tail_cols, p.nt - p.tail_cols);
}

// Logical unit L (0 .. units - 1) -> (split, tile).  Whole tiles cover tile
// columns 0 .. nt_w - 1 (all of them without a tail split), tpg_w per group.
__device__ __forceinline__ Unit logical_unit(const GemmParams& p, int L) {
  Unit un;
  un.tail = -1;
  if (L >= p.tail_start) {
    // piece un.split of tail tile un.tail (splits == 1)
    const int j = L - p.tail_start;
    un.split = j / p.tail_tiles;
    un.tail = j - un.split * p.tail_tiles;
    un.tl = tail_tile(p, un.tail);
    return un;
  }
  int pos, q;
  if (p.ready) {
    const int per_group = p.tpg_w * p.splits;
    pos = L / per_group;
    const int rem = L - pos * per_group;
    un.split = rem / p.tpg_w;
    q = rem - un.split * p.tpg_w;
  } else {
    const int whole = p.tpg_w * p.num_groups;
    un.split = L / whole;
    L -= un.split * whole;
    pos = L / p.tpg_w;
    q = L - pos * p.tpg_w;
  }
  un.tl = tile_of(p, pos, q, p.nt_w, 0);
  return un;
}

__device__ __forceinline__ Unit map_unit(const GemmParams& p, int u) { return logical_unit(p, xcd_logical(p, u)); }

// One of the sixteen-byte loads per thread that stage an operand tile of
// one K step: thread t of the work-group fills LDS chunk P = j * THREADS + t.
// kmajor: rows are the M (or N) index, 128 bytes of K each.  Otherwise: rows
// are K (64 of them), 512 bytes (256 bf16) of M or N each.
// GATED (MN-major B only): the 256 tile columns are 32-column blocks taken
// alternately from the gate half and the up half of B = [W_gate | W_up]
// (up half at column up_off), both for output columns mn0 + 32 b' .. +31 of
// block pair b', so that the two N fragments of a wave (64 columns) hold the
// gate and up products of the same 32 output columns.
template <bool KMAJ, int ESZ, int THREADS, bool GATED = false>
__device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int mn0, int mn_end, int k0,
                                          int K, uint32_t lds_tile, int j, int up_off = 0) {
  static_assert(KMAJ || ESZ == 2, "MN-major staging is bf16 only");
  static_assert(!(GATED && KMAJ), "gated staging is MN-major");
  constexpr int EPC = 16 / ESZ;  // elements per 16-byte chunk
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t P = (uint32_t)(j * THREADS + tid);
  uint32_t voff;
  if (KMAJ) {
    const uint32_t row = P >> 3;
    const uint32_t c = (P & 7u) ^ swz_k(row);   // inverse of kmaj_offset
    const int k = k0 + (int)c * EPC;
    const bool ok = (mn0 + (int)row < mn_end) && (k < K);
    voff = ok ? (uint32_t)((int64_t)(mn0 + (int)row) * ld_bytes + (int64_t)k * ESZ) : kOOB;
  } else {
    const uint32_t row = P >> 5;
    const uint32_t c = (P & 31u) ^ swz_mn(row);
    int mn, src;
    if constexpr (GATED) {
      mn = mn0 + (int)(c >> 3) * 32 + (int)(c & 3u) * 8;   // output column of chunk c
      src = mn + (((c >> 2) & 1u) ? up_off : 0);
    } else {
      mn = mn0 + (int)c * 8;
      src = mn;
    }
    const bool ok = (k0 + (int)row < K) && (mn < mn_end);
    voff = ok ? (uint32_t)((int64_t)(k0 + (int)row) * ld_bytes + (int64_t)src * 2) : kOOB;
  }
  load16_to_lds(rs, voff, lds_tile + (uint32_t)((j * THREADS + wave * 64) * 16));
}

// LDS fragment reads through a restrict-qualified pointer parameter: the
// compiler then knows each read from its own scope, so it does not make the
// read wait for the LDS DMA writes in flight (which the kernel orders itself
// with vmcnt waits and barriers).
__device__ __forceinline__ i32x4 lds_read16(const char* __restrict__ p) {
  return *(const lds_i32x4*)((lds_void*)p);
}
// two transposed 8-byte reads 2048 bytes (four K rows of an MN-major tile)
// apart: a 32 x 16 bf16 MFMA fragment
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char* __restrict__ p) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_void*)p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)((lds_void*)(p + 2048)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// One 32 (rows) x 16 (K) bf16 fragment for a 32x32x16 MFMA operand:
// lane l holds row rb + l%32, K elements 8*(l/32) .. +7 of substep kk (0..3).
template <bool KMAJ>
__device__ __forceinline__ bf16x8 read_frag(const char* lds_tile, int rb, int kk) {
  const int lane = threadIdx.x & 63;
  if (KMAJ) {
    const uint32_t r = (uint32_t)(rb + (lane & 31));
    const uint32_t c = (uint32_t)(2 * kk + (lane >> 5));
    const uint32_t addr = kmaj_offset(r, c);
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
// tile only): lane l holds row rb + l%32 and, of substep kk's 64 K bytes
// (64*kk ..), bytes 16*h .. +15 in its first 16 bytes and 32 + 16*h .. +15
// in its last 16, h = l/32.  That is the order the matrix core takes K in
// (measured with block scales: bytes 0-15 of both lane halves form the
// first 32-element block, scaled by lane l%32's scale, bytes 16-31 the
// second, scaled by lane 32 + l%32's), so the MX blocks of 32 consecutive
// K elements in memory are the MFMA's blocks.
__device__ __forceinline__ i32x8 read_frag_fp8(const char* lds_tile, int rb, int kk) {
  const int lane = threadIdx.x & 63;
  const uint32_t r = (uint32_t)(rb + (lane & 31));
  const uint32_t c0 = (uint32_t)(4 * kk + (lane >> 5));
  const i32x4 lo = *(const lds_i32x4*)((lds_void*)(lds_tile + kmaj_offset(r, c0)));
  const i32x4 hi = *(const lds_i32x4*)((lds_void*)(lds_tile + kmaj_offset(r, c0 + 2u)));
  i32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// amax of a 256-thread work-group's values into *amax: one atomic per
// work-group (per-wave atomics on one address, thousands within a few
// microseconds, serialise).  Called by every thread.
__device__ __forceinline__ void block_amax(float* amax, float v) {
  __shared__ float wmax[4];
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    atomicMax((unsigned int*)amax, __builtin_bit_cast(unsigned int, m));
  }
}

__device__ __forceinline__ bool wait_group(const GemmParams& p, int g, char* smem) {
  volatile int& timed_out = *reinterpret_cast<volatile int*>(smem + CTRL_WAIT);
  if (threadIdx.x == 0) {
    int bad = 0;
    uint32_t polls = 0;
    for (;;) {
      // relaxed device-coherent read of the flag; see the acquire at kernel
      // start for why no cache invalidation is needed per chunk
      const uint32_t v = __hip_atomic_load(p.ready + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int32_t)(v - p.epoch) >= 0) break;
      if (__hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u || ++polls > p.wait_limit) {
        __hip_atomic_store(p.err, kErrTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Epilogue shapes fixed at compile time, so that the element-wise code tests
// no parameter per element: tested per element, the flags and pointers the
// general path needs do not all fit in scalar registers next to the main
// loop's, and the compiler keeps them in vector-register lanes that it reads
// back one at a time.  FK_FWD: forward with a bf16 output; FK_DACT: the
// activation-gradient epilogue (bf16 Z, bf16 output); FK_AUX: the
// pre-activation saved as bf16; FK_AMAX: the output's amax recorded; FK_RAW:
// the fp32 partial of a K range; FK_ANY: everything else, tested at run time.
enum { FK_ANY = 0, FK_FWD = 1, FK_AUX = 2, FK_AMAX = 4, FK_DACT = 8, FK_RAW = 16 };
// The shapes of the general epilogue loop (FK_RAW only when RAW) and of
// the DACT loop (Z preloaded; none unless DACT).  Each shape is another copy
// of the loop: the fp8 kernels, whose one wave per SIMD holds 128 x 128
// accumulators, take only the forward shapes, which keep them free of
// register spills.
template <bool RAW, class F>
__device__ __forceinline__ void with_fk_general(int fk, F&& f) {
  switch (fk) {
    case FK_FWD: f(IC<FK_FWD>{}); break;
    case FK_FWD | FK_AUX: f(IC<FK_FWD | FK_AUX>{}); break;
    case FK_FWD | FK_AMAX: f(IC<FK_FWD | FK_AMAX>{}); break;
    case FK_FWD | FK_AUX | FK_AMAX: f(IC<FK_FWD | FK_AUX | FK_AMAX>{}); break;
    case FK_RAW:
      if constexpr (RAW) {
        f(IC<FK_RAW>{});
        break;
      }
      [[fallthrough]];
    default: f(IC<FK_ANY>{}); break;
  }
}
template <bool DACT, class F>
__device__ __forceinline__ void with_fk_dact(int fk, F&& f) {
  if constexpr (DACT) {
    switch (fk) {
      case FK_DACT: f(IC<FK_DACT>{}); return;
      case FK_DACT | FK_AMAX: f(IC<FK_DACT | FK_AMAX>{}); return;
      default: break;
    }
  }
  f(IC<FK_ANY>{});
}

// Epilogue of eight consecutive output columns (row, col..col+7) of one lane.
// 8 consecutive values of a row-major bf16 or fp32 matrix
__device__ __forceinline__ void load_oct(const void* base, int64_t ld, bool f32, int row, int col, float (&v)[8]) {
  if (f32) {
    const f32x4* src = (const f32x4*)((const float*)base + (int64_t)row * ld + col);
    const f32x4 a = src[0], b = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
  } else {
    const i32x4 zz = *(const i32x4*)((const uint16_t*)base + (int64_t)row * ld + col);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_to_f32((uint16_t)((uint32_t)zz[e] & 0xFFFFu));
      v[2 * e + 1] = bf16_to_f32((uint16_t)((uint32_t)zz[e] >> 16));
    }
  }
}
__device__ __forceinline__ void store_oct(void* base, int64_t ld, bool f32, int row, int col, const float (&v)[8]) {
  if (f32) {
    f32x4* dst = (f32x4*)((float*)base + (int64_t)row * ld + col);
    dst[0] = (f32x4){v[0], v[1], v[2], v[3]};
    dst[1] = (f32x4){v[4], v[5], v[6], v[7]};
  } else {
    i32x4 yy;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      yy[e] = (int)pack_bf16x2(v[2 * e], v[2 * e + 1]);
    *(i32x4*)((uint16_t*)base + (int64_t)row * ld + col) = yy;
  }
}

// Gated forward epilogue of 8 output columns: g, u are the gate and up
// products; aux (optional) keeps [G | U], Y = act(G) * U.
template <int ACT>
__device__ __forceinline__ void epi_gated_oct(const GemmParams& p, const float (&g)[8], const float (&u)[8], int row,
                                              int col) {
  if (p.aux) {
    store_oct(p.aux, p.ldaux, p.aux_f32, row, col, g);
    store_oct(p.aux, p.ldaux, p.aux_f32, row, p.gu_off + col, u);
  }
  float h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = act_fwd_c<ACT>(g[e]) * u[e];
  store_oct(p.Y, p.ldy, p.y_f32, row, col, h);
}

// bf16 store of 8 consecutive output values, with their amax when AMAX.
template <bool AMAX>
__device__ __forceinline__ void store_y_bf16(const GemmParams& p, const float (&v)[8], int row, int col,
                                             float& lmax) {
  i32x4 yy;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    yy[e] = (int)w;
    if constexpr (AMAX)
      lmax = fmaxf(lmax, fmaxf(fabsf(bf16_to_f32((uint16_t)(w & 0xFFFFu))), fabsf(bf16_to_f32((uint16_t)(w >> 16)))));
  }
  *(i32x4*)((uint16_t*)p.Y + (int64_t)row * p.ldy + col) = yy;
}

// (ACT: the activation p.act, fixed at compile time by with_act; ZPRE: the
// DACT epilogue's bf16 Z of these 8 columns already loaded, in zpre; FK: the
// epilogue shape when fixed at compile time)
template <int ACT, bool ZPRE = false, int FK = FK_ANY>
__device__ __forceinline__ void epi_oct(const GemmParams& p, float (&v)[8], int row, int col, float& lmax,
                                        i32x4 zpre = i32x4{0, 0, 0, 0}) {
  if constexpr ((FK & FK_FWD) != 0) {
    if constexpr ((FK & FK_AUX) != 0) store_oct(p.aux, p.ldaux, false, row, col, v);  // pre-activation
    if constexpr (ACT != ACT_NONE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = act_fwd_c<ACT>(v[e]);
    }
    store_y_bf16<(FK & FK_AMAX) != 0>(p, v, row, col, lmax);
    return;
  }
  if constexpr ((FK & FK_DACT) != 0) {
    static_assert(ZPRE, "the DACT shape takes its Z preloaded");
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] *= act_grad_c<ACT>(bf16_to_f32((uint16_t)((uint32_t)zpre[e] & 0xFFFFu)));
      v[2 * e + 1] *= act_grad_c<ACT>(bf16_to_f32((uint16_t)((uint32_t)zpre[e] >> 16)));
    }
    store_y_bf16<(FK & FK_AMAX) != 0>(p, v, row, col, lmax);
    return;
  }
  if (p.epi == EPI_DGATED) {
    // v = dH; aux = [G | U]: Y[:, col] = dG = dH U act'(G), Y[:, N + col] = dU = dH act(G)
    float g[8], u[8], du[8];
    load_oct(p.aux, p.ldaux, p.aux_f32, row, col, g);
    load_oct(p.aux, p.ldaux, p.aux_f32, row, p.gu_off + col, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      du[e] = v[e] * act_fwd_c<ACT>(g[e]);
      v[e] = v[e] * u[e] * act_grad_c<ACT>(g[e]);
    }
    store_oct(p.Y, p.ldy, p.y_f32, row, p.gu_off + col, du);
  } else if (p.epi == EPI_DACT) {
    float z[8];
    if constexpr (ZPRE) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[2 * e] = bf16_to_f32((uint16_t)((uint32_t)zpre[e] & 0xFFFFu));
        z[2 * e + 1] = bf16_to_f32((uint16_t)((uint32_t)zpre[e] >> 16));
      }
    } else if (p.aux_f32) {
      const f32x4* src = (const f32x4*)((const float*)p.aux + (int64_t)row * p.ldaux + col);
      const f32x4 z0 = src[0], z1 = src[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) { z[e] = z0[e]; z[4 + e] = z1[e]; }
    } else {
      const i32x4 zz = *(const i32x4*)((const uint16_t*)p.aux + (int64_t)row * p.ldaux + col);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[2 * e] = bf16_to_f32((uint16_t)((uint32_t)zz[e] & 0xFFFFu));
        z[2 * e + 1] = bf16_to_f32((uint16_t)((uint32_t)zz[e] >> 16));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= act_grad_c<ACT>(z[e]);
  } else {
    if (p.aux) {
      if (p.aux_f32) {
        f32x4* dst = (f32x4*)((float*)p.aux + (int64_t)row * p.ldaux + col);
        dst[0] = (f32x4){v[0], v[1], v[2], v[3]};
        dst[1] = (f32x4){v[4], v[5], v[6], v[7]};
      } else {
        i32x4 zz;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          zz[e] = (int)pack_bf16x2(v[2 * e], v[2 * e + 1]);
        *(i32x4*)((uint16_t*)p.aux + (int64_t)row * p.ldaux + col) = zz;
      }
    }
    if constexpr (ACT != ACT_NONE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = act_fwd_c<ACT>(v[e]);
    }
  }
  if (p.y_f32) {
    f32x4* dst = (f32x4*)((float*)p.Y + (int64_t)row * p.ldy + col);
    dst[0] = (f32x4){v[0], v[1], v[2], v[3]};
    dst[1] = (f32x4){v[4], v[5], v[6], v[7]};
    if (p.amax) {
#pragma unroll
      for (int e = 0; e < 8; ++e) lmax = fmaxf(lmax, fabsf(v[e]));
    }
  } else {
    i32x4 yy;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      const uint32_t b0 = w & 0xFFFFu, b1 = w >> 16;
      yy[e] = (int)w;
      if (p.amax) lmax = fmaxf(lmax, fmaxf(fabsf(bf16_to_f32((uint16_t)b0)), fabsf(bf16_to_f32((uint16_t)b1))));
    }
    *(i32x4*)((uint16_t*)p.Y + (int64_t)row * p.ldy + col) = yy;
  }
}

// One work unit (a K range of one output tile) of the GEMM p, staged
// through the work-group's LDS block `smem` (Layout<NW>::SMEM bytes).
template <bool FP8, bool AK, bool BKM, int NW, bool GATED = false, bool MX = false, int F8F = 0,
          bool BAR_BASES = true>
__device__ __forceinline__ void run_unit(const GemmParams& p, const Unit& un, char* __restrict__ smem) {
  // fp8 formats of the MFMA operands (0 e4m3, 1 e5m2): the first operand
  // is the B fragment, the second the A fragment
  constexpr int FMT0 = (F8F >> 1) & 1, FMT1 = F8F & 1;
  static_assert(!GATED || (!FP8 && !BKM && NW == 8), "gated: bf16, MN-major B, 8 waves (two N fragments)");
  static_assert(!MX || (FP8 && AK && BKM), "MXFP8: fp8 operands stored K-major");
  using LY = Layout<NW>;
  constexpr int THREADS = LY::THREADS, LOADS = LY::LOADS, NF = LY::NF;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int KSTEP = ROW_BYTES / ESZ;  // K elements per staged step
  constexpr int KSUB = FP8 ? 1 : 2;        // MFMA substeps per K step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int wm = (wave / LY::WAVES_N) * 128;
  const int wn = (wave % LY::WAVES_N) * LY::WN;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.B, p.b_bytes);
  // MXFP8 block scales (reads past the end of a scale array return zeros,
  // which only happens for rows or K steps whose operand data are zeros too)
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(MX ? (const void*)p.a_mx : p.A, MX ? p.a_mx_bytes : 0u);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(MX ? (const void*)p.b_mx : p.B, MX ? p.b_mx_bytes : 0u);
  const int64_t lda_b = p.lda * ESZ, ldb_b = p.ldb * ESZ;
  const int nk = (p.K + KSTEP - 1) / KSTEP;
  float scale = 1.f;
  if (p.a_scale) scale *= *p.a_scale;
  if (p.b_scale) scale *= *p.b_scale;

  {
    const Tile& tl = un.tl;
    // K steps [kbeg, kend) of this split or tail piece
    const int per = un.tail >= 0 ? p.tail_ksteps : p.ksteps_per_split;
    const int kbeg = un.split * per;
    const int kend = min(nk, kbeg + per);
    const int nks = kend - kbeg;
    __syncthreads();  // the previous tile's epilogue staging is done with the LDS
    if (p.ready) wait_group(p, tl.g, smem);

    f32x16 acc[4][NF];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    using Frag = typename std::conditional<FP8, i32x8, bf16x8>::type;
    // Ring tiles as byte offsets from smem.  A step's tiles are two slots
    // (mod 5) after the previous step's, so the loop carries the offsets of
    // the step being loaded (ld_a, ld_b) and of the step read next (rd_a,
    // rd_b) and advances them by one add and one select each.  DMA
    // destinations are 32-bit LDS addresses: dma_w is this wave's 1 KB slice
    // of a load (lane i writes 16 bytes at 16 i).
    const uint32_t dma_w = lds_address(smem) + (uint32_t)wave * 1024u;
    auto next_step = [](uint32_t o) {
      o += 2u * TILE_BYTES;
      return o >= (uint32_t)RING_BYTES ? o - (uint32_t)RING_BYTES : o;
    };
    uint32_t ld_a = 0u, ld_b = (uint32_t)TILE_BYTES;  // step 0: tiles 0 and 1

    // ---- per-lane address parts, fixed for the whole unit.
    // LDS reads.  K-major tile, fragment of rows wbase + 32 i, chunk
    // c = 2 kk + lane/32 (bf16; fp8: 4 kk + lane/32 and + 2): with
    // l = lane % 32 the swizzled position is (lane/32 ^ s(l)) ^ K for a
    // constant K in {0, 2, 4, 6} (the fragment parity flips bit 2), so the
    // address is wbase*128 + 4096 i + kpart[K/2].  MN-major tile, fragment
    // of columns wbase + 32 i: the K rows a lane reads differ by constants
    // (8192 kk + 2048 hh), so the address is mpart(i) + that constant.
    // (the thread index passes through an empty asm statement so that these
    // values are computed per unit instead of being hoisted to the kernel
    // start, where in the pair kernel they would stay live through the
    // other GEMM's loop)
    uint32_t tid_u = (uint32_t)tid;
    asm volatile("" : "+v"(tid_u));
    const uint32_t lane_u = tid_u & 63u;
    const uint32_t l32 = lane_u & 31u;
    const uint32_t p0 = (lane_u >> 5) ^ (((l32 & 7u) ^ (l32 >> 3)) & 7u);
    uint32_t kpart[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) kpart[q] = l32 * 128u + ((p0 ^ (2u * (uint32_t)q)) * 16u);
    const uint32_t g4 = lane_u >> 4, j16 = lane_u & 15u;
    const uint32_t klane = (8u * (g4 >> 1) + (j16 >> 2)) * 512u + 8u * (j16 & 1u);
    const uint32_t mlo = 2u * (g4 & 1u) + ((j16 & 3u) >> 1);
    const uint32_t msw = swz_mn(j16 >> 2);
    auto mpart = [&](int wbase, int i) {
      return klane + (((((uint32_t)wbase >> 3) + 4u * (uint32_t)i + mlo) ^ msw) << 4);
    };
    // A step's read offsets (bytes from smem): K-major: o[q] = tile +
    // wbase*128 + kpart[q]; MN-major: o[i] = tile + mpart(wbase, i).  Every
    // LDS read address is formed as smem + offset, so that the compiler sees
    // each read based on the restrict-qualified LDS block (with that
    // provenance it does not drain the in-flight LDS DMA before a read).
    struct Bases {
      uint32_t o[4];
    };
    auto bases = [&](uint32_t tile, auto kmc, int wbase, int nfr) {
      Bases b;
      if constexpr (decltype(kmc)::value) {
#pragma unroll
        for (int q = 0; q < 4; ++q) b.o[q] = tile + (uint32_t)wbase * 128u + kpart[q];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) b.o[i] = i < nfr ? tile + mpart(wbase, i) : tile;
      }
      return b;
    };
    auto frag = [&](const Bases& b, auto kmc, int i, int kk) -> Frag {
      if constexpr (FP8) {
        const int q = (2 * kk) ^ (2 * (i & 1));
        const i32x4 lo = lds_read16(smem + b.o[q] + 4096 * i);
        const i32x4 hi = lds_read16(smem + b.o[q ^ 1] + 4096 * i);
        return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else if constexpr (decltype(kmc)::value) {
        const int q = kk ^ (2 * (i & 1));
        return __builtin_bit_cast(bf16x8, lds_read16(smem + b.o[q] + 4096 * i));
      } else {
        return lds_read_tr_pair(smem + b.o[i] + 8192 * kk);
      }
    };
    auto step_bases = [&](uint32_t tile_a, uint32_t tile_b, Bases& ba, Bases& bb) {
      ba = bases(tile_a, IC<AK>{}, wm, 4);
      bb = bases(tile_b, IC<BKM>{}, wn, NF);
    };

    // DMA loads.  Load j of an operand tile stages LDS chunk j*THREADS + tid.
    // In a full tile (every row of the operand tile inside the matrix) and a
    // full K step, its global offset is a per-lane part fixed for the unit
    // plus a uniform part (row block of load j, K position of the step), which
    // goes into the scalar offset: no vector arithmetic per load.  Other steps
    // (the last one of a ragged K, those past the end of the split) and tiles
    // that cross the matrix edge take the checked form (issue_one).
    const bool a_full = tl.m0 + BM <= tl.m_end;
    const bool b_full = tl.n0 + (GATED ? BN / 2 : BN) <= p.N;
    auto lane_off = [&](auto kmc, int64_t ld_bytes, int mn0, int par, auto gc, int up_off) -> uint32_t {
      if constexpr (decltype(kmc)::value) {
        // K-major: row block tid/8, chunk (tid%8) ^ swz_k(row); the row's
        // bits 3-5 come from tid/64 and, with 4 waves, from load j's parity
        uint32_t c = (tid_u & 7u) ^ ((tid_u >> 3) & 7u) ^ ((tid_u >> 6) & 7u);
        if (THREADS == 256) c ^= 4u * (uint32_t)par;
        return (uint32_t)(((int64_t)(tid_u >> 3)) * ld_bytes) + c * 16u;
      } else {
        // MN-major (bf16): K row tid/32 (plus the load's row block), chunk
        // (tid%32) ^ swz_mn(row % 4)
        const uint32_t c = (tid_u & 31u) ^ swz_mn((tid_u >> 5) & 3u);
        int mn, src;
        if constexpr (decltype(gc)::value) {
          mn = mn0 + (int)(c >> 3) * 32 + (int)(c & 3u) * 8;
          src = mn + (((c >> 2) & 1u) ? up_off : 0);
        } else {
          mn = mn0 + (int)c * 8;
          src = mn;
        }
        return (uint32_t)(((int64_t)(tid_u >> 5)) * ld_bytes + (int64_t)src * 2);
      }
    };
    uint32_t va[2], vb[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      va[par] = lane_off(IC<AK>{}, lda_b, tl.m0, par, IC<false>{}, 0);
      vb[par] = lane_off(IC<BKM>{}, ldb_b, tl.n0, par, IC<GATED>{}, p.gu_off);
    }
    // uniform part of load j of step k (full steps only)
    auto uni_off = [&](auto kmc, int64_t ld_bytes, int mn0, int j, int k) -> uint32_t {
      const int k0 = (kbeg + k) * KSTEP;
      if constexpr (decltype(kmc)::value)
        return (uint32_t)((int64_t)(mn0 + j * (THREADS / 8)) * ld_bytes + (int64_t)k0 * ESZ);
      else
        return (uint32_t)((int64_t)(k0 + j * (THREADS / 32)) * ld_bytes);
    };
    // Load L (0 .. 2*LOADS-1: A loads, then B loads) of K step k of this
    // split into its ring tile.  Steps past the end of the split load zeros
    // (out-of-range offsets) into ring tiles that no later step of this unit
    // reads, so the issue pattern and the load counts are the same for every
    // step.  FAST: both operand tiles are full and the step is full and
    // inside the split (see above).
    // The tiles are those of ld_a / ld_b, which hold step k's.
    auto load_one = [&](int L, int k, auto fc) {
      constexpr bool FAST = decltype(fc)::value;
      if (L < LOADS) {
        if constexpr (FAST)
          load16_to_lds_s(ra, va[L & 1], uni_off(IC<AK>{}, lda_b, tl.m0, L, k),
                          dma_w + ld_a + (uint32_t)(L * THREADS * 16));
        else
          issue_one<AK, ESZ, THREADS>(ra, lda_b, tl.m0, tl.m_end, k < nks ? (kbeg + k) * KSTEP : p.K, p.K,
                                      lds_address(smem) + ld_a, L);
      } else {
        const int j = L - LOADS;
        if constexpr (FAST)
          load16_to_lds_s(rb, vb[j & 1], uni_off(IC<BKM>{}, ldb_b, tl.n0, j, k),
                          dma_w + ld_b + (uint32_t)(j * THREADS * 16));
        else
          issue_one<BKM, ESZ, THREADS, GATED>(rb, ldb_b, tl.n0, p.N, k < nks ? (kbeg + k) * KSTEP : p.K, p.K,
                                              lds_address(smem) + ld_b, j, p.gu_off);
      }
    };
    // fragment r of a set in the order the MFMAs first need them: A0, B0..B(NF-1), A1, A2, A3
    auto read_one = [&](const Bases& sa, const Bases& sb, int kk, int r, Frag (&af)[4], Frag (&bfr)[NF]) {
      if (r == 0 || r > NF) {
        const int i = r == 0 ? 0 : r - NF;
        af[i] = frag(sa, IC<AK>{}, i, kk);
      } else {
        const int j = r - 1;
        bfr[j] = frag(sb, IC<BKM>{}, j, kk);
      }
    };
    auto mfma_row = [&](const Frag& a, const Frag (&bfr)[NF], f32x16 (&accrow)[NF]) {
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        if constexpr (FP8)
          accrow[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], a, accrow[j], 0, 0, 0, 0, 0, 0);
        else
          accrow[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], a, accrow[j], 0, 0, 0);
      }
    };
    // During step k the loads of step k+2 are issued: A's in the first two
    // phases (into the tile B of step k-1 left), B's right after the barrier
    // that frees step k's tiles (into A of step k's).  Each part's loads are
    // spread evenly over the MFMAs of its phase, so that no gap between two
    // MFMAs holds more than one load's scalar set-up (with one wave per SIMD
    // a gap longer than an MFMA's own duration idles the matrix core).
    constexpr int LA0 = LOADS / 2, LA1 = LOADS - LOADS / 2;
    // MXFP8: the scale dwords of K step s for this lane's fragments (4 rows
    // of A, NF of B; bytes = the step's four 32-element blocks), and the same
    // shifted right by 8 bytes for lanes 32-63, which hold the second 32 K
    // elements of each 64-element MFMA: byte 0 then scales substep 0 and
    // byte 2 substep 1 for every lane (op_sel 0 / 2).
    int sa_next[4] = {0, 0, 0, 0}, sb_next[NF] = {}, sa_cur[4] = {0, 0, 0, 0}, sb_cur[NF] = {};
    auto load_scales = [&](int s) {
      if constexpr (MX) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sa_next[i] = (int)__builtin_amdgcn_raw_buffer_load_b32(
              rsa, mx_scale_offset((uint32_t)(tl.m0 + wm + 32 * i + (lane & 31)), 4u * (uint32_t)s, (uint32_t)p.mx_steps),
              0, 0);
#pragma unroll
        for (int j = 0; j < NF; ++j)
          sb_next[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(
              rsb, mx_scale_offset((uint32_t)(tl.n0 + wn + 32 * j + (lane & 31)), 4u * (uint32_t)s, (uint32_t)p.mx_steps),
              0, 0);
      }
    };
    auto take_scales = [&]() {
      if constexpr (MX) {
        const uint32_t h8 = 8u * (uint32_t)(lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) sa_cur[i] = (int)((uint32_t)sa_next[i] >> h8);
#pragma unroll
        for (int j = 0; j < NF; ++j) sb_cur[j] = (int)((uint32_t)sb_next[j] >> h8);
      }
    };
    // MFMAs of accumulator rows I0 .. I0+NI-1 from one fragment set, with the
    // reads R0 .. R0+NR-1 of the next set (substep rkk of bases rsa / rsb)
    // one after each MFMA and the loads L0 .. L0+NL-1 of K step kl after
    // every NM/NL-th MFMA.
    auto mfma_rows = [&](auto i0c, auto nic, auto l0c, auto nlc, const Frag (&fa)[4], const Frag (&fb)[NF], int kl,
                         auto fastc, auto r0c, auto nrc, const Bases& rsa, const Bases& rsb, int rkk, Frag (&rfa)[4],
                         Frag (&rfb)[NF], auto opc) {
      constexpr int OPS = decltype(opc)::value;  // MX: byte of the scale dwords (0: substep 0, 2: substep 1)
      constexpr int I0 = decltype(i0c)::value, NI = decltype(nic)::value;
      constexpr int L0 = decltype(l0c)::value, NL = decltype(nlc)::value;
      constexpr int R0 = decltype(r0c)::value, NR = decltype(nrc)::value;
      constexpr int NM = NI * NF;
      static_for<NI>([&](auto ic) {
        constexpr int ii = decltype(ic)::value;
        static_for<NF>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          constexpr int m = ii * NF + j;
          if constexpr (MX)
            acc[I0 + ii][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[I0 + ii], acc[I0 + ii][j], 0, 0,
                                                                              OPS, sb_cur[j], OPS, sa_cur[I0 + ii]);
          else if constexpr (FP8)
            acc[I0 + ii][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[I0 + ii], acc[I0 + ii][j], FMT0,
                                                                              FMT1, 0, 0, 0, 0);
          else
            acc[I0 + ii][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[I0 + ii], acc[I0 + ii][j], 0, 0, 0);
          static_for<NR>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            if constexpr (r * NM / NR == m) read_one(rsa, rsb, rkk, R0 + r, rfa, rfb);
          });
          static_for<NL>([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            if constexpr (l * NM / NL == m) load_one(L0 + l, kl, fastc);
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // Wait until this thread's loads of the next step have landed (only the
    // A loads of the step after it, issued last, may still be in flight: the
    // NPEND most recent vector-memory operations) and its LDS reads are done,
    // then synchronise the work-group with a bare s_barrier (__syncthreads()
    // would add a full fence).  The empty asm statements keep the compiler
    // from moving LDS accesses across it.
    auto step_barrier = [&](auto npc) {
      constexpr int NPEND = decltype(npc)::value;
      static_assert(NPEND < 64, "vmcnt field");
      __builtin_amdgcn_s_waitcnt((NPEND & 15) | 0x0070 | ((NPEND >> 4) << 14));  // vmcnt(NPEND) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // Software pipeline over the five-tile ring.  Step kt runs in four phases
    // (bf16: its four K=16 substeps; fp8: its two K=64 substeps, accumulator
    // rows 0-1 then 2-3).  The fragments of the next substep are read from
    // LDS while the current one's MFMAs run, one read after each MFMA in the
    // order the next phase first needs them.  Before the last phase every
    // thread waits for its loads of step kt+1 and for its reads of step kt,
    // and the barrier then (a) makes step kt+1 visible, whose first fragments
    // are read during the last phase, and (b) frees step kt's tiles, into
    // whose A tile the B loads of step kt+2 go in that same phase.
    Frag fa[2][4], fb[2][NF];
    load_scales(kbeg);
    static_for<2 * LOADS>([&](auto lc) { load_one(decltype(lc)::value, 0, IC<false>{}); });
    uint32_t rd_a = next_step(ld_a), rd_b = next_step(ld_b);  // step 1
    ld_a = rd_a;
    ld_b = rd_b;
    static_for<2 * LOADS>([&](auto lc) { load_one(decltype(lc)::value, 1, IC<false>{}); });
    ld_a = next_step(ld_a);  // step 2
    ld_b = next_step(ld_b);
    step_barrier(IC<2 * LOADS>{});
    constexpr int NRD = 4 + NF;  // fragment reads per set
    Bases ca, cb;
    step_bases(0u, (uint32_t)TILE_BYTES, ca, cb);
    static_for<NRD>([&](auto rc) { read_one(ca, cb, 0, decltype(rc)::value, fa[0], fb[0]); });
    // Step kt reads the tiles of step kt + 1 (rd_*) in its last phase and
    // loads step kt + 2 into ld_*.  The next step's read bases and ring
    // offsets are formed right before the step barrier, where the wave
    // waits for its LDS reads anyway: with one wave per SIMD every other
    // instruction sits in the issue stream between two MFMAs.  The current
    // bases are dead by then, so the new ones take their registers.  The
    // pair kernel holds two GEMMs' unit code in one register budget: its
    // second GEMM (both operands K-major) forms them at the top of the step
    // instead (BAR_BASES false), since at the barrier they cost that kernel
    // three VGPRs it does not have.
    uint32_t nld_a, nld_b;
    auto advance = [&]() {
      if constexpr (BAR_BASES) step_bases(rd_a, rd_b, ca, cb);
      nld_a = next_step(ld_a);
      nld_b = next_step(ld_b);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto body = [&](int kt, auto fc) {
      Bases na, nb;  // the next step's bases when BAR_BASES is false
      if constexpr (!BAR_BASES) step_bases(rd_a, rd_b, na, nb);
      Bases& xa = BAR_BASES ? ca : na;
      Bases& xb = BAR_BASES ? cb : nb;
      const int kl = kt + 2;
      if constexpr (FP8) {
        // phases 0-1 read substep 1; phase 3 reads step kt+1 substep 0.
        // MX: the scales of step kt+1 load during phase 0, before this
        // step's operand loads, and land by the barrier.
        take_scales();
        load_scales(kbeg + kt + 1);
        mfma_rows(IC<0>{}, IC<2>{}, IC<0>{}, IC<LA0>{}, fa[0], fb[0], kl, fc, IC<0>{}, IC<NRD / 2>{}, ca, cb, 1,
                  fa[1], fb[1], IC<0>{});
        mfma_rows(IC<2>{}, IC<2>{}, IC<LA0>{}, IC<LA1>{}, fa[0], fb[0], kl, fc, IC<NRD / 2>{}, IC<NRD - NRD / 2>{}, ca,
                  cb, 1, fa[1], fb[1], IC<0>{});
        mfma_rows(IC<0>{}, IC<2>{}, IC<0>{}, IC<0>{}, fa[1], fb[1], kl, fc, IC<0>{}, IC<0>{}, ca, cb, 0, fa[0], fb[0],
                  IC<2>{});
        advance();
        step_barrier(IC<LOADS>{});
        mfma_rows(IC<2>{}, IC<2>{}, IC<LOADS>{}, IC<LOADS>{}, fa[1], fb[1], kl, fc, IC<0>{}, IC<NRD>{}, xa, xb, 0,
                  fa[0], fb[0], IC<2>{});
      } else {
        mfma_rows(IC<0>{}, IC<4>{}, IC<0>{}, IC<LA0>{}, fa[0], fb[0], kl, fc, IC<0>{}, IC<NRD>{}, ca, cb, 1, fa[1],
                  fb[1], IC<0>{});
        mfma_rows(IC<0>{}, IC<4>{}, IC<LA0>{}, IC<LA1>{}, fa[1], fb[1], kl, fc, IC<0>{}, IC<NRD>{}, ca, cb, 2, fa[0],
                  fb[0], IC<0>{});
        mfma_rows(IC<0>{}, IC<4>{}, IC<0>{}, IC<0>{}, fa[0], fb[0], kl, fc, IC<0>{}, IC<NRD>{}, ca, cb, 3, fa[1],
                  fb[1], IC<0>{});
        advance();
        step_barrier(IC<LOADS>{});
        mfma_rows(IC<0>{}, IC<4>{}, IC<LOADS>{}, IC<LOADS>{}, fa[1], fb[1], kl, fc, IC<0>{}, IC<NRD>{}, xa, xb, 0,
                  fa[0], fb[0], IC<0>{});
      }
      if constexpr (!BAR_BASES) {
        ca = na;
        cb = nb;
      }
      rd_a = ld_a;
      rd_b = ld_b;
      ld_a = nld_a;
      ld_b = nld_b;
    };
    // In a unit whose operand tiles are both full, steps whose loads (of
    // step kt+2) are full and inside the split take the fast form:
    // kt + 2 < nfull, where only the split's last step can be partial (the
    // last step of a K that is not a multiple of the step).
    const int nfull = (a_full && b_full) ? (kend * KSTEP <= p.K ? nks : nks - 1) : 0;
    int kt = 0;
    for (; kt + 2 < nfull; ++kt) body(kt, IC<true>{});
    for (; kt < nks; ++kt) body(kt, IC<false>{});
    // every wave is done reading the ring, and every DMA write into it has
    // landed (the loads past the end of the split), before the epilogue
    // stages into it
    wait_vmem();
    __syncthreads();

    // ---- epilogue.  Lane l holds rows m0+wm+32i+l%32 and columns
    //      n0+wn+32j+8q+4*(l/32)+{0..3} in acc[i][j][4q..4q+3].  Each wave
    //      stages its 128 x WN fp32 block through a private LDS region,
    //      EPI_ROWS x 64 at a time (rows padded to 68 floats against bank
    //      conflicts), and reads it back as 8 consecutive columns per lane:
    //      the element-wise code then runs in one compact loop and every
    //      global store is 16 bytes wide, eight lanes covering 128 bytes.
    float lmax = 0.f;
    // a unit of a split K range stores its raw fp32 partial, whatever the
    // output (a finalisation pass applies the epilogue)
    const bool raw = p.splits > 1 || un.tail >= 0;
    float* stage = reinterpret_cast<float*>(smem) + wave * LY::EPI_WAVE_FLOATS;
    constexpr int EPI_LD = LY::EPI_LD, EPI_COLS = LY::EPI_COLS, EPI_ROWS = LY::EPI_ROWS;
    constexpr int FPP = EPI_COLS / 32;                 // column fragments per pass
    constexpr int IPP = EPI_ROWS / 32;                 // row fragments per pass
    static_for<LY::PASSES>([&](auto pc) {
      constexpr int pass = decltype(pc)::value;
      constexpr int rp = pass / LY::COL_PASSES, cp = pass % LY::COL_PASSES;
      static_for<IPP * FPP * 4>([&](auto c) {
        constexpr int ii = decltype(c)::value / (FPP * 4);
        constexpr int jj = (decltype(c)::value / 4) % FPP;
        constexpr int q = decltype(c)::value % 4;
        constexpr int i = IPP * rp + ii;
        constexpr int j = FPP * cp + jj;
        const f32x4 v = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        *(f32x4*)(stage + (32 * ii + (lane & 31)) * EPI_LD + 32 * jj + 8 * q + 4 * (lane >> 5)) = v;
      });
      if constexpr (GATED) {
        // staged columns 0..31 are the gate products and 32..63 the up
        // products of the wave's 32 output columns: 8 of each per lane, 4
        // lanes per row
        with_act(p.act, [&](auto ac) {
        constexpr int ACT = decltype(ac)::value;
#pragma unroll 1
        for (int it = 0; it < EPI_ROWS / 16; ++it) {
          const int rl = it * 16 + (lane >> 2);
          const int cl = (lane & 3) * 8;
          const f32x4 g0 = *(const f32x4*)(stage + rl * EPI_LD + cl);
          const f32x4 g1 = *(const f32x4*)(stage + rl * EPI_LD + cl + 4);
          const f32x4 u0 = *(const f32x4*)(stage + rl * EPI_LD + 32 + cl);
          const f32x4 u1 = *(const f32x4*)(stage + rl * EPI_LD + 36 + cl);
          const int row = tl.m0 + wm + EPI_ROWS * rp + rl;
          const int col = tl.n0 + wn / 2 + cl;
          if (row < tl.m_end && col < p.N) {
            const float g[8] = {g0[0] * scale, g0[1] * scale, g0[2] * scale, g0[3] * scale,
                                g1[0] * scale, g1[1] * scale, g1[2] * scale, g1[3] * scale};
            const float u[8] = {u0[0] * scale, u0[1] * scale, u0[2] * scale, u0[3] * scale,
                                u1[0] * scale, u1[1] * scale, u1[2] * scale, u1[3] * scale};
            epi_gated_oct<ACT>(p, g, u, row, col);
          }
        }
        });
      } else if (FP8 && p.y_q_scale && !raw) {
        // fp8 output with a scale fixed before the call (delayed scaling):
        // codes e4m3(v * fp32(1 / s)), nearest-even, saturating; amax of the
        // fp32 values quantised
        const float inv = 1.0f / *p.y_q_scale;
        with_act(p.act, [&](auto ac) {
        constexpr int ACT = decltype(ac)::value;
#pragma unroll 1
        for (int it = 0; it < EPI_ROWS / 8; ++it) {
          const int rl = it * 8 + (lane >> 3);
          const int cl = (lane & 7) * 8;
          const f32x4 v0 = *(const f32x4*)(stage + rl * EPI_LD + cl);
          const f32x4 v1 = *(const f32x4*)(stage + rl * EPI_LD + cl + 4);
          const int row = tl.m0 + wm + EPI_ROWS * rp + rl;
          const int col = tl.n0 + wn + EPI_COLS * cp + cl;
          if (row < tl.m_end && col < p.N) {
            float v[8] = {v0[0] * scale, v0[1] * scale, v0[2] * scale, v0[3] * scale,
                          v1[0] * scale, v1[1] * scale, v1[2] * scale, v1[3] * scale};
            if (p.aux) store_oct(p.aux, p.ldaux, false, row, col, v);  // pre-activation, bf16
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float h = act_fwd_c<ACT>(v[e]);
              lmax = fmaxf(lmax, fabsf(h));
              q[e] = h * inv;
            }
            *(uint2*)((uint8_t*)p.Y + (int64_t)row * p.ldy + col) =
                make_uint2(fp8x4<false>(q[0], q[1], q[2], q[3]), fp8x4<false>(q[4], q[5], q[6], q[7]));
          }
        }
        });
      } else if (FP8 && p.y_mx && !raw) {
        // MXFP8 output: each 32-column block of a row (4 lanes) shares one
        // scale 2^(E-127), E = exponent field of the block's amax - 8 (0 for
        // a zero block); codes are e4m3(v * 2^(127-E)), nearest-even,
        // saturating.  The four lanes of a block always share their row and
        // validity (N % 32 == 0), so the shuffles stay inside live groups.
        with_act(p.act, [&](auto ac) {
        constexpr int ACT = decltype(ac)::value;
#pragma unroll 1
        for (int it = 0; it < EPI_ROWS / 8; ++it) {
          const int rl = it * 8 + (lane >> 3);
          const int cl = (lane & 7) * 8;
          const f32x4 v0 = *(const f32x4*)(stage + rl * EPI_LD + cl);
          const f32x4 v1 = *(const f32x4*)(stage + rl * EPI_LD + cl + 4);
          const int row = tl.m0 + wm + EPI_ROWS * rp + rl;
          const int col = tl.n0 + wn + EPI_COLS * cp + cl;
          const bool ok = row < tl.m_end && col < p.N;
          float v[8] = {v0[0] * scale, v0[1] * scale, v0[2] * scale, v0[3] * scale,
                        v1[0] * scale, v1[1] * scale, v1[2] * scale, v1[3] * scale};
          if (ok && p.aux) store_oct(p.aux, p.ldaux, false, row, col, v);  // pre-activation, bf16
          float m = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            v[e] = act_fwd_c<ACT>(v[e]);
            m = fmaxf(m, fabsf(v[e]));
          }
          m = fmaxf(m, __shfl_xor(m, 1, 64));
          m = fmaxf(m, __shfl_xor(m, 2, 64));
          if (ok) {
            const int E = max((int)((__float_as_uint(m) >> 23) & 0xFFu) - 8, 0);
            const float inv = __uint_as_float((uint32_t)(254 - E) << 23);   // 2^(127 - E)
            *(uint2*)((uint8_t*)p.Y + (int64_t)row * p.ldy + col) =
                make_uint2(fp8x4<false>(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv),
                           fp8x4<false>(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv));
            if ((lane & 3) == 0)
              p.y_mx[mx_scale_offset((uint32_t)row, (uint32_t)col >> 5, (uint32_t)p.y_mx_steps)] = (uint8_t)E;
          }
        }
        });
      } else {
      // read back 8 consecutive columns per lane, 8 lanes per row
      with_act(p.act, [&](auto ac) {
      constexpr int ACT = decltype(ac)::value;
      if (p.epi == EPI_DACT && !p.aux_f32 && !raw) {
        // DACT with a bf16 Z: the Z loads of four row groups are issued
        // together before any is used, instead of one exposed load latency
        // per row group
        constexpr int GRP = 4;
        static_assert((EPI_ROWS / 8) % GRP == 0, "row groups");
        with_fk_dact<!FP8>(p.y_f32 ? FK_ANY : (FK_DACT | (p.amax ? FK_AMAX : 0)), [&](auto fkc) {
        constexpr int FK = decltype(fkc)::value;
#pragma unroll 1
        for (int it0 = 0; it0 < EPI_ROWS / 8; it0 += GRP) {
          i32x4 zq[GRP];
#pragma unroll
          for (int g = 0; g < GRP; ++g) {
            const int row = tl.m0 + wm + EPI_ROWS * rp + (it0 + g) * 8 + (lane >> 3);
            const int col = tl.n0 + wn + EPI_COLS * cp + (lane & 7) * 8;
            zq[g] = i32x4{0, 0, 0, 0};
            if (row < tl.m_end && col < p.N)
              zq[g] = *(const i32x4*)((const uint16_t*)p.aux + (int64_t)row * p.ldaux + col);
          }
#pragma unroll
          for (int g = 0; g < GRP; ++g) {
            const int rl = (it0 + g) * 8 + (lane >> 3);
            const int cl = (lane & 7) * 8;
            const f32x4 v0 = *(const f32x4*)(stage + rl * EPI_LD + cl);
            const f32x4 v1 = *(const f32x4*)(stage + rl * EPI_LD + cl + 4);
            const int row = tl.m0 + wm + EPI_ROWS * rp + rl;
            const int col = tl.n0 + wn + EPI_COLS * cp + cl;
            if (row < tl.m_end && col < p.N) {
              float v[8] = {v0[0] * scale, v0[1] * scale, v0[2] * scale, v0[3] * scale,
                            v1[0] * scale, v1[1] * scale, v1[2] * scale, v1[3] * scale};
              epi_oct<ACT, true, FK>(p, v, row, col, lmax, zq[g]);
            }
          }
        }
        });
        return;
      }
      // the staged values of four row groups are read before any is used,
      // so their LDS latency overlaps (with one wave per SIMD nothing else
      // would hide it)
      constexpr int GRP = 4;
      static_assert((EPI_ROWS / 8) % GRP == 0, "row groups");
      const int fk = raw ? FK_RAW
                         : (p.epi == EPI_FWD && !p.y_f32 && !(p.aux && p.aux_f32))
                               ? (FK_FWD | (p.aux ? FK_AUX : 0) | (p.amax ? FK_AMAX : 0)) : FK_ANY;
      with_fk_general<!FP8>(fk, [&](auto fkc) {
      constexpr int FK = decltype(fkc)::value;
#pragma unroll 1
      for (int it0 = 0; it0 < EPI_ROWS / 8; it0 += GRP) {
        f32x4 v0s[GRP], v1s[GRP];
#pragma unroll
        for (int g = 0; g < GRP; ++g) {
          const int rl = (it0 + g) * 8 + (lane >> 3);
          const int cl = (lane & 7) * 8;
          v0s[g] = *(const f32x4*)(stage + rl * EPI_LD + cl);
          v1s[g] = *(const f32x4*)(stage + rl * EPI_LD + cl + 4);
        }
#pragma unroll
        for (int g = 0; g < GRP; ++g) {
          const f32x4 v0 = v0s[g], v1 = v1s[g];
          const int rl = (it0 + g) * 8 + (lane >> 3);
          const int cl = (lane & 7) * 8;
          const int row = tl.m0 + wm + EPI_ROWS * rp + rl;
          const int col = tl.n0 + wn + EPI_COLS * cp + cl;
          if (row < tl.m_end && col < p.N) {
            if (FK == FK_RAW || (FK == FK_ANY && raw)) {
              // raw fp32 partial of this K range; splitk_finalize or
              // tail_finalize sums them
              f32x4* dst = un.tail >= 0
                  ? (f32x4*)(p.partial + ((int64_t)(un.split * p.tail_tiles + un.tail) * BM + (row - tl.m0)) * BN +
                             (col - tl.n0))
                  : (f32x4*)(p.partial + ((int64_t)un.split * p.M + row) * p.N + col);
              dst[0] = v0;
              dst[1] = v1;
            } else {
              float v[8] = {v0[0] * scale, v0[1] * scale, v0[2] * scale, v0[3] * scale,
                            v1[0] * scale, v1[1] * scale, v1[2] * scale, v1[3] * scale};
              epi_oct<ACT, false, FK>(p, v, row, col, lmax);
            }
          }
        }
      }
      });
      });
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

template <bool FP8, bool AK, bool BKM, int NW, bool GATED = false, bool MX = false, int F8F = 0>
__global__ void __launch_bounds__(64 * NW, 1) gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[Layout<NW>::SMEM];
  // Chunk-gated GEMM: invalidate this XCD's caches once, before any
  // operand is loaded.  A row of chunk c is only ever loaded after
  // ready[c] has been seen set, and the producer publishes the data before
  // the flag (release), so no cache can hold a stale copy of it afterwards:
  // the per-chunk wait needs no further invalidation (which would throw away
  // every tile's cached operands on each chunk arrival).
  if (p.ready) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  for (int u = blockIdx.x; u < p.units; u += gridDim.x)
    run_unit<FP8, AK, BKM, NW, GATED, MX, F8F>(p, map_unit(p, u), smem);
}

// Two independent bf16 GEMMs in one persistent launch (the weight and the
// input gradient of a linear layer, which read the same dY): each XCD
// (work-groups congruent mod 8) owns a contiguous eighth of each GEMM's
// logical units, those of GEMM FIRST listed first, and its work-groups take
// units from that list through a per-XCD ticket counter (queue[x], zero at
// launch), so that the longer units start first and the shorter ones fill
// in behind them.  Every unit is computed whole by the work-group that
// takes it, so results do not depend on which one does.  A work-group
// leaves the first GEMM's loop for good once its ticket passes that GEMM's
// units, so the two loops (and their loop-invariant registers) never
// overlap.
template <int NW, bool AK0, bool BK0, bool AK1, bool BK1, int FIRST>
__global__ void __launch_bounds__(64 * NW, 1) gemm_pair_kernel(const GemmParams p0, const GemmParams p1,
                                                              uint32_t* queue) {
  // the ticket word is a control word of the ring (a __shared__ variable of
  // its own makes the compiler wait for all LDS DMA before every LDS read of
  // the K loop); tickets are taken between work units, with no load in flight
  __shared__ __attribute__((aligned(1024))) char smem[Layout<NW>::SMEM];
  volatile int* ticket_word = reinterpret_cast<volatile int*>(smem + CTRL_TICKET);
  const int x = blockIdx.x & 7;
  const int n0 = p0.units, n1 = p1.units;
  const int b0 = (int)((int64_t)x * n0 / 8), c0 = (int)((int64_t)(x + 1) * n0 / 8) - b0;
  const int b1 = (int)((int64_t)x * n1 / 8), c1 = (int)((int64_t)(x + 1) * n1 / 8) - b1;
  // (every thread reads a ticket before thread 0 can take the next one:
  // the unit's body passes several work-group barriers)
  auto take = [&]() {
    if (threadIdx.x == 0) *ticket_word = (int)atomicAdd(queue + x, 1u);
    __syncthreads();
    return *ticket_word;
  };
  int i = take();
  if constexpr (FIRST == 0) {
    for (; i < c0; i = take()) run_unit<false, AK0, BK0, NW, false, false, 0, true>(p0, logical_unit(p0, b0 + i), smem);
    for (; i < c0 + c1; i = take()) run_unit<false, AK1, BK1, NW, false, false, 0, false>(p1, logical_unit(p1, b1 + i - c0), smem);
  } else {
    for (; i < c1; i = take()) run_unit<false, AK1, BK1, NW, false, false, 0, false>(p1, logical_unit(p1, b1 + i), smem);
    for (; i < c0 + c1; i = take()) run_unit<false, AK0, BK0, NW, false, false, 0, true>(p0, logical_unit(p0, b0 + i - c1), smem);
  }
}


// The epilogue of 8 summed values in a finalisation pass: the fp8 output of
// delayed scaling as the GEMM kernel writes it (pre-activation saved as
// bf16, codes e4m3(act(v) * fp32(1 / s)), amax of act(v)), else epi_oct.
template <int ACT>
__device__ __forceinline__ void finalize_oct(const GemmParams& p, float (&v)[8], int row, int col, float& lmax) {
  if (p.y_q_scale) {
    const float inv = 1.0f / *p.y_q_scale;
    if (p.aux) store_oct(p.aux, p.ldaux, false, row, col, v);
    float q[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float h = act_fwd_c<ACT>(v[e]);
      lmax = fmaxf(lmax, fabsf(h));
      q[e] = h * inv;
    }
    *(uint2*)((uint8_t*)p.Y + (int64_t)row * p.ldy + col) =
        make_uint2(fp8x4<false>(q[0], q[1], q[2], q[3]), fp8x4<false>(q[4], q[5], q[6], q[7]));
    return;
  }
  epi_oct<ACT>(p, v, row, col, lmax);
}

// Split-K finalisation: Y = epilogue(scale * sum_{s=0}^{S-1} partial_s),
// summed in ascending s (deterministic), 8 consecutive columns per lane.
__global__ void __launch_bounds__(256) splitk_finalize(const GemmParams p) {
  float scale = 1.f;
  if (p.a_scale) scale *= *p.a_scale;
  if (p.b_scale) scale *= *p.b_scale;
  const int64_t n8 = p.N / 8;
  const int64_t total = (int64_t)p.M * n8;
  const int64_t plane = (int64_t)p.M * p.N;
  float lmax = 0.f;
  with_act(p.act, [&](auto ac) {
  constexpr int ACT = decltype(ac)::value;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total; w += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(w / n8);
    const int col = (int)(w - (int64_t)row * n8) * 8;
    const float* src = p.partial + (int64_t)row * p.N + col;
    f32x4 a0 = __builtin_nontemporal_load((const f32x4*)src);
    f32x4 a1 = __builtin_nontemporal_load((const f32x4*)src + 1);
    for (int sp = 1; sp < p.splits; ++sp) {
      a0 += __builtin_nontemporal_load((const f32x4*)(src + sp * plane));
      a1 += __builtin_nontemporal_load((const f32x4*)(src + sp * plane) + 1);
    }
    float v[8] = {a0[0] * scale, a0[1] * scale, a0[2] * scale, a0[3] * scale,
                  a1[0] * scale, a1[1] * scale, a1[2] * scale, a1[3] * scale};
    finalize_oct<ACT>(p, v, row, col, lmax);
  }
  });
  if (p.amax) block_amax(p.amax, lmax);
}

// Tail finalisation: each tail tile's pieces summed in ascending piece order
// (deterministic), scaled, then the epilogue; one work-group per 64 rows of a
// tail tile, 8 rows at a time, 8 consecutive columns per lane.
constexpr int kTailRows = 64;
__global__ void __launch_bounds__(256) tail_finalize(const GemmParams p) {
  float scale = 1.f;
  if (p.a_scale) scale *= *p.a_scale;
  if (p.b_scale) scale *= *p.b_scale;
  constexpr int BLOCKS_PER_TILE = BM / kTailRows;
  const int t = blockIdx.x / BLOCKS_PER_TILE;
  const int r0 = (blockIdx.x - t * BLOCKS_PER_TILE) * kTailRows + (threadIdx.x >> 5);
  const int c = (threadIdx.x & 31) * 8;
  const Tile tl = tail_tile(p, t);
  const int col = tl.n0 + c;
  const int64_t piece = (int64_t)p.tail_tiles * BM * BN;
  float lmax = 0.f;
  with_act(p.act, [&](auto ac) {
    constexpr int ACT = decltype(ac)::value;
#pragma unroll 2
    for (int i = 0; i < kTailRows / 8; ++i) {
      const int r = r0 + 8 * i;
      const int row = tl.m0 + r;
      if (row < tl.m_end && col < p.N) {
        const float* src = p.partial + ((int64_t)t * BM + r) * BN + c;
        f32x4 a0 = __builtin_nontemporal_load((const f32x4*)src);
        f32x4 a1 = __builtin_nontemporal_load((const f32x4*)src + 1);
        for (int sp = 1; sp < p.tail_pieces; ++sp) {
          a0 += __builtin_nontemporal_load((const f32x4*)(src + sp * piece));
          a1 += __builtin_nontemporal_load((const f32x4*)(src + sp * piece) + 1);
        }
        float v[8] = {a0[0] * scale, a0[1] * scale, a0[2] * scale, a0[3] * scale,
                      a1[0] * scale, a1[1] * scale, a1[2] * scale, a1[3] * scale};
        finalize_oct<ACT>(p, v, row, col, lmax);
      }
    }
  });
  if (p.amax) block_amax(p.amax, lmax);
}

}  // namespace

static hipError_t finalize_if_split(const GemmParams& p, hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    int64_t work = (int64_t)p.M * (p.N / 8);
    int64_t blocks = (work + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    splitk_finalize<<<(int)blocks, 256, 0, s>>>(p);
  } else if (p.tail_pieces > 1) {
    tail_finalize<<<p.tail_tiles * (BM / kTailRows), 256, 0, s>>>(p);
  } else {
    return hipSuccess;
  }
  return hipGetLastError();
}

// bf16: 8 waves (two per SIMD, 128 x 64 each).  fp8: 4 waves (128 x 128
// each): two fp8 fragment sets of a 128 x 64 wave do not fit next to its
// accumulators in the registers of one of two waves per SIMD.
#ifndef TPM_GEMM_WAVES_BF16
#define TPM_GEMM_WAVES_BF16 8
#endif
#ifndef TPM_GEMM_WAVES_FP8
#define TPM_GEMM_WAVES_FP8 4
#endif
constexpr int kWaves = TPM_GEMM_WAVES_BF16, kWaves8 = TPM_GEMM_WAVES_FP8;
constexpr int kThreads = 64 * kWaves, kThreads8 = 64 * kWaves8;

hipError_t launch_gemm_bf16(const GemmParams& p, bool a_kmajor, bool b_kmajor, int grid, hipStream_t s) {
  if (p.epi == EPI_GATED) {
    if (!a_kmajor || b_kmajor || p.splits != 1) return hipErrorInvalidValue;  // rejected on the host first
    gemm_kernel<false, true, false, 8, true><<<grid, 512, 0, s>>>(p);
    return hipGetLastError();
  }
  if (a_kmajor && !b_kmajor) gemm_kernel<false, true, false, kWaves><<<grid, kThreads, 0, s>>>(p);
  else if (a_kmajor && b_kmajor) gemm_kernel<false, true, true, kWaves><<<grid, kThreads, 0, s>>>(p);
  else if (!a_kmajor && !b_kmajor) gemm_kernel<false, false, false, kWaves><<<grid, kThreads, 0, s>>>(p);
  else gemm_kernel<false, false, true, kWaves><<<grid, kThreads, 0, s>>>(p);
  return finalize_if_split(p, s);
}

hipError_t launch_gemm_pair_bf16(const GemmParams& p0, bool a0_kmajor, bool b0_kmajor, const GemmParams& p1,
                                 bool a1_kmajor, bool b1_kmajor, int first, uint32_t* queue, int grid, hipStream_t s) {
  // instantiated for a linear layer's backward: dW = X^T dY (both operands
  // MN-major) and dX = dY W^T (both K-major)
  if (a0_kmajor || b0_kmajor || !a1_kmajor || !b1_kmajor) return hipErrorInvalidValue;  // rejected on the host first
  if (first == 0) gemm_pair_kernel<kWaves, false, false, true, true, 0><<<grid, kThreads, 0, s>>>(p0, p1, queue);
  else gemm_pair_kernel<kWaves, false, false, true, true, 1><<<grid, kThreads, 0, s>>>(p0, p1, queue);
  hipError_t e = finalize_if_split(p0, s);
  if (e != hipSuccess) return e;
  return finalize_if_split(p1, s);
}

hipError_t launch_gemm_fp8(const GemmParams& p, bool a_kmajor, bool b_kmajor, int grid, hipStream_t s) {
  if (!a_kmajor || !b_kmajor) return hipErrorInvalidValue;  // rejected on the host first
  if (p.a_mx) gemm_kernel<true, true, true, kWaves8, false, true><<<grid, kThreads8, 0, s>>>(p);
  else if (p.f8fmt == 1) gemm_kernel<true, true, true, kWaves8, false, false, 1><<<grid, kThreads8, 0, s>>>(p);
  else if (p.f8fmt == 2) gemm_kernel<true, true, true, kWaves8, false, false, 2><<<grid, kThreads8, 0, s>>>(p);
  else if (p.f8fmt == 0) gemm_kernel<true, true, true, kWaves8><<<grid, kThreads8, 0, s>>>(p);
  else return hipErrorInvalidValue;  // both operands e5m2: rejected on the host first
  return finalize_if_split(p, s);
}

}  // namespace tpm

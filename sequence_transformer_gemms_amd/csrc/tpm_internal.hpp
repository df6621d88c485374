// Private interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpm {

constexpr int kMaxGroups = 256;  // chunks or destination ranges per call
// Value of a workspace's error word after a chunk wait gave up (the word is
// zeroed by every chunk-gated call before its kernels run).
constexpr uint32_t kErrTimeout = 0x54504D31u;

// One GEMM launch: Y[M,N] = epilogue(op(A)[M,K] . op(B)[K,N]).
// Rows of Y are cut into `num_groups` equal groups of `group_rows` rows
// (sequence chunks, or destination token ranges); tiles never straddle a
// group, and groups are visited in `order`.
struct GemmParams {
  const void* A;
  const void* B;
  void* Y;
  void* aux;                 // FWD: pre-activation save (or null); DACT: Z input
  const float* a_scale;      // device fp32 dequant factor or null (= 1)
  const float* b_scale;
  float* amax;               // device: atomic max of |Y as stored| (or null)
  const uint32_t* ready;     // device, per group: tile waits for ready[g] >= epoch (or null)
  uint32_t* done;            // device, per group: set to epoch when all its tiles are stored
  uint32_t* err;             // device error word (watchdog), needed when ready != null
  uint32_t* group_cnt;       // device per-group finished-tile counters (zeroed per call)
  uint32_t a_bytes, b_bytes;  // extents of A and B for the buffer descriptors
  int64_t lda, ldb, ldy, ldaux;  // elements
  int M, N, K;
  int group_rows, num_groups;
  int mt_per_group, nt, tiles_per_group, total_tiles, band_m;
  uint32_t epoch;
  uint32_t wait_limit;       // polls before a wait gives up (watchdog)
  int act, epi, y_f32, aux_f32;
  int splits;                // K-range splits (1: none); > 1 needs `partial`
  int ksteps_per_split;      // K steps (of 32 bf16 / 64 fp8) per split
  float* partial;            // device fp32 [splits][M][N] partial sums, or the tail's pieces
  // Tail split (splits == 1 only): the tiles of the last tail_cols tile
  // columns (tail_tiles of them, t = their index in the group order) are cut
  // into tail_pieces K ranges of tail_ksteps steps, units tail_start + piece
  // * tail_tiles + t, whose fp32 partials go to partial[piece][t][256][256].
  // Units 0 .. tail_start - 1 are the whole tiles of the first nt_w tile
  // columns, tpg_w per group.  Without a tail: tail_cols = 0, nt_w = nt,
  // tail_start = units.
  int units;                 // work units of the launch
  int nt_w, tpg_w;
  int tail_start, tail_tiles, tail_cols, tail_pieces, tail_ksteps;
  // MXFP8 (fp8 kernel only): E8M0 block scales of A and B in the MFMA
  // layout (mx_scale_offset), K / 128 records per 32-row group; y_mx: Y is
  // written as MXFP8 codes with its scales there (N / 128 records per group)
  const uint8_t* a_mx;
  const uint8_t* b_mx;
  uint32_t a_mx_bytes, b_mx_bytes;
  int mx_steps;
  uint8_t* y_mx;
  int y_mx_steps;
  const float* y_q_scale;    // fp8 per-tensor output: Y = e4m3(v / *y_q_scale) (or null)
  int f8fmt;                 // fp8 operand formats: bit 0 A is e5m2, bit 1 B is e5m2 (else e4m3)
  int a_dt, b_dt;            // element types of A and B (tpm dtype codes), read by the generic kernel
  int gu_off;                // gated epilogues: column offset of the up half in B / aux / Y (= N)
  int bn_out;                // output columns per tile (256; 128 for EPI_GATED)
  int16_t order[kMaxGroups];
};

enum { EPI_FWD = 0, EPI_DACT = 1, EPI_GATED = 2, EPI_DGATED = 3 };

// Byte offset of the E8M0 scale of (row, 32-element block kb) of an MXFP8
// operand in the layout the scaled MFMA reads: rows in groups of 32, each
// group a run of 128-byte records, one per K step of 128 elements, holding
// 4 bytes (blocks 4s .. 4s+3) for each of its 32 rows.  One fragment's 32
// lanes then read one 128-byte line per K step.
__host__ __device__ inline uint32_t mx_scale_offset(uint32_t row, uint32_t kb, uint32_t ksteps) {
  return (((row >> 5) * ksteps + (kb >> 2)) * 32u + (row & 31u)) * 4u + (kb & 3u);
}

// Side-stream chunk writer: chunks order[0..n-1] of chunk_bytes each, copied
// src -> dst when copy[c] != 0, then ready[c] = epoch.
struct WriterParams {
  const char* src;
  char* dst;
  int64_t chunk_bytes;
  uint32_t* ready;
  uint32_t* counters;        // per chunk, zero between calls
  uint32_t epoch;
  int n;
  int16_t order[kMaxGroups];
  uint8_t copy[kMaxGroups];
};

// kernels' launchers (return hipError_t of the launch)
hipError_t launch_gemm_bf16(const GemmParams& p, bool a_kmajor, bool b_kmajor, int grid, hipStream_t s);
// Two bf16 GEMMs in one persistent launch (p0: both operands MN-major, p1:
// both K-major), units taken from per-XCD ticket counters queue[0..7]
// (zero at launch); `first` (0 or 1) names the GEMM whose units go first.
hipError_t launch_gemm_pair_bf16(const GemmParams& p0, bool a0_kmajor, bool b0_kmajor, const GemmParams& p1,
                                 bool a1_kmajor, bool b1_kmajor, int first, uint32_t* queue, int grid, hipStream_t s);
hipError_t launch_gemm_fp8(const GemmParams& p, bool a_kmajor, bool b_kmajor, int grid, hipStream_t s);
hipError_t launch_delayed_scale(const float* history, int n, float* scale_out, hipStream_t s);
hipError_t launch_amax_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint32_t* out, hipStream_t s);
hipError_t launch_cast_fp8_t(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* amax, bool e5m2,
                             uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, float* s_out, hipStream_t s);
hipError_t launch_transpose_u8(const uint8_t* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* y, int64_t ldy,
                               hipStream_t s);
hipError_t launch_mx_swizzle(const uint8_t* src, int64_t ld, int rows, int kblocks, uint8_t* dst, hipStream_t s);
// Predicated LDS-tiled FMA GEMM: any shape, layout, alignment and element
// types (a_dt / b_dt); FWD and DACT epilogues, amax, fp32 or bf16 output.
hipError_t launch_gemm_generic(const GemmParams& p, bool trans_a, bool trans_b, hipStream_t s);
hipError_t launch_ctrl_init(uint32_t* words, int n, hipStream_t s);
hipError_t launch_reduce(int T, int64_t rows, int64_t D, const void* partials, int64_t pstride,
                         int64_t ld, int in_f32, void* out, int64_t ldo, int out_f32, hipStream_t s);
hipError_t launch_quant_e4m3(const uint16_t* h, int64_t M, int64_t N, int64_t ldh, const float* amax,
                             uint8_t* q, int64_t ldq, float* s_out, hipStream_t s);
hipError_t launch_signal(uint32_t* flag, uint32_t value, hipStream_t s);
hipError_t launch_write_chunks(const WriterParams& p, int groups, hipStream_t s);

constexpr int kTileM = 256, kTileN = 256;
constexpr int kStepBytes = 128;  // K bytes per staged step of the MFMA kernel

}  // namespace tpm

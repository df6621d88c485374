// C-ABI layer of libtpmlp: argument validation (host-side, before anything
// is enqueued), kernel selection, workspace carving, launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/tpmlp.h"
#include "tpm_internal.hpp"

using namespace tpm;

namespace {

thread_local char g_err[512] = "no error";
uint32_t g_wait_limit = 1u << 22;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TPM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// control words at the head of every workspace
constexpr int kCtrlErr = 0, kCtrlAmax = 1, kCtrlScale = 2, kCtrlCnt = 4;
constexpr int kCtrlQueue = kCtrlCnt + kMaxGroups;   // 8 per-XCD ticket counters of paired launches
constexpr int kCtrlWords = kCtrlQueue + 8;
constexpr size_t kCtrlBytes = 2048;
static_assert(kCtrlWords * 4 <= (int)kCtrlBytes, "control block");

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Compute units a kernel enqueued on stream s may use: the popcount of the
// stream's CU mask (streams made with hipExtStreamCreateWithCUMask), else
// the device's count.
int stream_cus(hipStream_t s) {
  const int dev_cus = num_cus();
  uint32_t mask[32] = {0};
  const uint32_t words = (uint32_t)std::min(32, (dev_cus + 31) / 32);
  if (hipExtStreamGetCUMask(s, words, mask) != hipSuccess) {
    (void)hipGetLastError();
    return dev_cus;
  }
  int n = 0;
  for (uint32_t i = 0; i < words; ++i) n += __builtin_popcount(mask[i]);
  return (n > 0 && n <= dev_cus) ? n : dev_cus;
}

int esize(int dt) { return dt == TPM_F32 ? 4 : dt == TPM_BF16 ? 2 : 1; }
bool valid_dt(int dt) { return dt == TPM_F32 || dt == TPM_BF16 || dt == TPM_FP8_E4M3 || dt == TPM_FP8_E5M2; }
bool is_fp8(int dt) { return dt == TPM_FP8_E4M3 || dt == TPM_FP8_E5M2; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Split-K plan.  A GEMM with fewer output tiles than about three quarters of
// the CUs leaves the chip idle; its K range is then cut into S pieces whose
// fp32 partial sums are added in a fixed order by a second kernel.  S
// minimises rounds(tiles * S) / S with a small per-split cost, keeping at
// least 8 K steps per piece.  The plan assumes 256 CUs (MI355X) so that the
// workspace size can be computed without a device.
constexpr int kPlanCUs = 256;

int plan_splits(int64_t M, int64_t N, int64_t K, int groups, int dt) {
  if (dt == TPM_F32 || M <= 0 || N <= 0 || K <= 0) return 1;
  const int64_t group_rows = M / std::max(groups, 1);
  const int64_t tiles = ((group_rows + kTileM - 1) / kTileM) * groups * ((N + kTileN - 1) / kTileN);
  if (tiles * 4 >= (int64_t)kPlanCUs * 3) return 1;
  const int64_t nk = (K * esize(dt) + kStepBytes - 1) / kStepBytes;
  int best = 1;
  double best_cost = 1e30;
  for (int S = 1; S <= 8; ++S) {
    if (S > 1 && nk / S < 8) break;
    const double rounds = (double)((tiles * S + kPlanCUs - 1) / kPlanCUs);
    const double cost = rounds / S * (1.0 + 0.04 * S);
    if (cost < best_cost) { best_cost = cost; best = S; }
  }
  return best;
}

size_t partial_bytes(int64_t M, int64_t N, int S) {
  return S > 1 ? round_up((size_t)S * (size_t)M * (size_t)N * 4, 256) : 0;
}

// Split plan of one launch: S K-range splits of every tile (few tiles), or
// a tail split.  Whole tiles fill rounds of kPlanCUs work-groups; when the
// last round is partly empty, most CUs idle through one whole tile time.  A
// tail split takes the tiles of the last tail_cols tile columns out of the
// whole-tile rounds and cuts each into tail_pieces K ranges, which fill the
// idle slots and one short round after; a second kernel sums each tile's
// fp32 partials in piece order and applies the epilogue.  Whether an output
// element is split depends only on its column and on (M, N, K, element
// type): any chunk count and chunk order give the same bits.  At most
// kPlanCUs pieces (64 MiB of partials when the tile rows are whole).
// The plan minimises an estimate, in K steps, of the busiest work-group's
// time under the round-robin schedule: whole tiles cost nk + 2, pieces
// ceil(nk / P) + 4 (a 256 KB fp32 store), and the finalisation pass
// tail_tiles * P / 32 (256 KB per piece read at ~6 TB/s, a K step being
// ~1.5 us); at least 8 K steps per piece.
struct SplitPlan {
  int S = 1;
  int tail_cols = 0, tail_pieces = 1;
};

SplitPlan plan_gemm(int64_t M, int64_t N, int64_t K, int groups, int dt) {
  SplitPlan pl;
  pl.S = plan_splits(M, N, K, groups, dt);
  if (pl.S > 1 || dt == TPM_F32 || M <= 0 || N <= 0 || K <= 0) return pl;
  const int64_t mt = (M + kTileM - 1) / kTileM, nt = (N + kTileN - 1) / kTileN;
  const int64_t total = mt * nt, G = kPlanCUs;
  if (total <= G) return pl;
  const int64_t nk = (K * esize(dt) + kStepBytes - 1) / kStepBytes;
  const double tw = (double)nk + 2.0;
  double best = (double)((total + G - 1) / G) * tw;
  for (int64_t c = 1; c < nt && c * mt <= G; ++c) {
    const int64_t tail = c * mt, whole = total - tail;
    const int64_t whole_rounds = (whole + G - 1) / G;
    for (int P = 2; P <= 8 && tail * P <= G && nk / P >= 8; ++P) {
      const int64_t rounds = (whole + tail * P + G - 1) / G;
      const double tp = (double)((nk + P - 1) / P) + 4.0;
      const double cost = (double)whole_rounds * tw + (double)(rounds - whole_rounds) * tp + (double)(tail * P) / 32.0;
      if (cost < best) {
        best = cost;
        pl.tail_cols = (int)c;
        pl.tail_pieces = P;
      }
    }
  }
  return pl;
}

// Row tiles of a launch over M rows in `groups` equal groups.
int64_t row_tiles(int64_t M, int groups) {
  groups = std::max(groups, 1);
  return ((M / groups + kTileM - 1) / kTileM) * groups;
}

size_t plan_bytes(const SplitPlan& pl, int64_t M, int64_t N, int groups) {
  if (pl.S > 1) return partial_bytes(M, N, pl.S);
  if (pl.tail_pieces <= 1) return 0;
  return round_up((size_t)row_tiles(M, groups) * pl.tail_cols * pl.tail_pieces * kTileM * kTileN * 4, 256);
}

// Partial-sum scratch of the launch plan_gemm makes for this shape.
size_t plan_bytes(int64_t M, int64_t N, int64_t K, int groups, int dt) {
  return plan_bytes(plan_gemm(M, N, K, groups, dt), M, N, groups);
}

// Split plan of the paired launch of a linear layer's backward (dW = X^T dY:
// [K, N] over M; dX = dY W^T: [M, K] over N; S[0], S[1]).  The launch
// shares the two GEMMs' K steps over kPlanCUs work-groups; a GEMM whose
// whole-tile units are longer than that per-CU share is cut into
// ceil(steps / share) K ranges (at most 8, each of at least 8 steps), so
// that no unit outlasts the balanced finish by much.  BF16 only; else 1.
void plan_linear_bwd(int64_t M, int64_t N, int64_t K, int dt, int (&S)[2]) {
  S[0] = S[1] = 1;
  if (dt != TPM_BF16 || M <= 0 || N <= 0 || K <= 0) return;
  const int64_t tiles[2] = {((K + kTileM - 1) / kTileM) * ((N + kTileN - 1) / kTileN),
                            ((M + kTileM - 1) / kTileM) * ((K + kTileN - 1) / kTileN)};
  const int64_t nk[2] = {(M * esize(dt) + kStepBytes - 1) / kStepBytes, (N * esize(dt) + kStepBytes - 1) / kStepBytes};
  const int64_t work = tiles[0] * nk[0] + tiles[1] * nk[1];
  const int64_t share = std::max<int64_t>(1, (work + kPlanCUs - 1) / kPlanCUs);
  for (int i = 0; i < 2; ++i) {
    int64_t s = (nk[i] + share - 1) / share;
    s = std::min<int64_t>(s, 8);
    while (s > 1 && nk[i] / s < 8) --s;
    S[i] = (int)std::max<int64_t>(s, 1);
  }
}

struct GemmDesc {
  int64_t M, N, K;
  const void* A; int64_t lda; bool ta; int adt; const float* asc;
  const void* B; int64_t ldb; bool tb; int bdt; const float* bsc;
  void* Y; int64_t ldy; int ydt;
  int epi, act; void* aux; int64_t ldaux; float* amax;
  int groups; const int32_t* order; const uint32_t* ready; uint32_t* done; uint32_t epoch;
  uint32_t* ctrl;   // device control words (err, amax, counters) or null
  float* part = nullptr;   // device scratch for split-K partial sums
  size_t part_bytes = 0;
  // MXFP8: block scales of A and B (MFMA layout), and of Y when Y is MXFP8
  const uint8_t* a_mx = nullptr;
  const uint8_t* b_mx = nullptr;
  uint8_t* y_mx = nullptr;
  const float* y_qs = nullptr;   // fp8 per-tensor output scale (dequant factor), delayed scaling
};

size_t mx_scales_bytes(int64_t rows, int64_t k) { return (size_t)((rows + 31) / 32) * 32 * (size_t)(k / 32); }

// Rows the predicated kernel takes (its grid's y dimension is M / 16).
constexpr int64_t kGenericMaxM = 65535 * 16;

// Why the matrix-core kernel cannot take this GEMM, or nullptr if it can.
// Its loads and stores move 16-byte chunks through buffer descriptors of
// at most 4 GiB; anything else runs on the predicated kernel.
const char* fast_path_blocker(const GemmDesc& g) {
  if (g.adt == TPM_F32) return "fp32 operands";
  const int q = g.adt == TPM_BF16 ? 8 : 16;
  if (is_fp8(g.adt) && (g.ta || !g.tb)) return "fp8 operands stored MN-major";
  if (g.N % 8 != 0) return "N % 8 != 0";
  if (g.K % q != 0) return "K not a whole number of 16-byte chunks";
  if (g.ldy % 4 != 0 || (g.aux && g.ldaux % 4 != 0)) return "ldy or ldaux % 4 != 0";
  if ((g.y_mx || g.y_qs) && g.ldy % 8 != 0) return "fp8 output with ldy % 8 != 0";
  if (((uintptr_t)g.Y & 15) || (g.aux && ((uintptr_t)g.aux & 15))) return "Y or aux not 16-byte aligned";
  if (g.K == 0) return nullptr;
  if (g.ta && g.M % 8 != 0) return "trans_a with M % 8 != 0";
  if (g.lda % q != 0 || g.ldb % q != 0) return "lda or ldb not a whole number of 16-byte chunks";
  if (!aligned16(g.A) || !aligned16(g.B)) return "A or B not 16-byte aligned";
  const int64_t a_rows = g.ta ? g.K : g.M, b_rows = g.tb ? g.N : g.K;
  const double a_ext = (double)a_rows * g.lda * esize(g.adt), b_ext = (double)b_rows * g.ldb * esize(g.bdt);
  if (a_ext >= 4294967040.0 || b_ext >= 4294967040.0) return "an operand spans >= 4 GiB";
  return nullptr;
}

// Full host-side validation of one GEMM; returns TPM_OK or an error code.
int check_gemm(const GemmDesc& g, const char* who) {
  if (g.M < 0 || g.N < 0 || g.K < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (g.M > INT32_MAX || g.N > INT32_MAX || g.K > INT32_MAX) return fail(TPM_EUNSUPPORTED, "%s: size >= 2^31", who);
  if (!valid_dt(g.adt) || !valid_dt(g.bdt) || (g.adt != g.bdt && !(is_fp8(g.adt) && is_fp8(g.bdt))))
    return fail(TPM_EINVAL, "%s: operand dtypes must match (or both be fp8)", who);
  if (g.adt == TPM_FP8_E5M2 && g.bdt == TPM_FP8_E5M2)
    return fail(TPM_EUNSUPPORTED, "%s: e5m2 x e5m2 is not implemented", who);
  if (g.ydt != TPM_F32 && g.ydt != TPM_BF16 && !(g.ydt == TPM_FP8_E4M3 && (g.y_mx || g.y_qs)))
    return fail(TPM_EINVAL, "%s: output dtype must be F32 or BF16 (or MXFP8)", who);
  if (g.epi < TPM_EPI_FWD || g.epi > TPM_EPI_DGATED) return fail(TPM_EINVAL, "%s: bad epilogue", who);
  if (g.act < TPM_ACT_NONE || g.act > TPM_ACT_SILU) return fail(TPM_EINVAL, "%s: bad activation", who);
  const bool gated = g.epi == TPM_EPI_GATED || g.epi == TPM_EPI_DGATED;
  if (gated) {
    if (g.adt != TPM_BF16) return fail(TPM_EUNSUPPORTED, "%s: gated epilogues take bf16 operands", who);
    if (g.amax) return fail(TPM_EUNSUPPORTED, "%s: no amax with a gated epilogue", who);
    if (g.epi == TPM_EPI_GATED && (g.ta || g.tb))
      return fail(TPM_EUNSUPPORTED, "%s: EPI_GATED needs trans_a = 0 and trans_b = 0", who);
    if (g.epi == TPM_EPI_DGATED && !g.aux) return fail(TPM_EINVAL, "%s: DGATED epilogue needs aux ([G | U])", who);
    if (g.aux && g.ldaux < 2 * g.N) return fail(TPM_EINVAL, "%s: gated aux needs ldaux >= 2N", who);
    if (g.epi == TPM_EPI_DGATED && g.ldy < 2 * g.N) return fail(TPM_EINVAL, "%s: DGATED needs ldy >= 2N", who);
    if (g.epi == TPM_EPI_GATED && g.K > 0 && g.ldb < 2 * g.N)
      return fail(TPM_EINVAL, "%s: EPI_GATED needs ldb >= 2N ([W_gate | W_up])", who);
  }
  if (g.groups < 1 || g.groups > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks must be in [1, %d]", who, TPM_MAX_CHUNKS);
  if (g.M % g.groups != 0) return fail(TPM_EINVAL, "%s: M (%lld) %% num_chunks (%d) != 0", who, (long long)g.M, g.groups);
  if (g.order) {
    std::vector<char> seen(g.groups, 0);
    for (int i = 0; i < g.groups; ++i) {
      const int c = g.order[i];
      if (c < 0 || c >= g.groups || seen[c]) return fail(TPM_EINVAL, "%s: chunk order is not a permutation", who);
      seen[c] = 1;
    }
  }
  if (g.a_mx || g.b_mx || g.y_mx) {
    if (g.adt != TPM_FP8_E4M3 || !g.a_mx || !g.b_mx)
      return fail(TPM_EINVAL, "%s: MXFP8 needs fp8 operands and both scale arrays", who);
    if (g.ta || !g.tb) return fail(TPM_EUNSUPPORTED, "%s: MXFP8 operands must be K-major (trans_a = 0, trans_b = 1)", who);
    if (g.K % 128 != 0) return fail(TPM_EUNSUPPORTED, "%s: MXFP8 needs K %% 128 == 0", who);
    if (g.asc || g.bsc || g.amax) return fail(TPM_EINVAL, "%s: MXFP8 takes no per-tensor scales or amax", who);
    if (g.epi != TPM_EPI_FWD) return fail(TPM_EUNSUPPORTED, "%s: MXFP8 with the FWD epilogue only", who);
  }
  if (g.ydt == TPM_FP8_E4M3 && g.y_qs) {
    if (g.y_mx || g.adt != TPM_FP8_E4M3 || g.epi != TPM_EPI_FWD)
      return fail(TPM_EUNSUPPORTED, "%s: a per-tensor fp8 output needs fp8 operands and the FWD epilogue", who);
  } else if (g.ydt == TPM_FP8_E4M3 && (!g.y_mx || g.N % 128 != 0)) {
    return fail(TPM_EUNSUPPORTED, "%s: an fp8 output is MXFP8 (scales required, N %% 128 == 0)", who);
  }
  if (g.y_mx && g.ydt != TPM_FP8_E4M3) return fail(TPM_EINVAL, "%s: output scales given for a non-fp8 output", who);
  if (g.M == 0 || g.N == 0) return TPM_OK;
  if (!g.Y) return fail(TPM_EINVAL, "%s: null output", who);
  if (g.K > 0 && (!g.A || !g.B)) return fail(TPM_EINVAL, "%s: null operand", who);
  const int64_t a_cols = g.ta ? g.M : g.K, b_cols = g.tb ? g.K : g.N;
  if (g.ldy < g.N || (g.K > 0 && (g.lda < a_cols || g.ldb < b_cols)))
    return fail(TPM_EINVAL, "%s: leading dimension smaller than the row width", who);
  if (g.epi == TPM_EPI_DACT && !g.aux) return fail(TPM_EINVAL, "%s: DACT epilogue needs aux (Z)", who);
  if (g.aux && g.ldaux < (gated ? 2 * g.N : g.N)) return fail(TPM_EINVAL, "%s: ldaux < N", who);
  if ((g.ready || g.amax || g.done) && !g.ctrl) return fail(TPM_EWORKSPACE, "%s: workspace required", who);
  if (g.adt == TPM_F32) {
    if (g.ydt != TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: fp32 operands give fp32 output", who);
    if (g.ready || g.done) return fail(TPM_EUNSUPPORTED, "%s: chunk gating is implemented on the bf16/fp8 path", who);
  }
  const char* why = fast_path_blocker(g);
  if (why) {
    // the predicated kernel: FWD / DACT epilogues, per-tensor scales, amax
    if (g.ready || g.done)
      return fail(TPM_EUNSUPPORTED, "%s: chunk gating needs the matrix-core kernel (%s)", who, why);
    if (gated || g.a_mx || g.b_mx || g.y_mx || g.y_qs)
      return fail(TPM_EUNSUPPORTED, "%s: this epilogue or format needs the matrix-core kernel (%s)", who, why);
    if (g.M > kGenericMaxM) return fail(TPM_EUNSUPPORTED, "%s: M > %lld on the predicated path (%s)", who,
                                        (long long)kGenericMaxM, why);
    return TPM_OK;
  }
  if (g.ready) {
    // A chunk's rows are loaded only after its flag is seen, and no cache
    // line of a chunk may be fetched earlier as part of another chunk's
    // rows: A token-major, its base and every chunk boundary on a 128-byte
    // cache line.
    if (g.ta) return fail(TPM_EUNSUPPORTED, "%s: a chunk-gated A must be stored token-major (trans_a = 0)", who);
    const int64_t chunk_bytes = (g.M / g.groups) * g.lda * esize(g.adt);
    if (((uintptr_t)g.A & 127) || chunk_bytes % 128 != 0)
      return fail(TPM_EUNSUPPORTED, "%s: a chunk-gated A needs a 128-byte aligned base and chunk boundaries", who);
  }
  return TPM_OK;
}

// Kernel parameters of one checked GEMM under split plan pl (the caller has
// made sure the partial-sum scratch holds what the plan needs).
void make_params(const GemmDesc& g, const SplitPlan& pl, GemmParams& p) {
  const int S = pl.S;
  std::memset(&p, 0, sizeof(p));
  p.A = g.A; p.B = g.B; p.Y = g.Y; p.aux = g.aux;
  p.a_scale = g.asc; p.b_scale = g.bsc; p.amax = g.amax;
  p.ready = g.ready; p.done = g.done;
  p.err = g.ctrl ? g.ctrl + kCtrlErr : nullptr;
  p.group_cnt = g.ctrl ? g.ctrl + kCtrlCnt : nullptr;
  p.lda = g.lda; p.ldb = g.ldb; p.ldy = g.ldy; p.ldaux = g.ldaux;
  p.M = (int)g.M; p.N = (int)g.N; p.K = (int)g.K;
  // Without chunk flags or range-done signalling the groups only order the
  // tiles.  When their rows are whole tiles, the launch walks all of M as one
  // group instead: its bands of band_m tile rows then span the groups, which
  // gives the 32 tiles an XCD runs at once a squarer footprint of A and B
  // panels in its L2.  The tiles, hence the results, are the same.
  const bool one_group = !g.ready && !g.done && g.groups > 1 && (g.M / g.groups) % kTileM == 0;
  const int groups = one_group ? 1 : g.groups;
  p.num_groups = groups;
  p.group_rows = (int)(g.M / groups);
  p.epoch = g.epoch;
  p.wait_limit = g_wait_limit;
  p.act = g.act; p.epi = g.epi; p.y_f32 = g.ydt == TPM_F32; p.aux_f32 = p.y_f32;
  for (int i = 0; i < groups; ++i) p.order[i] = (int16_t)(g.order && !one_group ? g.order[i] : i);
  const int64_t nk = (g.K * esize(g.adt) + kStepBytes - 1) / kStepBytes;
  p.splits = S;
  p.ksteps_per_split = (int)((nk + S - 1) / S);
  p.partial = S > 1 ? g.part : nullptr;
  const int64_t a_rows = g.ta ? g.K : g.M, b_rows = g.tb ? g.N : g.K;
  p.a_bytes = g.K == 0 ? 0u : (uint32_t)(a_rows * g.lda * esize(g.adt));
  p.b_bytes = g.K == 0 ? 0u : (uint32_t)(b_rows * g.ldb * esize(g.bdt));
  p.a_mx = g.a_mx; p.b_mx = g.b_mx; p.y_mx = g.y_mx; p.y_q_scale = g.y_qs;
  p.f8fmt = (g.adt == TPM_FP8_E5M2 ? 1 : 0) | (g.bdt == TPM_FP8_E5M2 ? 2 : 0);
  p.a_dt = g.adt;
  p.b_dt = g.bdt;
  p.mx_steps = (int)(g.K / 128);
  p.y_mx_steps = (int)(g.N / 128);
  p.a_mx_bytes = g.a_mx ? (uint32_t)mx_scales_bytes(g.M, g.K) : 0u;
  p.b_mx_bytes = g.b_mx ? (uint32_t)mx_scales_bytes(g.N, g.K) : 0u;
  p.gu_off = (g.epi == TPM_EPI_GATED || g.epi == TPM_EPI_DGATED) ? (int)g.N : 0;
  p.bn_out = g.epi == TPM_EPI_GATED ? kTileN / 2 : kTileN;
  p.mt_per_group = (p.group_rows + kTileM - 1) / kTileM;
  p.nt = (p.N + p.bn_out - 1) / p.bn_out;
  p.tiles_per_group = p.mt_per_group * p.nt;
  p.total_tiles = p.tiles_per_group * p.num_groups;
  p.band_m = std::min(p.mt_per_group, 4);
  p.units = p.total_tiles * S;
  p.nt_w = p.nt;
  p.tpg_w = p.tiles_per_group;
  p.tail_start = p.units;
  p.tail_tiles = p.tail_cols = p.tail_ksteps = 0;
  p.tail_pieces = 1;
  if (S == 1 && pl.tail_pieces > 1 && pl.tail_cols > 0 && pl.tail_cols < p.nt) {
    p.tail_cols = pl.tail_cols;
    p.tail_pieces = pl.tail_pieces;
    p.tail_ksteps = (int)((nk + pl.tail_pieces - 1) / pl.tail_pieces);
    p.nt_w = p.nt - pl.tail_cols;
    p.tpg_w = p.mt_per_group * p.nt_w;
    p.tail_tiles = p.mt_per_group * pl.tail_cols * p.num_groups;
    p.tail_start = p.tpg_w * p.num_groups;
    p.units = p.tail_start + p.tail_tiles * pl.tail_pieces;
    p.partial = g.part;
  }
}

// Split plan the matrix-core path makes for a GEMM (none on the predicated
// path).  Chunk-gated GEMMs split too; range-done signalling needs whole
// tiles, and the gated forward and the MXFP8 output pair or scale whole
// tiles in their epilogues (the finalisation passes write the delayed-
// scaling fp8 output as the GEMM kernel does).  The plan depends on the shape, the chunk count
// and the element type only, never on the stream or the grid, so that a
// chunk-fed call and a resident one give the same bits.
SplitPlan planned_split(const GemmDesc& g) {
  if (fast_path_blocker(g) || g.done || g.epi == TPM_EPI_GATED || g.y_mx) return SplitPlan{};
  return plan_gemm(g.M, g.N, g.K, g.groups, g.adt);
}

int run_gemm(const GemmDesc& g, hipStream_t s, const char* who) {
  if (g.M == 0 || g.N == 0) return TPM_OK;
  GemmParams p;
  hipError_t e;
  if (fast_path_blocker(g)) {
    make_params(g, SplitPlan{}, p);
    e = launch_gemm_generic(p, g.ta, g.tb, s);
    return e == hipSuccess ? TPM_OK : hip_fail(e, who);
  }
  // split-K or a tail split when the plan asks for it and the scratch is there
  SplitPlan pl = planned_split(g);
  const size_t need = plan_bytes(pl, g.M, g.N, g.groups);
  if (need > 0 && (!g.part || g.part_bytes < need)) pl = SplitPlan{};
  make_params(g, pl, p);
  // persistent grid: one work-group per CU the stream may use.  A
  // chunk-gated GEMM on a stream that may use every CU leaves one CU per XCD
  // to a producer that runs kernels on this device; a stream with a CU mask
  // is taken to leave the producer its own CUs.
  const int cus = num_cus();
  const int avail = stream_cus(s);
  int grid = (g.ready && avail == cus) ? cus - 8 : avail;
  grid = std::max(8, grid);
  grid = std::min(grid, p.units);
  if (g.adt == TPM_BF16) e = launch_gemm_bf16(p, !g.ta, g.tb, grid, s);
  else e = launch_gemm_fp8(p, !g.ta, g.tb, grid, s);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

uint32_t* ctrl_of(void* ws, size_t bytes) { return (ws && bytes >= kCtrlBytes) ? (uint32_t*)ws : nullptr; }

void ring_order(int T, int C, int rank, int32_t* out) {
  if (T >= 1 && C % T == 0 && rank >= 0 && rank < T) {
    const int per = C / T;
    int n = 0;
    for (int step = 0; step < T; ++step) {
      const int q = ((rank - step) % T + T) % T;
      for (int i = 0; i < per; ++i) out[n++] = q * per + i;
    }
  } else {
    for (int i = 0; i < C; ++i) out[i] = i;
  }
}

}  // namespace

extern "C" {

const char* tpm_version(void) { return "tpmlp 0.1 (gfx950)"; }
const char* tpm_last_error(void) { return g_err; }

int tpm_set_wait_limit(uint32_t polls) {
  g_wait_limit = polls == 0 ? 1 : polls;
  return TPM_OK;
}

size_t tpm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int T, int num_chunks, int dtype) {
  if (M < 0 || N < 0 || K < 0 || num_chunks < 1) return 0;
  switch (op) {
    case TPM_OP_SEQ_CHUNK_GEMM:
      return kCtrlBytes + plan_bytes(M, N, K, num_chunks, dtype);
    case TPM_OP_LINEAR_BWD: {
      int S[2];
      plan_linear_bwd(M, N, K, dtype, S);
      return kCtrlBytes + partial_bytes(K, N, S[0]) + partial_bytes(M, K, S[1]);
    }
    case TPM_OP_MLP_FWD: {
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      const size_t hq = dtype == TPM_FP8_E4M3 ? round_up((size_t)M * (size_t)Ft, 256) : 0;
      const size_t part = std::max(plan_bytes(M, Ft, D, num_chunks, dtype),
                                   plan_bytes(M, D, Ft, T, dtype));
      return kCtrlBytes + hq + part;
    }
    case TPM_OP_MLP_BWD: {
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      const size_t dz = round_up((size_t)M * (size_t)Ft * (size_t)esize(dtype == TPM_F32 ? TPM_F32 : TPM_BF16), 256);
      size_t part = plan_bytes(M, Ft, D, num_chunks, dtype);
      part = std::max(part, plan_bytes(Ft, D, M, 1, dtype));
      part = std::max(part, plan_bytes(D, Ft, M, 1, dtype));
      part = std::max(part, plan_bytes(M, D, Ft, 1, dtype));
      return kCtrlBytes + dz + part;
    }
    case TPM_OP_MX_MLP_FWD: {   // GEMM1 writes MXFP8 whole tiles: only GEMM2 may split
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      return kCtrlBytes + plan_bytes(M, D, Ft, T, TPM_FP8_E4M3);
    }
    case TPM_OP_FP8_DELAYED_MLP_FWD: {
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      return kCtrlBytes + std::max(plan_bytes(M, Ft, D, num_chunks, TPM_FP8_E4M3),
                                   plan_bytes(M, D, Ft, T, TPM_FP8_E4M3));
    }
    case TPM_OP_CAST_FP8:
      return kCtrlBytes;
    case TPM_OP_MLP_BWD_FP8: {
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      const int f8 = TPM_FP8_E4M3;
      size_t part = plan_bytes(M, Ft, D, 1, f8);
      part = std::max(part, plan_bytes(Ft, D, M, 1, f8));
      part = std::max(part, plan_bytes(D, Ft, M, 1, f8));
      part = std::max(part, plan_bytes(M, D, Ft, 1, f8));
      const size_t md = round_up((size_t)M * (size_t)D, 256), mf = round_up((size_t)M * (size_t)Ft, 256);
      return kCtrlBytes + 3 * md + 2 * mf + 3 * mf + part;   // dY8, dY8^T, X8^T; dZ (bf16); dZ8, dZ8^T, H8^T
    }
    case TPM_OP_GATED_MLP_FWD: {
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      return kCtrlBytes + plan_bytes(M, D, Ft, T, dtype);
    }
    case TPM_OP_GATED_MLP_BWD: {
      if (T <= 0) return 0;
      const int64_t D = N, Ft = K / T;
      const size_t dgu = round_up((size_t)M * (size_t)(2 * Ft) * 2, 256);
      size_t part = plan_bytes(M, Ft, D, num_chunks, dtype);
      part = std::max(part, plan_bytes(Ft, D, M, 1, dtype));
      part = std::max(part, plan_bytes(D, 2 * Ft, M, 1, dtype));
      part = std::max(part, plan_bytes(M, D, 2 * Ft, 1, dtype));
      return kCtrlBytes + dgu + part;
    }
    default: return 0;
  }
}

int tpm_write_chunks(void* dst, const void* src, int64_t chunk_bytes, int num_chunks, const int32_t* order,
                     const uint8_t* copy, uint32_t* ready, uint32_t epoch, uint32_t* counters, void* stream) {
  const char* who = "tpm_write_chunks";
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks out of range", who);
  if (chunk_bytes < 0 || chunk_bytes % 16 != 0) return fail(TPM_EINVAL, "%s: chunk_bytes must be a multiple of 16", who);
  if (!order || !ready || !counters) return fail(TPM_EINVAL, "%s: null order, ready or counters", who);
  if (chunk_bytes > 0 && (!dst || !src)) return fail(TPM_EINVAL, "%s: null buffer", who);
  if ((((uintptr_t)dst | (uintptr_t)src) & 15) != 0) return fail(TPM_EINVAL, "%s: buffers must be 16-byte aligned", who);
  WriterParams p;
  std::memset(&p, 0, sizeof(p));
  std::vector<int> seen(num_chunks, 0);
  for (int i = 0; i < num_chunks; ++i) {
    const int c = order[i];
    if (c < 0 || c >= num_chunks || seen[c]++) return fail(TPM_EINVAL, "%s: order is not a permutation", who);
    p.order[i] = (int16_t)c;
  }
  for (int c = 0; c < num_chunks; ++c) p.copy[c] = (uint8_t)(copy ? (copy[c] != 0) : 1);
  p.src = (const char*)src;
  p.dst = (char*)dst;
  p.chunk_bytes = chunk_bytes;
  p.ready = ready;
  p.counters = counters;
  p.epoch = epoch;
  p.n = num_chunks;
  // one work-group per CU of the stream's mask (a producer stream confined
  // to a few CUs), 8 on a stream that may use every CU
  const hipStream_t s = (hipStream_t)stream;
  const int avail = stream_cus(s);
  const int groups = std::max(1, std::min(64, avail == num_cus() ? 8 : avail));
  hipError_t e = launch_write_chunks(p, groups, s);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

int tpm_signal_chunk(void* stream, uint32_t* flag, uint32_t value) {
  if (!flag) return fail(TPM_EINVAL, "tpm_signal_chunk: null flag");
  hipError_t e = launch_signal(flag, value, (hipStream_t)stream);
  return e == hipSuccess ? TPM_OK : hip_fail(e, "tpm_signal_chunk");
}

int tpm_poll_device_error(const void* workspace) {
  if (!workspace) return fail(TPM_EWORKSPACE, "tpm_poll_device_error: null workspace");
  uint32_t w = 0;
  hipError_t e = hipMemcpy(&w, workspace, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "tpm_poll_device_error");
  if (w == kErrTimeout) return fail(TPM_ETIMEOUT, "a device-side chunk wait gave up (watchdog)");
  return TPM_OK;
}

int seq_chunk_gemm(int64_t M, int64_t N, int64_t K,
                   const void* A, int64_t lda, int trans_a, int a_dtype, const float* a_scale,
                   const void* B, int64_t ldb, int trans_b, int b_dtype, const float* b_scale,
                   void* Y, int64_t ldy, int y_dtype,
                   int epilogue, int act, void* aux, int64_t ldaux, float* amax_out,
                   int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "seq_chunk_gemm";
  uint32_t* ctrl = ctrl_of(workspace, workspace_bytes);
  if ((chunk_ready || amax_out) && workspace && !ctrl)
    return fail(TPM_EWORKSPACE, "%s: workspace smaller than %zu bytes", who, kCtrlBytes);
  GemmDesc g{M, N, K, A, lda, trans_a != 0, a_dtype, a_scale, B, ldb, trans_b != 0, b_dtype, b_scale,
             Y, ldy, y_dtype, epilogue, act, aux, ldaux, amax_out,
             num_chunks, chunk_order, chunk_ready, nullptr, epoch, ctrl};
  if (ctrl) {
    g.part = (float*)((char*)workspace + kCtrlBytes);
    g.part_bytes = workspace_bytes - kCtrlBytes;
  }
  int rc = check_gemm(g, who);
  if (rc != TPM_OK) return rc;
  if (amax_out && a_dtype == TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: amax on the fp32 path", who);
  hipStream_t s = (hipStream_t)stream;
  if (M == 0 || N == 0) return TPM_OK;
  if (chunk_ready || amax_out) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
    if (amax_out) {
      e = launch_ctrl_init((uint32_t*)amax_out, 1, s);
      if (e != hipSuccess) return hip_fail(e, who);
    }
  }
  return run_gemm(g, s, who);
}

}  // extern "C"

// ---------------------------------------------------- allocation-free calls
namespace {

// The scratch of seq_chunk_gemm_noalloc: control words, then the fp32
// split-K partial sums.  One copy per GPU, held until the process ends.
constexpr size_t kNoAllocScratchBytes = kCtrlBytes + (size_t(64) << 20);
static_assert(kNoAllocScratchBytes == TPM_NOALLOC_SCRATCH_BYTES, "header constant");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device with that device current (the host-side name is only a stand-in).
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {nullptr};

int scratch_on_current_device(void** out, const char* who) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, who);
  if (dev < 0 || dev >= 64) return fail(TPM_EUNSUPPORTED, "%s: device index %d", who, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return e != hipSuccess ? hip_fail(e, who) : fail(TPM_EHIP, "%s: no scratch", who);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TPM_OK;
}

}  // namespace

extern "C" {

int seq_chunk_gemm_noalloc(int64_t M, int64_t N, int64_t K,
                           const void* A, int64_t lda, int trans_a, int a_dtype, const float* a_scale,
                           const void* B, int64_t ldb, int trans_b, int b_dtype, const float* b_scale,
                           void* Y, int64_t ldy, int y_dtype,
                           int epilogue, int act, void* aux, int64_t ldaux, float* amax_out,
                           int num_chunks, const int32_t* chunk_order, void* stream) {
  const char* who = "seq_chunk_gemm_noalloc";
  // validation and the split plan on the host, before any device call; a
  // non-null placeholder stands for the control words until the device's
  // scratch address is known
  GemmDesc g{M, N, K, A, lda, trans_a != 0, a_dtype, a_scale, B, ldb, trans_b != 0, b_dtype, b_scale,
             Y, ldy, y_dtype, epilogue, act, aux, ldaux, amax_out,
             num_chunks, chunk_order, nullptr, nullptr, 0, reinterpret_cast<uint32_t*>(uintptr_t(256))};
  int rc = check_gemm(g, who);
  if (rc != TPM_OK) return rc;
  if (amax_out && a_dtype == TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: amax on the fp32 path", who);
  if (M == 0 || N == 0) return TPM_OK;
  const size_t need = kCtrlBytes + plan_bytes(planned_split(g), M, N, num_chunks);
  if (need > kNoAllocScratchBytes)
    return fail(TPM_EUNSUPPORTED, "%s: this GEMM's split-K plan needs %zu bytes of scratch, more than the %zu the "
                "library holds per GPU; call seq_chunk_gemm with a workspace", who, need, kNoAllocScratchBytes);
  void* base = nullptr;
  rc = scratch_on_current_device(&base, who);
  if (rc != TPM_OK) return rc;
  g.ctrl = (uint32_t*)base;
  g.part = (float*)((char*)base + kCtrlBytes);
  g.part_bytes = kNoAllocScratchBytes - kCtrlBytes;
  hipStream_t s = (hipStream_t)stream;
  if (amax_out) {
    hipError_t e = launch_ctrl_init((uint32_t*)amax_out, 1, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  return run_gemm(g, s, who);
}

int tp_mlp_fwd(int64_t M, int64_t D, int64_t F, int T, int rank,
               const void* X, const void* W_up_t, const void* W_down_t,
               int dtype, const float* scales, int act,
               void* Z_t, void* H_t, void* P_t, float* h_scale_out,
               int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
               const int32_t* range_order, uint32_t* range_done,
               void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_mlp_fwd";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0) return fail(TPM_EINVAL, "%s: F %% T != 0", who);
  if (M % T != 0) return fail(TPM_EINVAL, "%s: M %% T != 0", who);
  if (!valid_dt(dtype)) return fail(TPM_EINVAL, "%s: bad dtype", who);
  if (dtype == TPM_FP8_E4M3 && !scales) return fail(TPM_EINVAL, "%s: fp8 needs scales", who);
  if (dtype == TPM_FP8_E4M3 && (F / T) % 8 != 0)
    return fail(TPM_EUNSUPPORTED, "%s: fp8 needs F/T %% 8 == 0 (H is quantised 8 columns at a time)", who);
  if (!H_t || !P_t) return fail(TPM_EINVAL, "%s: null H_t or P_t", who);
  const int64_t Ft = F / T;
  const size_t need = tpm_workspace_bytes(TPM_OP_MLP_FWD, M, D, F, T, num_chunks, dtype);
  const bool need_ctrl = chunk_ready || range_done || dtype == TPM_FP8_E4M3;
  if (need_ctrl && (!workspace || workspace_bytes < need))
    return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  uint32_t* ctrl = (workspace && workspace_bytes >= kCtrlBytes) ? (uint32_t*)workspace : nullptr;
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  int32_t corder[TPM_MAX_CHUNKS], rorder[TPM_MAX_CHUNKS];
  if (chunk_order) std::memcpy(corder, chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  if (range_order) std::memcpy(rorder, range_order, sizeof(int32_t) * T);
  else for (int i = 0; i < T; ++i) rorder[i] = (rank + 1 + i) % T;

  const int ydt = dtype == TPM_F32 ? TPM_F32 : TPM_BF16;
  const bool fp8 = dtype == TPM_FP8_E4M3;
  float* amax = fp8 ? (float*)(ctrl + kCtrlAmax) : nullptr;
  // GEMM1: column-parallel, chunk-fed.  bf16 / fp32 weights are the pages'
  // W[K,N]; fp8 weights are stored K-major (W_up,t as [F/T, D], W_down,t as
  // [D, F/T]), the transposed copies the fp8 recipes keep, as B^T.
  GemmDesc g1{M, Ft, D, X, D, false, dtype, fp8 ? scales + 0 : nullptr,
              W_up_t, fp8 ? D : Ft, fp8, dtype, fp8 ? scales + 1 : nullptr,
              H_t, Ft, ydt, TPM_EPI_FWD, act, Z_t, Ft, amax,
              num_chunks, corder, chunk_ready, nullptr, epoch, ctrl};
  int rc = check_gemm(g1, who);
  if (rc != TPM_OK) return rc;
  uint8_t* hq = fp8 ? (uint8_t*)workspace + kCtrlBytes : nullptr;
  float* sH = fp8 ? (h_scale_out ? h_scale_out : (float*)(ctrl + kCtrlScale)) : nullptr;
  GemmDesc g2{M, D, Ft, fp8 ? (const void*)hq : (const void*)H_t, Ft, false, dtype, sH,
              W_down_t, fp8 ? Ft : D, fp8, dtype, fp8 ? scales + 2 : nullptr,
              P_t, D, ydt, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
              T, rorder, nullptr, range_done, epoch, ctrl};
  rc = check_gemm(g2, who);
  if (rc != TPM_OK) return rc;
  if (workspace && workspace_bytes >= need) {
    const size_t hq_bytes = fp8 ? round_up((size_t)M * (size_t)Ft, 256) : 0;
    g1.part = g2.part = (float*)((char*)workspace + kCtrlBytes + hq_bytes);
    g1.part_bytes = g2.part_bytes = workspace_bytes - kCtrlBytes - hq_bytes;
  }
  if (M == 0 || D == 0) return TPM_OK;
  hipStream_t s = (hipStream_t)stream;
  if (need_ctrl) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  rc = run_gemm(g1, s, who);
  if (rc != TPM_OK) return rc;
  if (fp8) {
    hipError_t e = launch_quant_e4m3((const uint16_t*)H_t, M, Ft, Ft, amax, hq, Ft, sH, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  return run_gemm(g2, s, who);
}

int tp_linear_bwd(int64_t M, int64_t N, int64_t K,
                  const void* X, const void* W, const void* dY, int dtype,
                  void* dW, void* dX, int dw_dtype,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_linear_bwd";
  if (M < 0 || N < 0 || K < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (dtype != TPM_BF16 && dtype != TPM_F32) return fail(TPM_EINVAL, "%s: dtype BF16 or F32", who);
  if (dw_dtype != TPM_BF16 && dw_dtype != TPM_F32) return fail(TPM_EINVAL, "%s: dw_dtype", who);
  if (dtype == TPM_F32 && dw_dtype != TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: fp32 inputs give fp32 dW", who);
  // every array with elements needs a pointer (empty ones may be null)
  auto given = [](const void* p, int64_t rows, int64_t cols) { return p != nullptr || rows == 0 || cols == 0; };
  if (!given(X, M, K) || !given(W, K, N) || !given(dY, M, N) || !given(dW, K, N) || !given(dX, M, K))
    return fail(TPM_EINVAL, "%s: null pointer", who);
  const size_t need = tpm_workspace_bytes(TPM_OP_LINEAR_BWD, M, N, K, 1, 1, dtype);
  if (!workspace || workspace_bytes < need) return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  uint32_t* ctrl = (uint32_t*)workspace;
  // dW = X^T . dY    [K, N], contraction over M; X [M, K] stored: op(A) = X^T
  GemmDesc g_dw{K, N, M, X, K, true, dtype, nullptr, dY, N, false, dtype, nullptr,
                dW, N, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, 0, ctrl};
  // dX = dY . W^T    [M, K], contraction over N; W [K, N] stored: op(B) = W^T
  GemmDesc g_dx{M, K, N, dY, N, false, dtype, nullptr, W, N, true, dtype, nullptr,
                dX, K, dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, 0, ctrl};
  int S[2];
  plan_linear_bwd(M, N, K, dtype, S);
  g_dw.part = (float*)((char*)workspace + kCtrlBytes);
  g_dw.part_bytes = partial_bytes(K, N, S[0]);
  g_dx.part = (float*)((char*)workspace + kCtrlBytes + g_dw.part_bytes);
  g_dx.part_bytes = partial_bytes(M, K, S[1]);
  for (const GemmDesc* g : {&g_dw, &g_dx}) {
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  hipStream_t s = (hipStream_t)stream;
  if (dtype != TPM_BF16 || K == 0 || N == 0 || M == 0 || fast_path_blocker(g_dw) || fast_path_blocker(g_dx)) {
    // fp32, ragged or unaligned shapes (the predicated kernel), or one
    // product empty: the two products one after the other
    for (const GemmDesc* g : {&g_dw, &g_dx}) {
      int rc = run_gemm(*g, s, who);
      if (rc != TPM_OK) return rc;
    }
    return TPM_OK;
  }
  GemmParams p_dw, p_dx;
  make_params(g_dw, SplitPlan{S[0]}, p_dw);
  make_params(g_dx, SplitPlan{S[1]}, p_dx);
  const int units = p_dw.units + p_dx.units;
  // at least one work-group per XCD queue, at most one per CU the stream may use
  const int grid = std::max(8, std::min(stream_cus(s), units));
  const int first = p_dx.ksteps_per_split > p_dw.ksteps_per_split ? 1 : 0;
  hipError_t e = launch_ctrl_init(ctrl + kCtrlQueue, 8, s);
  if (e == hipSuccess) e = launch_gemm_pair_bf16(p_dw, false, false, p_dx, true, true, first, ctrl + kCtrlQueue, grid, s);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

int tp_mlp_bwd(int64_t M, int64_t D, int64_t F, int T, int rank,
               const void* X, const void* W_up_t, const void* W_down_t,
               const void* Z_t, const void* H_t, const void* dY,
               int dtype, int act,
               void* dW_up_t, void* dW_down_t, void* dX_t, int dw_dtype,
               int num_chunks, const int32_t* dy_chunk_order, const uint32_t* dy_ready, uint32_t epoch,
               void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_mlp_bwd";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0 || M % T != 0) return fail(TPM_EINVAL, "%s: F %% T or M %% T != 0", who);
  if (dtype != TPM_BF16 && dtype != TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: backward dtype BF16 or F32", who);
  if (dw_dtype != TPM_BF16 && dw_dtype != TPM_F32) return fail(TPM_EINVAL, "%s: dw_dtype", who);
  if (dtype == TPM_F32 && dw_dtype != TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: fp32 inputs give fp32 dW", who);
  if (!Z_t || !H_t || !dY || !dW_up_t || !dW_down_t || !dX_t || !X || !W_up_t || !W_down_t)
    return fail(TPM_EINVAL, "%s: null pointer", who);
  const int64_t Ft = F / T;
  const size_t need = tpm_workspace_bytes(TPM_OP_MLP_BWD, M, D, F, T, num_chunks, dtype);
  if (!workspace || workspace_bytes < need) return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  uint32_t* ctrl = (uint32_t*)workspace;
  void* dZ = (char*)workspace + kCtrlBytes;
  int32_t corder[TPM_MAX_CHUNKS];
  if (dy_chunk_order) std::memcpy(corder, dy_chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  const int adt = dtype, zdt = dtype == TPM_F32 ? TPM_F32 : TPM_BF16;
  // dZ = (dY . W_down^T) * act'(Z)           W_down_t [Ft, D]: op(B) = W_down^T, stored [N=Ft, K=D]
  GemmDesc g_dz{M, Ft, D, dY, D, false, adt, nullptr, W_down_t, D, true, adt, nullptr,
                dZ, Ft, zdt, TPM_EPI_DACT, act, const_cast<void*>(Z_t), Ft, nullptr,
                num_chunks, corder, dy_ready, nullptr, epoch, ctrl};
  // dW_down = H^T . dY                        H [M, Ft] stored: op(A) = H^T
  GemmDesc g_wd{Ft, D, M, H_t, Ft, true, adt, nullptr, dY, D, false, adt, nullptr,
                dW_down_t, D, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, epoch, ctrl};
  // dW_up = X^T . dZ
  GemmDesc g_wu{D, Ft, M, X, D, true, adt, nullptr, dZ, Ft, false, adt, nullptr,
                dW_up_t, Ft, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, epoch, ctrl};
  // dX = dZ . W_up^T                          W_up_t [D, Ft]: op(B) = W_up^T, stored [N=D, K=Ft]
  GemmDesc g_dx{M, D, Ft, dZ, Ft, false, adt, nullptr, W_up_t, Ft, true, adt, nullptr,
                dX_t, D, zdt, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, epoch, ctrl};
  {
    const size_t dz_bytes = round_up((size_t)M * (size_t)Ft * (size_t)esize(zdt), 256);
    for (GemmDesc* g : {&g_dz, &g_wd, &g_wu, &g_dx}) {
      g->part = (float*)((char*)workspace + kCtrlBytes + dz_bytes);
      g->part_bytes = workspace_bytes - kCtrlBytes - dz_bytes;
    }
  }
  for (const GemmDesc* g : {&g_dz, &g_wd, &g_wu, &g_dx}) {
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  hipStream_t s = (hipStream_t)stream;
  if (dy_ready) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  for (const GemmDesc* g : {&g_dz, &g_wd, &g_wu, &g_dx}) {
    int rc = run_gemm(*g, s, who);
    if (rc != TPM_OK) return rc;
  }
  return TPM_OK;
}

size_t tpm_mx_scales_bytes(int64_t rows, int64_t k) {
  if (rows < 0 || k < 0) return 0;
  return mx_scales_bytes(rows, k);
}

int tpm_mx_swizzle_scales(int64_t rows, int64_t k, const uint8_t* src, int64_t ld, uint8_t* dst, void* stream) {
  const char* who = "tpm_mx_swizzle_scales";
  if (rows < 0 || k < 0 || k % 128 != 0) return fail(TPM_EINVAL, "%s: rows >= 0 and k %% 128 == 0 required", who);
  if (rows > INT32_MAX / 2 || k / 32 > INT32_MAX) return fail(TPM_EUNSUPPORTED, "%s: too large", who);
  if (rows == 0 || k == 0) return TPM_OK;
  if (!src || !dst || ld < k / 32) return fail(TPM_EINVAL, "%s: null pointer or ld < k/32", who);
  hipError_t e = launch_mx_swizzle(src, ld, (int)rows, (int)(k / 32), dst, (hipStream_t)stream);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

// control words of the fp8 backward (after the per-group counters)
constexpr int kCtrlF8 = kCtrlWords + 4;
static_assert((kCtrlF8 + 8) * 4 <= (int)kCtrlBytes, "control block");

int tpm_cast_fp8(int64_t rows, int64_t cols, const void* x, int64_t ld, int dtype,
                 void* q, int64_t ldq, void* qt, int64_t ldqt, float* scale_out,
                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tpm_cast_fp8";
  if (dtype != TPM_FP8_E4M3 && dtype != TPM_FP8_E5M2) return fail(TPM_EINVAL, "%s: dtype must be fp8", who);
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0)
    return fail(TPM_EUNSUPPORTED, "%s: rows and cols must be multiples of 16", who);
  if (!workspace || workspace_bytes < kCtrlBytes) return fail(TPM_EWORKSPACE, "%s: workspace required", who);
  if (rows == 0 || cols == 0) return TPM_OK;
  if (!x || ld < cols || ld % 8 != 0 || !aligned16(x)) return fail(TPM_EINVAL, "%s: x, ld", who);
  if ((q && (ldq < cols || ldq % 16 != 0 || !aligned16(q))) || (qt && (ldqt < rows || ldqt % 16 != 0 || !aligned16(qt))))
    return fail(TPM_EINVAL, "%s: output leading dimensions / alignment", who);
  hipStream_t s = (hipStream_t)stream;
  uint32_t* amax = (uint32_t*)workspace + kCtrlF8;
  hipError_t e = launch_ctrl_init(amax, 1, s);
  if (e == hipSuccess) e = launch_amax_bf16((const uint16_t*)x, rows, cols, ld, amax, s);
  if (e == hipSuccess)
    e = launch_cast_fp8_t((const uint16_t*)x, rows, cols, ld, (const float*)amax, dtype == TPM_FP8_E5M2,
                          (uint8_t*)q, ldq, (uint8_t*)qt, ldqt, scale_out, s);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

int tp_mlp_bwd_fp8(int64_t M, int64_t D, int64_t F, int T, int rank,
                   const void* X, const void* W_up_t, const void* W_down_t, const float* scales,
                   const void* Z_t, const void* H_t, const void* dY, int dy_dtype, const float* dy_scale, int act,
                   void* dW_up_t, void* dW_down_t, void* dX_t, int dw_dtype,
                   int num_chunks, const int32_t* dy_chunk_order, const uint32_t* dy_ready, uint32_t epoch,
                   void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_mlp_bwd_fp8";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0 || M % T != 0) return fail(TPM_EINVAL, "%s: F %% T or M %% T != 0", who);
  const int64_t Ft = F / T;
  if (M % 16 != 0 || D % 16 != 0 || Ft % 16 != 0) return fail(TPM_EUNSUPPORTED, "%s: M, D, F/T multiples of 16", who);
  if (dw_dtype != TPM_BF16 && dw_dtype != TPM_F32) return fail(TPM_EINVAL, "%s: dw_dtype", who);
  if (dy_dtype != TPM_BF16 && dy_dtype != TPM_FP8_E5M2) return fail(TPM_EINVAL, "%s: dy_dtype BF16 or FP8_E5M2", who);
  const bool dy_codes = dy_dtype == TPM_FP8_E5M2;
  if (dy_codes && !dy_scale) return fail(TPM_EINVAL, "%s: e5m2 dY needs dy_scale", who);
  if (!dy_codes && dy_ready)
    return fail(TPM_EUNSUPPORTED, "%s: a chunk-fed dY must arrive quantised (dy_dtype FP8_E5M2): the current "
                "scale of a bf16 dY needs every row", who);
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  if (!X || !W_up_t || !W_down_t || !scales || !Z_t || !H_t || !dY || !dW_up_t || !dW_down_t || !dX_t)
    return fail(TPM_EINVAL, "%s: null pointer", who);
  const size_t need = tpm_workspace_bytes(TPM_OP_MLP_BWD_FP8, M, D, F, T, num_chunks, TPM_FP8_E4M3);
  if (!workspace || workspace_bytes < need) return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  if (!aligned16(dY) || !aligned16(H_t)) return fail(TPM_EUNSUPPORTED, "%s: dY, H_t must be 16-byte aligned", who);
  uint32_t* ctrl = (uint32_t*)workspace;
  float* cw = (float*)(ctrl + kCtrlF8);   // amax dY, s dY, amax dZ, s dZ, amax H, s H
  const size_t md = round_up((size_t)M * (size_t)D, 256), mf = round_up((size_t)M * (size_t)Ft, 256);
  char* w = (char*)workspace + kCtrlBytes;
  uint8_t* dy8 = (uint8_t*)w;              w += md;
  uint8_t* dy8t = (uint8_t*)w;             w += md;
  uint8_t* x8t = (uint8_t*)w;              w += md;
  uint16_t* dz = (uint16_t*)w;             w += 2 * mf;
  uint8_t* dz8 = (uint8_t*)w;              w += mf;
  uint8_t* dz8t = (uint8_t*)w;             w += mf;
  uint8_t* h8t = (uint8_t*)w;              w += mf;
  float* part = (float*)w;
  const size_t part_bytes = workspace_bytes - (size_t)(w - (char*)workspace);
  const int e4 = TPM_FP8_E4M3, e5 = TPM_FP8_E5M2;
  // dY's codes and dequantisation factor: the caller's (chunk-fed), or this
  // call's current-scaling cast of the bf16 dY
  const uint8_t* dyq = dy_codes ? (const uint8_t*)dY : dy8;
  const float* s_dy = dy_codes ? dy_scale : cw + 1;
  int32_t corder[TPM_MAX_CHUNKS];
  if (dy_chunk_order) std::memcpy(corder, dy_chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  // dZ = (dYq . W_down^T) * act'(Z), bf16, amax   W_down_t [Ft, D]: stored [N=Ft, K=D]; chunk-fed by dY rows
  GemmDesc g_dz{M, Ft, D, dyq, D, false, e5, s_dy, W_down_t, D, true, e4, scales + 2,
                dz, Ft, TPM_BF16, TPM_EPI_DACT, act, const_cast<void*>(Z_t), Ft, cw + 2,
                num_chunks, corder, dy_ready, nullptr, epoch, ctrl};
  // dW_down = H^T . dY:  A = H8^T [Ft, M], B stored [N=D, K=M] = dYq^T
  GemmDesc g_wd{Ft, D, M, h8t, M, false, e4, cw + 5, dy8t, M, true, e5, s_dy,
                dW_down_t, D, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, 0, ctrl};
  // dW_up = X^T . dZ:  A = X8^T [D, M], B stored [N=Ft, K=M] = dZ8^T
  GemmDesc g_wu{D, Ft, M, x8t, M, false, e4, scales + 0, dz8t, M, true, e5, cw + 3,
                dW_up_t, Ft, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, 0, ctrl};
  // dX = dZ . W_up^T:  A = dZ8 [M, Ft], B stored [N=D, K=Ft] = W_up_t [D, Ft]
  GemmDesc g_dx{M, D, Ft, dz8, Ft, false, e5, cw + 3, W_up_t, Ft, true, e4, scales + 1,
                dX_t, D, TPM_BF16, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, 0, ctrl};
  for (GemmDesc* g : {&g_dz, &g_wd, &g_wu, &g_dx}) {
    g->part = part;
    g->part_bytes = part_bytes;
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  if (M == 0 || D == 0 || Ft == 0) return TPM_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_ctrl_init(ctrl, kCtrlF8 + 8, s);
  // activation casts (independent of dY): H -> e4m3 transposed, X transposed
  if (e == hipSuccess) e = launch_amax_bf16((const uint16_t*)H_t, M, Ft, Ft, (uint32_t*)(cw + 4), s);
  if (e == hipSuccess) e = launch_cast_fp8_t((const uint16_t*)H_t, M, Ft, Ft, cw + 4, false, nullptr, 0, h8t, M, cw + 5, s);
  if (e == hipSuccess) e = launch_transpose_u8((const uint8_t*)X, M, D, D, x8t, M, s);
  // bf16 dY: its current-scaling cast to e5m2, row-major and transposed
  if (!dy_codes) {
    if (e == hipSuccess) e = launch_amax_bf16((const uint16_t*)dY, M, D, D, (uint32_t*)(cw + 0), s);
    if (e == hipSuccess) e = launch_cast_fp8_t((const uint16_t*)dY, M, D, D, cw + 0, true, dy8, D, dy8t, M, cw + 1, s);
  }
  if (e != hipSuccess) return hip_fail(e, who);
  int rc = run_gemm(g_dz, s, who);
  if (rc != TPM_OK) return rc;
  // e5m2 dY: every chunk has landed once the dZ GEMM is done; its transposed copy for dW_down
  if (dy_codes) e = launch_transpose_u8(dyq, M, D, D, dy8t, M, s);
  if (e == hipSuccess) e = launch_cast_fp8_t(dz, M, Ft, Ft, cw + 2, true, dz8, Ft, dz8t, M, cw + 3, s);
  if (e != hipSuccess) return hip_fail(e, who);
  for (const GemmDesc* g : {&g_wd, &g_wu, &g_dx}) {
    rc = run_gemm(*g, s, who);
    if (rc != TPM_OK) return rc;
  }
  return TPM_OK;
}

int tpm_fp8_delayed_scale(const float* amax_history, int n, float* scale_out, void* stream) {
  const char* who = "tpm_fp8_delayed_scale";
  if (n < 1 || !amax_history || !scale_out) return fail(TPM_EINVAL, "%s: n >= 1 and non-null pointers", who);
  hipError_t e = launch_delayed_scale(amax_history, n, scale_out, (hipStream_t)stream);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

int tp_mlp_fwd_delayed(int64_t M, int64_t D, int64_t F, int T, int rank,
                       const void* X, const void* W_up_t, const void* W_down_t, const float* scales,
                       const float* h_scale, float* h_amax_out, int act,
                       void* Z_t, void* H_t, void* P_t,
                       int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                       const int32_t* range_order, uint32_t* range_done,
                       void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_mlp_fwd_delayed";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0 || M % T != 0) return fail(TPM_EINVAL, "%s: F %% T or M %% T != 0", who);
  if (!scales || !h_scale || !H_t || !P_t) return fail(TPM_EINVAL, "%s: null pointer", who);
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  const int64_t Ft = F / T;
  const size_t need = tpm_workspace_bytes(TPM_OP_FP8_DELAYED_MLP_FWD, M, D, F, T, num_chunks, TPM_FP8_E4M3);
  const bool need_ctrl = chunk_ready || range_done || h_amax_out;
  if (need_ctrl && (!workspace || workspace_bytes < need))
    return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  uint32_t* ctrl = (workspace && workspace_bytes >= kCtrlBytes) ? (uint32_t*)workspace : nullptr;
  int32_t corder[TPM_MAX_CHUNKS], rorder[TPM_MAX_CHUNKS];
  if (chunk_order) std::memcpy(corder, chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  if (range_order) std::memcpy(rorder, range_order, sizeof(int32_t) * T);
  else for (int i = 0; i < T; ++i) rorder[i] = (rank + 1 + i) % T;
  const int f8 = TPM_FP8_E4M3;
  // GEMM1: H = e4m3(act(X W_up) / s_H), chunk-fed; amax of act(.) recorded
  GemmDesc g1{M, Ft, D, X, D, false, f8, scales + 0, W_up_t, D, true, f8, scales + 1,
              H_t, Ft, f8, TPM_EPI_FWD, act, Z_t, Ft, h_amax_out,
              num_chunks, corder, chunk_ready, nullptr, epoch, ctrl};
  g1.y_qs = h_scale;
  // GEMM2: P = (Hq W_down) s_H s_Wdown
  GemmDesc g2{M, D, Ft, H_t, Ft, false, f8, h_scale, W_down_t, Ft, true, f8, scales + 2,
              P_t, D, TPM_BF16, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
              T, rorder, nullptr, range_done, epoch, ctrl};
  for (const GemmDesc* g : {&g1, &g2}) {
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  if (workspace && workspace_bytes >= need) {
    g1.part = g2.part = (float*)((char*)workspace + kCtrlBytes);
    g1.part_bytes = g2.part_bytes = workspace_bytes - kCtrlBytes;
  }
  if (M == 0 || D == 0) return TPM_OK;
  hipStream_t s = (hipStream_t)stream;
  if (need_ctrl) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  if (h_amax_out) {
    hipError_t e = launch_ctrl_init((uint32_t*)h_amax_out, 1, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  int rc = run_gemm(g1, s, who);
  if (rc != TPM_OK) return rc;
  return run_gemm(g2, s, who);
}

int seq_chunk_gemm_mx(int64_t M, int64_t N, int64_t K,
                      const void* A, int64_t lda, const uint8_t* a_scales,
                      const void* B, int64_t ldb, const uint8_t* b_scales,
                      void* Y, int64_t ldy, int y_dtype, uint8_t* y_scales,
                      int act, void* aux, int64_t ldaux,
                      int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "seq_chunk_gemm_mx";
  uint32_t* ctrl = ctrl_of(workspace, workspace_bytes);
  if (chunk_ready && !ctrl) return fail(TPM_EWORKSPACE, "%s: workspace smaller than %zu bytes", who, kCtrlBytes);
  if (!a_scales || !b_scales) return fail(TPM_EINVAL, "%s: null scales", who);
  GemmDesc g{M, N, K, A, lda, false, TPM_FP8_E4M3, nullptr, B, ldb, true, TPM_FP8_E4M3, nullptr,
             Y, ldy, y_dtype, TPM_EPI_FWD, act, aux, ldaux, nullptr,
             num_chunks, chunk_order, chunk_ready, nullptr, epoch, ctrl};
  g.a_mx = a_scales;
  g.b_mx = b_scales;
  g.y_mx = y_dtype == TPM_FP8_E4M3 ? y_scales : nullptr;
  if (y_dtype == TPM_FP8_E4M3 && !y_scales) return fail(TPM_EINVAL, "%s: MXFP8 output needs y_scales", who);
  if (aux && y_dtype == TPM_F32) return fail(TPM_EUNSUPPORTED, "%s: aux with an fp32 output", who);
  if (ctrl) {
    g.part = (float*)((char*)workspace + kCtrlBytes);
    g.part_bytes = workspace_bytes - kCtrlBytes;
  }
  int rc = check_gemm(g, who);
  if (rc != TPM_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  if (M == 0 || N == 0) return TPM_OK;
  if (chunk_ready) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  return run_gemm(g, s, who);
}

int tp_mlp_fwd_mx(int64_t M, int64_t D, int64_t F, int T, int rank,
                  const void* X, const uint8_t* x_scales, const void* W_up_t, const uint8_t* w_up_scales,
                  const void* W_down_t, const uint8_t* w_down_scales, int act,
                  void* Z_t, void* H_t, uint8_t* h_scales, void* P_t,
                  int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                  const int32_t* range_order, uint32_t* range_done,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_mlp_fwd_mx";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0 || M % T != 0) return fail(TPM_EINVAL, "%s: F %% T or M %% T != 0", who);
  if (!H_t || !h_scales || !P_t || !x_scales || !w_up_scales || !w_down_scales)
    return fail(TPM_EINVAL, "%s: null pointer", who);
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  const int64_t Ft = F / T;
  if (D % 128 != 0 || Ft % 128 != 0) return fail(TPM_EUNSUPPORTED, "%s: D and F/T must be multiples of 128", who);
  const size_t need = tpm_workspace_bytes(TPM_OP_MX_MLP_FWD, M, D, F, T, num_chunks, TPM_FP8_E4M3);
  const bool need_ctrl = chunk_ready || range_done;
  if (need_ctrl && (!workspace || workspace_bytes < need))
    return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  uint32_t* ctrl = (workspace && workspace_bytes >= kCtrlBytes) ? (uint32_t*)workspace : nullptr;
  int32_t corder[TPM_MAX_CHUNKS], rorder[TPM_MAX_CHUNKS];
  if (chunk_order) std::memcpy(corder, chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  if (range_order) std::memcpy(rorder, range_order, sizeof(int32_t) * T);
  else for (int i = 0; i < T; ++i) rorder[i] = (rank + 1 + i) % T;
  const int f8 = TPM_FP8_E4M3;
  // GEMM1: H = MXFP8(act(X W_up)), chunk-fed; W_up,t stored K-major [Ft, D]
  GemmDesc g1{M, Ft, D, X, D, false, f8, nullptr, W_up_t, D, true, f8, nullptr,
              H_t, Ft, f8, TPM_EPI_FWD, act, Z_t, Ft, nullptr,
              num_chunks, corder, chunk_ready, nullptr, epoch, ctrl};
  g1.a_mx = x_scales; g1.b_mx = w_up_scales; g1.y_mx = h_scales;
  // GEMM2: P = H W_down (row-parallel partial, bf16); W_down,t stored K-major [D, Ft]
  GemmDesc g2{M, D, Ft, H_t, Ft, false, f8, nullptr, W_down_t, Ft, true, f8, nullptr,
              P_t, D, TPM_BF16, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
              T, rorder, nullptr, range_done, epoch, ctrl};
  g2.a_mx = h_scales; g2.b_mx = w_down_scales;
  for (const GemmDesc* g : {&g1, &g2}) {
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  if (workspace && workspace_bytes >= need) {
    g1.part = g2.part = (float*)((char*)workspace + kCtrlBytes);
    g1.part_bytes = g2.part_bytes = workspace_bytes - kCtrlBytes;
  }
  if (M == 0 || D == 0) return TPM_OK;
  hipStream_t s = (hipStream_t)stream;
  if (need_ctrl) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  int rc = run_gemm(g1, s, who);
  if (rc != TPM_OK) return rc;
  return run_gemm(g2, s, who);
}

int tp_gated_mlp_fwd(int64_t M, int64_t D, int64_t F, int T, int rank,
                     const void* X, const void* W_gu_t, const void* W_down_t, int dtype, int act,
                     void* GU_t, void* H_t, void* P_t,
                     int num_chunks, const int32_t* chunk_order, const uint32_t* chunk_ready, uint32_t epoch,
                     const int32_t* range_order, uint32_t* range_done,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_gated_mlp_fwd";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0 || M % T != 0) return fail(TPM_EINVAL, "%s: F %% T or M %% T != 0", who);
  if (dtype != TPM_BF16) return fail(TPM_EUNSUPPORTED, "%s: the gated MLP runs in bf16", who);
  if (!H_t || !P_t) return fail(TPM_EINVAL, "%s: null H_t or P_t", who);
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  const int64_t Ft = F / T;
  const size_t need = tpm_workspace_bytes(TPM_OP_GATED_MLP_FWD, M, D, F, T, num_chunks, dtype);
  const bool need_ctrl = chunk_ready || range_done;
  if (need_ctrl && (!workspace || workspace_bytes < need))
    return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  uint32_t* ctrl = (workspace && workspace_bytes >= kCtrlBytes) ? (uint32_t*)workspace : nullptr;
  int32_t corder[TPM_MAX_CHUNKS], rorder[TPM_MAX_CHUNKS];
  if (chunk_order) std::memcpy(corder, chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  if (range_order) std::memcpy(rorder, range_order, sizeof(int32_t) * T);
  else for (int i = 0; i < T; ++i) rorder[i] = (rank + 1 + i) % T;
  // GEMM1: H = act(X W_gate) * (X W_up), chunk-fed; W_gu_t = [W_gate,t | W_up,t] [D, 2Ft]
  GemmDesc g1{M, Ft, D, X, D, false, TPM_BF16, nullptr, W_gu_t, 2 * Ft, false, TPM_BF16, nullptr,
              H_t, Ft, TPM_BF16, TPM_EPI_GATED, act, GU_t, 2 * Ft, nullptr,
              num_chunks, corder, chunk_ready, nullptr, epoch, ctrl};
  // GEMM2: row-parallel partial P = H W_down, destination ranges in order
  GemmDesc g2{M, D, Ft, H_t, Ft, false, TPM_BF16, nullptr, W_down_t, D, false, TPM_BF16, nullptr,
              P_t, D, TPM_BF16, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
              T, rorder, nullptr, range_done, epoch, ctrl};
  for (const GemmDesc* g : {&g1, &g2}) {
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  if (workspace && workspace_bytes >= need) {
    g1.part = g2.part = (float*)((char*)workspace + kCtrlBytes);
    g1.part_bytes = g2.part_bytes = workspace_bytes - kCtrlBytes;
  }
  if (M == 0 || D == 0) return TPM_OK;
  hipStream_t s = (hipStream_t)stream;
  if (need_ctrl) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  int rc = run_gemm(g1, s, who);
  if (rc != TPM_OK) return rc;
  return run_gemm(g2, s, who);
}

int tp_gated_mlp_bwd(int64_t M, int64_t D, int64_t F, int T, int rank,
                     const void* X, const void* W_gu_t, const void* W_down_t,
                     const void* GU_t, const void* H_t, const void* dY, int dtype, int act,
                     void* dW_gu_t, void* dW_down_t, void* dX_t, int dw_dtype,
                     int num_chunks, const int32_t* dy_chunk_order, const uint32_t* dy_ready, uint32_t epoch,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const char* who = "tp_gated_mlp_bwd";
  if (T < 1 || T > TPM_MAX_CHUNKS || rank < 0 || rank >= T) return fail(TPM_EINVAL, "%s: bad T/rank", who);
  if (M < 0 || D < 0 || F < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (F % T != 0 || M % T != 0) return fail(TPM_EINVAL, "%s: F %% T or M %% T != 0", who);
  if (dtype != TPM_BF16) return fail(TPM_EUNSUPPORTED, "%s: the gated MLP runs in bf16", who);
  if (dw_dtype != TPM_BF16 && dw_dtype != TPM_F32) return fail(TPM_EINVAL, "%s: dw_dtype", who);
  if (!GU_t || !H_t || !dY || !dW_gu_t || !dW_down_t || !dX_t || !X || !W_gu_t || !W_down_t)
    return fail(TPM_EINVAL, "%s: null pointer", who);
  if (num_chunks < 1 || num_chunks > TPM_MAX_CHUNKS) return fail(TPM_EINVAL, "%s: num_chunks", who);
  const int64_t Ft = F / T;
  const size_t need = tpm_workspace_bytes(TPM_OP_GATED_MLP_BWD, M, D, F, T, num_chunks, dtype);
  if (!workspace || workspace_bytes < need) return fail(TPM_EWORKSPACE, "%s: workspace of %zu bytes required", who, need);
  uint32_t* ctrl = (uint32_t*)workspace;
  void* dGU = (char*)workspace + kCtrlBytes;
  int32_t corder[TPM_MAX_CHUNKS];
  if (dy_chunk_order) std::memcpy(corder, dy_chunk_order, sizeof(int32_t) * num_chunks);
  else ring_order(T, num_chunks, rank, corder);
  const int bf = TPM_BF16;
  // [dG | dU] from dH = dY . W_down^T       W_down_t [Ft, D]: op(B) = W_down^T, stored [N=Ft, K=D]
  GemmDesc g_dh{M, Ft, D, dY, D, false, bf, nullptr, W_down_t, D, true, bf, nullptr,
                dGU, 2 * Ft, bf, TPM_EPI_DGATED, act, const_cast<void*>(GU_t), 2 * Ft, nullptr,
                num_chunks, corder, dy_ready, nullptr, epoch, ctrl};
  // dW_down = H^T . dY
  GemmDesc g_wd{Ft, D, M, H_t, Ft, true, bf, nullptr, dY, D, false, bf, nullptr,
                dW_down_t, D, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, epoch, ctrl};
  // [dW_gate | dW_up] = X^T . [dG | dU]
  GemmDesc g_wgu{D, 2 * Ft, M, X, D, true, bf, nullptr, dGU, 2 * Ft, false, bf, nullptr,
                 dW_gu_t, 2 * Ft, dw_dtype, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                 1, nullptr, nullptr, nullptr, epoch, ctrl};
  // dX = [dG | dU] . [W_gate | W_up]^T       W_gu_t [D, 2Ft]: op(B) = W_gu^T, stored [N=D, K=2Ft]
  GemmDesc g_dx{M, D, 2 * Ft, dGU, 2 * Ft, false, bf, nullptr, W_gu_t, 2 * Ft, true, bf, nullptr,
                dX_t, D, bf, TPM_EPI_FWD, TPM_ACT_NONE, nullptr, 0, nullptr,
                1, nullptr, nullptr, nullptr, epoch, ctrl};
  {
    const size_t dgu_bytes = round_up((size_t)M * (size_t)(2 * Ft) * 2, 256);
    for (GemmDesc* g : {&g_dh, &g_wd, &g_wgu, &g_dx}) {
      g->part = (float*)((char*)workspace + kCtrlBytes + dgu_bytes);
      g->part_bytes = workspace_bytes - kCtrlBytes - dgu_bytes;
    }
  }
  for (const GemmDesc* g : {&g_dh, &g_wd, &g_wgu, &g_dx}) {
    int rc = check_gemm(*g, who);
    if (rc != TPM_OK) return rc;
  }
  hipStream_t s = (hipStream_t)stream;
  if (dy_ready) {
    hipError_t e = launch_ctrl_init(ctrl, kCtrlWords, s);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  for (const GemmDesc* g : {&g_dh, &g_wd, &g_wgu, &g_dx}) {
    int rc = run_gemm(*g, s, who);
    if (rc != TPM_OK) return rc;
  }
  return TPM_OK;
}

int partial_reduce_seqshard(int T, int64_t M, int64_t D, int rank,
                            const void* partials, int64_t partial_stride, int64_t ld, int in_dtype,
                            void* out, int64_t ldo, int out_dtype, void* stream) {
  const char* who = "partial_reduce_seqshard";
  if (T < 1) return fail(TPM_EINVAL, "%s: T < 1", who);
  if (M < 0 || D < 0) return fail(TPM_EINVAL, "%s: negative size", who);
  if (M % T != 0) return fail(TPM_EINVAL, "%s: M %% T != 0", who);
  if (rank < -1 || rank >= T) return fail(TPM_EINVAL, "%s: bad rank", who);
  if ((in_dtype != TPM_BF16 && in_dtype != TPM_F32) || (out_dtype != TPM_BF16 && out_dtype != TPM_F32))
    return fail(TPM_EINVAL, "%s: dtypes BF16 or F32", who);
  const int64_t rows = M / T;
  if (rows == 0 || D == 0) return TPM_OK;
  if (!partials || !out) return fail(TPM_EINVAL, "%s: null pointer", who);
  if (ld < D || ldo < D) return fail(TPM_EINVAL, "%s: leading dimension < D", who);
  const int64_t held_rows = rank < 0 ? rows : M;
  if (T > 1 && partial_stride < (held_rows - 1) * ld + D)
    return fail(TPM_EINVAL, "%s: partials overlap (partial_stride too small)", who);
  const int64_t row0 = rank < 0 ? 0 : (int64_t)rank * rows;
  const int in_f32 = in_dtype == TPM_F32;
  const char* base = (const char*)partials + row0 * ld * (in_f32 ? 4 : 2);
  hipError_t e = launch_reduce(T, rows, D, base, partial_stride, ld, in_f32, out, ldo, out_dtype == TPM_F32,
                               (hipStream_t)stream);
  return e == hipSuccess ? TPM_OK : hip_fail(e, who);
}

}  // extern "C"

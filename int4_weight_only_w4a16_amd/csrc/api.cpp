// C-ABI front end of libw4a16.so: argument checks, launch planning and error
// mapping for the device entry points declared in include/w4a16.h.
#include <algorithm>
#include <cstdint>

#include "w4a16.h"
#include "w4a16_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by the GEMV entry points. Returns W4A16_OK, an error,
// or 1 for a valid empty call.
int check_shape(int M, int N, int K) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 0 || N < 0) return W4A16_EINVAL;
  if (M > W4A16_MAX_M) return W4A16_EUNSUPPORTED;
  if (M == 0 || N == 0) return 1;
  return W4A16_OK;
}

bool pointers_ok(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return false;
  return true;
}

// Smallest instantiated share size that holds `tiles` tiles (10 at most;
// longer shares run in several rounds).
int share_for(int tiles) {
  static const int kShares[] = {2, 3, 4, 5, 7, 8, 10};
  for (int s : kShares)
    if (tiles <= s) return s;
  return 10;
}

// Launch plan for one shape. Waves per workgroup and the share size depend
// on N and K only (never on M), so row m of an M-row call is bit-identical to
// the same row computed alone: every engine below performs the same fp32
// operations in the same order for a given (waves, K range). The fewest
// waves (a power of two, at most 16) whose shares hold at most 10 tiles: the
// whole K range is then in flight at once, in as few waves as possible (a
// sweep of all instantiated plans on the 7B and 27B shapes put this choice
// first or within 2% of the best; small matrices take shorter shares, below).
// MFMA with x from LDS when the per-wave x slices fit, else from global
// memory.
w4a16::LaunchPlan plan_for(int M, int N, int K, int splits) {
  const int groups = K / W4A16_GROUP;
  const int64_t row_tiles = (int64_t(N) + 15) / 16;
  const int range = (groups + splits - 1) / splits;
  // Split-K grids are large already: shorter shares (more waves per
  // workgroup) measured faster there (3584 x 18944 at 8 splits: 4 waves x 5
  // tiles 8.9 us, 2 waves x 10 tiles 9.6 us). A matrix too small to fill
  // the GPU with at most 8 groups (the 0.5B model's 896 columns) waits
  // mostly on each wave's serial unpack once its few tiles arrive: two tiles
  // per wave (896 x 896: 4 waves x 2 tiles 2.34 us, 1 wave x 7 tiles 2.53
  // us or more).
  const int target = splits > 1 ? 5 : (groups <= 8 && row_tiles < 256 ? 2 : 10);
  w4a16::LaunchPlan plan;
  plan.engine = w4a16::kEngineMfma;
  plan.splits = splits;
  plan.tiles_per_wg = 1;
  plan.epilogue = w4a16::kEpiStore;
  plan.waves = 1;
  while (plan.waves < 16 && (range + plan.waves - 1) / plan.waves > target) plan.waves *= 2;
  while (plan.waves > 1 && plan.waves > range) plan.waves /= 2;  // every wave gets at least one group
  const int per_wave = (range + plan.waves - 1) / plan.waves;
  plan.share = share_for(per_wave);
  if (!w4a16::plan_supported(M, K, plan)) {
    plan.engine = w4a16::kEngineMfmaGlobalX;
    plan.share = plan.waves == 16 ? 3 : 4;
  }
  return plan;
}

// Split count for w4a16_gemv_splitk (never depends on M, so a caller who
// follows it keeps rows batch invariant). From a sweep of split counts on
// MI355X, each with the plan plan_for gives it:
//  - a long K (at least 96 groups) unsplit runs one 16-wave workgroup per
//    row tile, one per CU at a time; with 256 to 1024 row tiles that takes
//    two or more passes over the CUs, and splitting pays, about one split
//    per 16 groups (5120 x 17408: 15.5 -> about 12 us at M = 1, 28 -> 16 us
//    at M = 8). With at most 256 row tiles one pass holds them and it did
//    not (3584 x 18944: 8.7 us unsplit, 9.4 us at 9 splits in a decode step);
//  - fewer than 128 row tiles with K of 24 groups or more: about one split
//    per 12 groups (128 x 18944: 7.3 -> 3.7 us);
//  - 1024 to 2047 row tiles with K of 40 groups or more: 2 splits. Each
//    workgroup then stages x of half the K range in LDS, and more of them
//    stay resident when x has several rows (17408 x 5120: M = 5 16.2 ->
//    13.5 us, M = 8 22.8 -> 15.3 us, at a cost of 10.6 -> 11.3 us at M = 1
//    and 11.3 -> 12.1 us at M = 2);
//  - elsewhere it lost (qkv 4608 x 3584: 4.65 us unsplit, 5.25 us at 2).
int choose_splits(int N, int K) {
  const int groups = K / W4A16_GROUP;
  const int64_t row_tiles = (int64_t(N) + 15) / 16;
  int splits = 1;
  if (groups >= 96 && row_tiles > 256 && row_tiles < 1024)
    splits = groups / 16;
  else if (row_tiles < 128 && groups >= 24)
    splits = groups / 12 < 2 ? 2 : groups / 12;
  else if (groups >= 40 && row_tiles >= 1024 && row_tiles < 2048)
    splits = 2;
  return splits > 16 ? 16 : splits;
}

// Split count for w4a16_gemm_splitk, measured on MI355X (7B-shaped
// matrices, M = 1 .. 2048). Each split adds a pass of 64-bit atomics over
// its output tile, whose cost grows with the tile's rows, against
// K/128 / splits groups of products. A long K (>= 96 groups) pays for it up
// to about one workgroup per compute unit (two for 16-row tiles) and 8
// splits (16 for 16-row tiles), or 3 splits for two per CU where one split
// per CU would leave the grid unsplit; a short K takes 4 while the grid is
// small and the tile holds at most 96 rows (128 on a grid of at most 32
// tiles).
int choose_gemm_splits(int M, int N, int K) {
  const int groups = K / W4A16_GROUP;
  const int bm = 16 * w4a16::gemm_m_blocks(M);
  const int64_t wgs = (int64_t(M) + bm - 1) / bm * ((int64_t(N) + 127) / 128);
  if (wgs >= 256) return 1;
  int64_t splits;
  if (groups >= 96) {
    splits = (bm == 16 ? 512 : 256) / wgs;
    const int64_t cap = bm == 16 ? 16 : 8;
    splits = splits > cap ? cap : splits;
    // 129 to 170 tiles: 3 splits give about two workgroups per CU, where 2
    // leave some CUs one (3584x18944 at M = 768: 141 us, against 164 us
    // unsplit and 164 us in 2).
    if (splits == 1 && 3 * wgs <= 512) splits = 3;
  } else {
    const int rows = M < 128 ? M : 128;
    splits = wgs <= 40 && (rows <= 96 || wgs <= 32) ? 4 : 1;
    splits = splits > 256 / wgs ? 256 / wgs : splits;
  }
  splits = splits > groups / 4 ? groups / 4 : splits;
  splits = splits > w4a16::kMaxSplits ? w4a16::kMaxSplits : splits;
  return splits < 1 ? 1 : int(splits);
}

// Split count for w4a16_gemm_splitk_partials, fitted to a sweep of split
// counts on MI355X (7B-shaped matrices, M = 16 .. 384). With W the output
// tiles of w4a16_gemm: none from 256 tiles on; else about 160 workgroups
// (ceil(160 / W) splits), raised toward 20 groups of K per split while the
// grid stays within 256 workgroups (the long-K down projection), at most 16
// splits and at least 4 groups each. More splits than that lost: each adds
// 4 * M * N bytes of partials, written once and read once more. (qkv
// 4608x3584 at M = 128: 19.2 us in 4, 20.1 in 7, 23.0 in 14; down
// 3584x18944 at M = 384: 66.6 us in 3, 75.6 in 4, 86.4 in 2.)
int choose_gemm_partials(int M, int N, int K) {
  const int groups = K / W4A16_GROUP;
  const int bm = 16 * w4a16::gemm_m_blocks(M);
  const int64_t wgs = (int64_t(M) + bm - 1) / bm * ((int64_t(N) + 127) / 128);
  if (wgs >= 256) return 1;
  int64_t splits = (160 + wgs - 1) / wgs;
  const int64_t long_k = std::min<int64_t>((groups + 19) / 20, 256 / wgs);
  if (long_k > splits) splits = long_k;
  if (splits > 16) splits = 16;
  if (splits > groups / 4) splits = groups / 4;
  return splits < 1 ? 1 : int(splits);
}

// Plan of the INT8-activation GEMV: as many waves as plan_for gives the
// same shape (so rows are batch invariant: the fp32 order depends on the
// waves only), each wave's groups in one round of a 4-, 7- or 10-tile share, or
// in rounds of a smaller share where the workgroup's LDS (codes of all M
// rows) would not hold the larger one.
w4a16::LaunchPlan plan_a8(int M, int N, int K) {
  w4a16::LaunchPlan plan = plan_for(1, N, K, 1);
  const int groups = K / W4A16_GROUP;
  const int per_wave = (groups + plan.waves - 1) / plan.waves;
  plan.engine = w4a16::kEngineMfma;
  plan.share = per_wave <= 4 ? 4 : (per_wave <= 7 ? 7 : 10);
  while (plan.share > 4 && !w4a16::a8_instantiated(M, plan.waves, plan.share)) plan.share = plan.share == 10 ? 7 : 4;
  return plan;
}

}  // namespace

namespace w4a16 {

int gemv_splitk_status(int M, int N, int K, int splits, const void* wq, const void* scales, const void* zeros,
                       const void* x, void* y, unsigned long long* acc, void* stream) {
  const LaunchPlan plan = plan_for(M, N, K, splits);
  if (launch_gemv(M, N, K, plan, wq, scales, zeros, x, y, acc, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

}  // namespace w4a16

extern "C" int w4a16_act_quant_i8(int M, int K, const void* x, void* xq, void* sx, void* xsum, void* stream) {
  const int rc = check_shape(M, 1, K);
  if (rc != W4A16_OK) return rc == 1 ? W4A16_OK : rc;
  if (!pointers_ok({x, xq, sx, xsum})) return W4A16_EINVAL;
  if (w4a16::launch_act_quant_i8(M, K, x, xq, sx, xsum, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_gemv_a8(int M, int N, int K, const void* Wq, const void* scales, const void* zeros,
                             const void* xq, const void* sx, const void* xsum, void* y, void* stream) {
  const int rc = check_shape(M, N, K);
  if (rc != W4A16_OK) return rc == 1 ? W4A16_OK : rc;
  if (!pointers_ok({Wq, scales, zeros, xq, sx, xsum, y})) return W4A16_EINVAL;
  const w4a16::LaunchPlan plan = plan_a8(M, N, K);
  if (!w4a16::a8_instantiated(M, plan.waves, plan.share)) return W4A16_EUNSUPPORTED;
  if (w4a16::launch_gemv_a8(M, N, K, plan, Wq, scales, zeros, xq, sx, xsum, y, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_gemv_a8_fused(int M, int N, int K, const void* Wq, const void* scales, const void* zeros,
                                   const void* x, void* y, void* stream) {
  const int rc = check_shape(M, N, K);
  if (rc != W4A16_OK) return rc == 1 ? W4A16_OK : rc;
  if (!pointers_ok({Wq, scales, zeros, x, y})) return W4A16_EINVAL;
  // The separate path's waves (so the same sums in the same order), in
  // shares short enough for the round's x to sit in registers.
  w4a16::LaunchPlan plan = plan_a8(M, N, K);
  while (plan.share > 4 && !w4a16::a8_fused_instantiated(M, plan.waves, plan.share))
    plan.share = plan.share == 10 ? 7 : 4;
  if (!w4a16::a8_fused_instantiated(M, plan.waves, plan.share)) return W4A16_EUNSUPPORTED;
  if (w4a16::launch_gemv_a8_fused(M, N, K, plan, Wq, scales, zeros, x, y, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_gemv(int M, int N, int K, const void* Wq, const void* scales, const void* zeros,
                          const void* x, void* y, void* stream) {
  const int rc = check_shape(M, N, K);
  if (rc != W4A16_OK) return rc == 1 ? W4A16_OK : rc;
  if (!pointers_ok({Wq, scales, zeros, x, y})) return W4A16_EINVAL;
  const w4a16::LaunchPlan plan = plan_for(M, N, K, 1);
  if (w4a16::launch_gemv(M, N, K, plan, Wq, scales, zeros, x, y, nullptr, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_gemv_swiglu(int M, int F, int K, const void* Wq, const void* scales, const void* zeros,
                                 const void* x, void* y, void* stream) {
  const int rc = check_shape(M, F, K);
  if (rc != W4A16_OK) return rc == 1 ? W4A16_OK : rc;
  if (!pointers_ok({Wq, scales, zeros, x, y})) return W4A16_EINVAL;
  // The plain GEMV's plan for the packed matrix (ceil(F/8) row tiles of 16
  // rows): the same waves and shares, so rows stay batch invariant, and any
  // K the GEMV takes.
  if ((int64_t(F) + 7) / 8 * 16 > INT32_MAX) return W4A16_EUNSUPPORTED;
  w4a16::LaunchPlan plan = plan_for(M, 16 * ((F + 7) / 8), K, 1);
  plan.epilogue = w4a16::kEpiSwiglu;
  if (!w4a16::plan_supported(M, K, plan)) return W4A16_EUNSUPPORTED;
  if (w4a16::launch_gemv(M, F, K, plan, Wq, scales, zeros, x, y, nullptr, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" size_t w4a16_splitk_workspace_bytes(int M, int N, int splits) {
  if (M < 0 || N < 0 || splits < 0) return 0;
  return w4a16::splitk_workspace_bytes(M, N);
}

extern "C" int w4a16_splitk_choose(int M, int N, int K) {
  if (check_shape(M, N, K) < 0) return 0;
  return choose_splits(N, K);
}

extern "C" int w4a16_gemv_splitk(int M, int N, int K, int splits, const void* Wq, const void* scales,
                                 const void* zeros, const void* x, void* y, void* workspace,
                                 size_t ws_bytes, void* stream) {
  const int rc = check_shape(M, N, K);
  if (rc < 0) return rc;
  if (splits < 1 || splits > K / W4A16_GROUP || splits > w4a16::kMaxSplits) return W4A16_EINVAL;
  if (rc == 1) return W4A16_OK;
  if (splits == 1) return w4a16_gemv(M, N, K, Wq, scales, zeros, x, y, stream);
  if (!pointers_ok({Wq, scales, zeros, x, y, workspace})) return W4A16_EINVAL;
  if (ws_bytes < w4a16::splitk_workspace_bytes(M, N)) return W4A16_EINVAL;
  return w4a16::gemv_splitk_status(M, N, K, splits, Wq, scales, zeros, x, y,
                                   static_cast<unsigned long long*>(workspace), stream);
}

extern "C" int w4a16_gemm(int M, int N, int K, const void* Wq, const void* scales, const void* zeros,
                          const void* x, void* y, void* stream) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 0 || N < 0) return W4A16_EINVAL;
  if (M == 0 || N == 0) return W4A16_OK;
  if (K >= w4a16::kGemmMaxK) return W4A16_EUNSUPPORTED;
  if (!pointers_ok({Wq, scales, zeros, x, y})) return W4A16_EINVAL;
  if (w4a16::launch_gemm(M, N, K, 1, Wq, scales, zeros, x, y, nullptr, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_gemm_splitk_choose(int M, int N, int K) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 1 || N < 1 || K >= w4a16::kGemmMaxK) return 0;
  return choose_gemm_splits(M, N, K);
}

extern "C" int w4a16_gemm_splitk(int M, int N, int K, int splits, const void* Wq, const void* scales,
                                 const void* zeros, const void* x, void* y, void* workspace, size_t ws_bytes,
                                 void* stream) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 0 || N < 0) return W4A16_EINVAL;
  if (splits < 1 || splits > K / W4A16_GROUP || splits > w4a16::kMaxSplits) return W4A16_EINVAL;
  if (M == 0 || N == 0) return W4A16_OK;
  if (K >= w4a16::kGemmMaxK) return W4A16_EUNSUPPORTED;
  if (splits == 1) return w4a16_gemm(M, N, K, Wq, scales, zeros, x, y, stream);
  if (!pointers_ok({Wq, scales, zeros, x, y, workspace})) return W4A16_EINVAL;
  if (ws_bytes < w4a16::splitk_workspace_bytes(M, N)) return W4A16_EINVAL;
  auto* ws = static_cast<unsigned long long*>(workspace);
  if (w4a16::launch_gemm(M, N, K, splits, Wq, scales, zeros, x, y, ws, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" size_t w4a16_gemm_partials_bytes(int M, int N, int splits) {
  if (M < 0 || N < 0 || splits < 1) return 0;
  return w4a16::gemm_partials_bytes(M, N, splits);
}

extern "C" int w4a16_gemm_partials_choose(int M, int N, int K) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 1 || N < 1 || K >= w4a16::kGemmMaxK) return 0;
  return choose_gemm_partials(M, N, K);
}

extern "C" int w4a16_gemm_splitk_partials(int M, int N, int K, int splits, const void* Wq, const void* scales,
                                          const void* zeros, const void* x, void* y, void* partials,
                                          size_t partials_bytes, void* stream) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 0 || N < 0) return W4A16_EINVAL;
  if (splits < 1 || splits > K / W4A16_GROUP || splits > w4a16::kMaxSplits) return W4A16_EINVAL;
  if (M == 0 || N == 0) return W4A16_OK;
  if (K >= w4a16::kGemmMaxK) return W4A16_EUNSUPPORTED;
  if (splits == 1) return w4a16_gemm(M, N, K, Wq, scales, zeros, x, y, stream);
  if (!pointers_ok({Wq, scales, zeros, x, y, partials})) return W4A16_EINVAL;
  if (partials_bytes < w4a16::gemm_partials_bytes(M, N, splits)) return W4A16_EINVAL;
  if (w4a16::launch_gemm(M, N, K, splits, Wq, scales, zeros, x, y, nullptr, stream, static_cast<float*>(partials)) != 0)
    return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_dequant_f16(int N, int K, const void* Wq, const void* scales, const void* zeros,
                                 void* W_out, void* stream) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || N < 0) return W4A16_EINVAL;
  if (N == 0) return W4A16_OK;
  if (!pointers_ok({Wq, scales, zeros, W_out})) return W4A16_EINVAL;
  if (w4a16::launch_dequant_f16(N, K, Wq, scales, zeros, W_out, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_read_probe(const void* buf, size_t bytes, int grid, void* sink, void* stream) {
  if (bytes % 16 != 0 || grid < 1 || grid > 65535) return W4A16_EINVAL;
  if (bytes == 0) return W4A16_OK;
  if (!pointers_ok({buf, sink})) return W4A16_EINVAL;
  if (w4a16::launch_read_probe(buf, bytes, grid, sink, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" int w4a16_dequant_f32(int N, int K, const void* Wq, const void* scales, const void* zeros,
                                 float* W_out, void* stream) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || N < 0) return W4A16_EINVAL;
  if (N == 0) return W4A16_OK;
  if (!pointers_ok({Wq, scales, zeros, W_out})) return W4A16_EINVAL;
  if (w4a16::launch_dequant(N, K, Wq, scales, zeros, W_out, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

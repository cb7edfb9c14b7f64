// C-ABI front end of libw4a16.so: argument checks, launch planning and error
// mapping for the device entry points declared in include/w4a16.h.
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

// Waves per workgroup grow with the number of groups so that long rows are
// streamed by more waves at once.
w4a16::LaunchPlan plan_for(int M, int K, int splits) {
  const int groups = K / W4A16_GROUP;
  const int per_split = (groups + splits - 1) / splits;
  w4a16::LaunchPlan plan;
  plan.waves = per_split >= 64 ? 16 : per_split >= 16 ? 8 : 4;
  plan.splits = splits;
  const int cap = w4a16::max_slice_groups(M);
  plan.slice_groups = per_split < cap ? per_split : cap;
  return plan;
}

}  // namespace

extern "C" int w4a16_gemv(int M, int N, int K, const void* Wq, const void* scales, const void* zeros,
                          const void* x, void* y, void* stream) {
  const int rc = check_shape(M, N, K);
  if (rc != W4A16_OK) return rc == 1 ? W4A16_OK : rc;
  if (!pointers_ok({Wq, scales, zeros, x, y})) return W4A16_EINVAL;
  const w4a16::LaunchPlan plan = plan_for(M, K, 1);
  if (w4a16::launch_gemv(M, N, K, plan, Wq, scales, zeros, x, y, nullptr, stream) != 0) return W4A16_EHIP;
  return W4A16_OK;
}

extern "C" size_t w4a16_splitk_workspace_bytes(int M, int N, int splits) {
  if (M < 0 || N < 0 || splits < 0) return 0;
  return size_t(4) * size_t(splits) * size_t(M) * size_t(N);
}

extern "C" int w4a16_gemv_splitk(int M, int N, int K, int splits, const void* Wq, const void* scales,
                                 const void* zeros, const void* x, void* y, void* workspace,
                                 size_t ws_bytes, void* stream) {
  const int rc = check_shape(M, N, K);
  if (rc < 0) return rc;
  if (splits < 1 || splits > K / W4A16_GROUP) return W4A16_EINVAL;
  if (rc == 1) return W4A16_OK;
  if (!pointers_ok({Wq, scales, zeros, x, y, workspace})) return W4A16_EINVAL;
  if (ws_bytes < w4a16_splitk_workspace_bytes(M, N, splits)) return W4A16_EINVAL;
  const w4a16::LaunchPlan plan = plan_for(M, K, splits);
  float* partials = static_cast<float*>(workspace);
  if (w4a16::launch_gemv(M, N, K, plan, Wq, scales, zeros, x, y, partials, stream) != 0) return W4A16_EHIP;
  if (w4a16::launch_splitk_reduce(M, N, splits, partials, y, stream) != 0) return W4A16_EHIP;
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

// HIP kernels of libw4a16.so for gfx950 (CDNA4, wave64) other than the GEMV
// template (gemv_kernel.h, instantiated per M in gemv_m*.hip): the dequant
// test hook, and the launchers.
#include "w4a16_device.h"

namespace w4a16 {
namespace dev {

// out[n][k] = float(q - z) * float(s): one thread per packed word.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros,
                                                      float* __restrict__ out, int N, int K) {
  const int G = K / kGroup;
  const int64_t tile = blockIdx.x;
  const int64_t t = tile / G;
  const int g = int(tile - t * G);
  const int lane = threadIdx.x >> 2, kb = threadIdx.x & 3;
  const int64_t row = t * kTileRows + (lane & 15);
  if (row >= N) return;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(wq + tile * kTileBytes + lane * 16 + kb * 4);
  const int64_t e = tile * kTileRows + (lane & 15);  // this row's scale / zero slot
  const float s = half_bits_to_float(scales[e]);
  half2_t p[4];
  unpack8(w, kMagic1024, zero_pairs((zeros[e >> 1] >> ((lane & 1) * 4)) & 15u), p);
  float* dst = out + row * K + int64_t(g) * kGroup + 32 * kb + 8 * (lane >> 4);
  const f32x4 a = {float(p[0].x) * s, float(p[0].y) * s, float(p[1].x) * s, float(p[1].y) * s};
  const f32x4 b = {float(p[2].x) * s, float(p[2].y) * s, float(p[3].x) * s, float(p[3].y) * s};
  reinterpret_cast<f32x4*>(dst)[0] = a;
  reinterpret_cast<f32x4*>(dst)[1] = b;
}

}  // namespace dev

size_t lds_bytes(int M, int K, const LaunchPlan& plan) {
  (void)K;
  return gemv_lds_bytes(M, plan.waves, plan.share, plan.engine, plan.epilogue);
}

bool plan_supported(int M, int K, const LaunchPlan& plan) {
  if (M < 1 || M > 8 || plan.splits < 1 || plan.splits > K / kGroup || plan.splits > kMaxSplits) return false;
  if (plan.tiles_per_wg < 1 || plan.tiles_per_wg > 3) return false;
  if (plan.engine < kEngineDot2 || plan.engine > kEngineMfmaGlobalX) return false;
  const int w = plan.waves, sh = plan.share;
  if (!(w == 1 || w == 2 || w == 4 || w == 8 || w == 16)) return false;
  if (!(sh == 2 || sh == 3 || sh == 4 || sh == 5 || sh == 7 || sh == 8 || sh == 10)) return false;
  if (plan.epilogue == kEpiSwiglu) {
    // One round per wave, every wave with at least one group (the kernel
    // relies on it for its one staging barrier).
    const int groups = K / kGroup, half = plan.waves / 2;
    if (plan.splits != 1 || groups < half || (groups + half - 1) / half > plan.share) return false;
  }
  if (!instantiated(M, w, sh, plan.engine, plan.tiles_per_wg, plan.epilogue)) return false;
  return lds_bytes(M, K, plan) <= kMaxLdsBytes;
}

int launch_gemv(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                const void* zeros, const void* x, void* y, unsigned long long* acc, void* stream_ptr) {
  switch (M) {
    case 1: return launch_gemv_m1(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 2: return launch_gemv_m2(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 3: return launch_gemv_m3(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 4: return launch_gemv_m4(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 5: return launch_gemv_m5(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 6: return launch_gemv_m6(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 7: return launch_gemv_m7(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    case 8: return launch_gemv_m8(N, K, plan, wq, scales, zeros, x, y, acc, stream_ptr);
    default: return int(hipErrorInvalidValue);
  }
}

int launch_dequant(int N, int K, const void* wq, const void* scales, const void* zeros, float* out,
                   void* stream_ptr) {
  const int64_t tiles = (int64_t(N) + kTileRows - 1) / kTileRows * (K / kGroup);
  hipLaunchKernelGGL(dev::dequant_kernel, dim3(unsigned(tiles)), dim3(256), 0, static_cast<hipStream_t>(stream_ptr),
                     static_cast<const uint8_t*>(wq), static_cast<const uint16_t*>(scales),
                     static_cast<const uint8_t*>(zeros), out, N, K);
  return int(hipGetLastError());
}

}  // namespace w4a16

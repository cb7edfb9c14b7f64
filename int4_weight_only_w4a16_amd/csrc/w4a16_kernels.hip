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
  const int64_t t = int64_t(unsigned(tile) / unsigned(G));  // tile = blockIdx.x < 2^32
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

// Standalone dequantization to fp16 (the dequantize entry point of "Custom
// AWQ Dequantization Kernel", for this library's layout): one wave per 1 KiB
// tile, four tiles per workgroup (consecutive groups of one row tile, so a
// workgroup's stores cover 512 contiguous columns of 16 rows). A lane loads
// its 16 bytes (32 weights of one row) and its scale and zero words, forms
// the exact (q - z) * s in fp32 and rounds once to fp16: the result is the
// exact product rounded to nearest even. 2.5 bytes of HBM traffic per weight
// (0.5 read + 2 written), plus the scales and zeros.
__global__ __launch_bounds__(256) void dequant_f16_kernel(int N, int K, int64_t tiles,
                                                          const uint8_t* __restrict__ wq,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros,
                                                          _Float16* __restrict__ out) {
  const int G = K / kGroup;
  const int lane = threadIdx.x & 63;
  const int64_t tile = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (tile >= tiles) return;
  // 32-bit division whenever the tile index fits (always short of 2^32 tiles).
  const int64_t t = tile < (int64_t(1) << 32) ? int64_t(unsigned(tile) / unsigned(G)) : tile / G;
  const int g = int(tile - t * G);
  const int rlane = lane & 15;
  const int64_t row = t * kTileRows + rlane;
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wq + tile * kTileBytes) + lane);
  const uint32_t sw = reinterpret_cast<const uint32_t*>(scales)[tile * (kTileRows / 2) + (rlane >> 1)];
  const uint32_t zw = reinterpret_cast<const uint32_t*>(zeros)[tile * (kTileRows / 8) + (rlane >> 3)];
  if (row >= N) return;  // padding rows: nothing to write
  const float s = half_bits_to_float((sw >> ((rlane & 1) * 16)) & 0xFFFFu);
  const ZeroPairs zp = zero_pairs((zw >> ((rlane & 7) * 4)) & 15u);
  _Float16* dst = out + row * K + int64_t(g) * kGroup + 8 * (lane >> 4);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    half2_t p[4];
    unpack8(w[kb], kMagic1024, zp, p);
    half8_t h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (_Float16)(float(p[i].x) * s);
      h[2 * i + 1] = (_Float16)(float(p[i].y) * s);
    }
    *reinterpret_cast<half8_t*>(dst + 32 * kb) = h;
  }
}

// Plain read of n 16-byte words with the GEMV's non-temporal loads, four in
// flight per thread; nothing is stored unless the XOR of a thread's words
// equals one constant (then one word of sink), so the loads cannot be
// dropped and the traffic is reads alone.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, int64_t n,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride), d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace dev

int launch_read_probe(const void* buf, size_t bytes, int grid, void* sink, void* stream_ptr) {
  return int(dev::launch_kernel(&dev::read_probe_kernel, dim3(unsigned(grid)), dim3(256), 0,
                                static_cast<hipStream_t>(stream_ptr), static_cast<const dev::u32x4*>(buf),
                                int64_t(bytes / 16), static_cast<uint32_t*>(sink)));
}

size_t lds_bytes(int M, int K, const LaunchPlan& plan) {
  (void)K;
  return gemv_lds_bytes(M, plan.waves, plan.share, plan.engine, plan.epilogue);
}

bool plan_supported(int M, int K, const LaunchPlan& plan) {
  if (M < 1 || M > 8 || plan.splits < 1 || plan.splits > K / kGroup || plan.splits > kMaxSplits) return false;
  if (plan.tiles_per_wg != 1) return false;
  if (plan.engine != kEngineMfma && plan.engine != kEngineMfmaGlobalX) return false;
  const int w = plan.waves, sh = plan.share;
  if (!(w == 1 || w == 2 || w == 4 || w == 8 || w == 16)) return false;
  if (!(sh == 2 || sh == 3 || sh == 4 || sh == 5 || sh == 7 || sh == 8 || sh == 10)) return false;
  if (plan.epilogue == kEpiSwiglu && plan.splits != 1) return false;
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

int launch_dequant_f16(int N, int K, const void* wq, const void* scales, const void* zeros, void* out,
                       void* stream_ptr) {
  const int64_t tiles = (int64_t(N) + kTileRows - 1) / kTileRows * (K / kGroup);
  return int(dev::launch_kernel(&dev::dequant_f16_kernel, dim3(unsigned((tiles + 3) / 4)), dim3(256), 0,
                                static_cast<hipStream_t>(stream_ptr), N, K, tiles, static_cast<const uint8_t*>(wq),
                                static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                                static_cast<_Float16*>(out)));
}

int launch_dequant(int N, int K, const void* wq, const void* scales, const void* zeros, float* out,
                   void* stream_ptr) {
  const int64_t tiles = (int64_t(N) + kTileRows - 1) / kTileRows * (K / kGroup);
  return int(dev::launch_kernel(&dev::dequant_kernel, dim3(unsigned(tiles)), dim3(256), 0,
                                static_cast<hipStream_t>(stream_ptr), static_cast<const uint8_t*>(wq),
                                static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros), out,
                                N, K));
}

}  // namespace w4a16

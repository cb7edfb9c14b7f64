// HIP kernels of libw4a16.so for gfx950 (CDNA4, wave64).
//
// GEMV y = W x with W in layout ID 1 (16-row x 128-column tiles of 1 KiB).
// Workgroup = one 16-row tile x one K range; its waves split the range's
// groups into contiguous shares. Per group a lane issues one 16-byte
// non-temporal load (32 weights of its row), turns the nibbles into exact
// fp16 (q - z) pairs in registers and feeds v_dot2_f32_f16 against x pairs
// read from LDS; the group's fp32 dot is scaled once by s. Lanes l, l^16,
// l^32, l^48 share a row and are combined with two xor shuffles, waves
// through LDS, always in the same order, so results are bit-identical run to
// run (the determinism rule of the qengine page, "Learnings").
#include <hip/hip_runtime.h>

#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLoadsInFlight = 4;          // tiles a wave requests before using any
constexpr int kLdsXBytes = 48 * 1024;      // x staging budget per workgroup
constexpr uint32_t kMagic1024 = 0x64006400u;  // fp16 pair (1024, 1024)

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// fp16 pairs (1024 + z, 1024 + z) and (64 + z, 64 + z) for a zero point z.
// 1024 + z has bits 0x6400 | z (spacing 1 in [1024, 2048)); 64 + z has bits
// 0x5400 | (z << 4) (spacing 1/16 in [64, 128)).
struct ZeroPairs {
  half2_t z1024, z64;
};

__device__ __forceinline__ ZeroPairs zero_pairs(uint32_t z) {
  return {as_h2((0x6400u | z) * 0x00010001u), as_h2((0x5400u | (z << 4)) * 0x00010001u)};
}

// (w & mask) | magic in one VALU op. gfx9 VOP3 has no literal operand, so the
// compiler splits this into v_and_b32 + v_or_b32 with literals; with the mask
// in an SGPR and the magic in a VGPR a single v_and_or_b32 does it.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

// Eight weights of one ValueShuffle word -> (q - z) as four fp16 pairs in
// column order (w0,w1), (w2,w3), (w4,w5), (w6,w7). OR-ing a nibble into the
// mantissa of 1024.0 gives 1024 + q exactly; a nibble four bits higher gives
// 1024 + 16q, and (1024 + 16q)/16 - (64 + z) = q - z. Every step is exact in
// fp16 (all values are integers or sixteenths below 2048).
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t magic, const ZeroPairs& zp, half2_t p[4]) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  p[0] = as_h2(and_or(w, 0x000F000Fu, magic)) - zp.z1024;
  p[1] = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, magic)), sixteenth, -zp.z64);
  p[2] = as_h2(and_or(w8, 0x000F000Fu, magic)) - zp.z1024;
  p[3] = __builtin_elementwise_fma(as_h2(and_or(w8, 0x00F000F0u, magic)), sixteenth, -zp.z64);
}

__device__ __forceinline__ uint32_t zero_nibble(const uint8_t* zrow, int g) {
  return (uint32_t(zrow[g >> 1]) >> ((g & 1) * 4)) & 15u;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// One workgroup: row tile blockIdx.x, K range blockIdx.y of gridDim.y.
// MR = activation rows (1..8), WAVES = waves per workgroup.
// Writes fp16 y[MR][N] when `part` is null, else fp32 part[split][MR][N].
template <int MR, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const _Float16* __restrict__ x, _Float16* __restrict__ y,
    float* __restrict__ part, int N, int K, int slice_groups) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);                                   // [WAVES][MR][16]
  _Float16* xs = reinterpret_cast<_Float16*>(smem + WAVES * MR * 16 * sizeof(float));  // [MR][slice]

  const int G = K / kGroup;
  const int GP = (G + 7) & ~7;
  const int64_t t = blockIdx.x;
  const int split = blockIdx.y, splits = gridDim.y;
  const int g_beg = int(int64_t(split) * G / splits);
  const int g_end = int(int64_t(split + 1) * G / splits);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int piece = lane >> 4;  // which 8-column piece of each 32 columns
  const int64_t row = t * kTileRows + (lane & 15);  // < padded row count: always valid memory
  const uint8_t* wlane = wq + t * G * int64_t(kTileBytes) + lane * 16;
  const uint16_t* srow = scales + row * GP;
  const uint8_t* zrow = zeros + row * (GP / 2);
  const int slice_len = slice_groups * kGroup;
  const uint32_t magic = kMagic1024;

  float acc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = 0.f;

  for (int s0 = g_beg; s0 < g_end; s0 += slice_groups) {
    const int ng = min(slice_groups, g_end - s0);
    // Stage x[:, 128*s0 : 128*(s0+ng)) into LDS, 16 bytes per thread and step.
    __syncthreads();
    const int chunks = ng * (kGroup / 8);
    for (int c = tid; c < MR * chunks; c += WAVES * 64) {
      const int m = c / chunks, cc = c - m * chunks;
      const u32x4 v = *reinterpret_cast<const u32x4*>(x + int64_t(m) * K + int64_t(s0) * kGroup + cc * 8);
      *reinterpret_cast<u32x4*>(xs + m * slice_len + cc * 8) = v;
    }
    __syncthreads();

    const int g0 = s0 + (wave * ng) / WAVES;
    const int g1 = s0 + ((wave + 1) * ng) / WAVES;
    for (int g = g0; g < g1; g += kLoadsInFlight) {
      u32x4 wv[kLoadsInFlight];
      uint32_t sv[kLoadsInFlight], zv[kLoadsInFlight];
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u) {
        if (g + u < g1) {
          wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wlane + int64_t(g + u) * kTileBytes));
          sv[u] = srow[g + u];
          zv[u] = zero_nibble(zrow, g + u);
        }
      }
#pragma unroll
      for (int u = 0; u < kLoadsInFlight; ++u) {
        if (g + u < g1) {
          const ZeroPairs zp = zero_pairs(zv[u]);
          const _Float16* xg = xs + (g + u - s0) * kGroup + 8 * piece;
          float dot[MR];
#pragma unroll
          for (int m = 0; m < MR; ++m) dot[m] = 0.f;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            half2_t p[4];
            unpack8(wv[u][kb], magic, zp, p);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const u32x4 xv = *reinterpret_cast<const u32x4*>(xg + m * slice_len + 32 * kb);
              dot[m] = __builtin_amdgcn_fdot2(p[0], as_h2(xv.x), dot[m], false);
              dot[m] = __builtin_amdgcn_fdot2(p[1], as_h2(xv.y), dot[m], false);
              dot[m] = __builtin_amdgcn_fdot2(p[2], as_h2(xv.z), dot[m], false);
              dot[m] = __builtin_amdgcn_fdot2(p[3], as_h2(xv.w), dot[m], false);
            }
          }
          const float s = half_bits_to_float(sv[u]);
#pragma unroll
          for (int m = 0; m < MR; ++m) acc[m] = __builtin_fmaf(dot[m], s, acc[m]);
        }
      }
    }
  }

  // Lanes l, l^16, l^32, l^48 hold the same row: fold them.
#pragma unroll
  for (int m = 0; m < MR; ++m) {
    float v = acc[m];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    acc[m] = v;
  }
  if (lane < 16) {
#pragma unroll
    for (int m = 0; m < MR; ++m) red[(wave * MR + m) * 16 + lane] = acc[m];
  }
  __syncthreads();
  if (tid < MR * 16) {
    const int m = tid >> 4, i = tid & 15;
    float sum = red[m * 16 + i];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += red[(w * MR + m) * 16 + i];
    const int64_t n = t * kTileRows + i;
    if (n < N) {
      if (part)
        part[(int64_t(split) * MR + m) * N + n] = sum;
      else
        y[int64_t(m) * N + n] = (_Float16)sum;
    }
  }
}

// y[i] = fp16(sum over splits of part[split][i]), splits in ascending order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part,
                                                            _Float16* __restrict__ y, int64_t count,
                                                            int splits) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float sum = part[i];
  for (int s = 1; s < splits; ++s) sum += part[int64_t(s) * count + i];
  y[i] = (_Float16)sum;
}

// out[n][k] = float(q - z) * float(s): one thread per packed word.
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ wq,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ zeros,
                                                      float* __restrict__ out, int N, int K) {
  const int G = K / kGroup;
  const int GP = (G + 7) & ~7;
  const int64_t tile = blockIdx.x;
  const int64_t t = tile / G;
  const int g = int(tile - t * G);
  const int lane = threadIdx.x >> 2, kb = threadIdx.x & 3;
  const int64_t row = t * kTileRows + (lane & 15);
  if (row >= N) return;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(wq + tile * kTileBytes + lane * 16 + kb * 4);
  const float s = half_bits_to_float(scales[row * GP + g]);
  half2_t p[4];
  unpack8(w, kMagic1024, zero_pairs(zero_nibble(zeros + row * (GP / 2), g)), p);
  float* dst = out + row * K + int64_t(g) * kGroup + 32 * kb + 8 * (lane >> 4);
  const f32x4 a = {float(p[0].x) * s, float(p[0].y) * s, float(p[1].x) * s, float(p[1].y) * s};
  const f32x4 b = {float(p[2].x) * s, float(p[2].y) * s, float(p[3].x) * s, float(p[3].y) * s};
  reinterpret_cast<f32x4*>(dst)[0] = a;
  reinterpret_cast<f32x4*>(dst)[1] = b;
}

template <int MR, int WAVES>
hipError_t launch_typed(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                        const void* zeros, const void* x, void* y, float* partials, hipStream_t stream) {
  const int64_t row_tiles = (int64_t(N) + kTileRows - 1) / kTileRows;
  const size_t lds = size_t(WAVES) * MR * 16 * sizeof(float) + size_t(MR) * plan.slice_groups * kGroup * 2;
  hipLaunchKernelGGL((gemv_kernel<MR, WAVES>), dim3(unsigned(row_tiles), unsigned(plan.splits)),
                     dim3(WAVES * 64), lds, stream, static_cast<const uint8_t*>(wq),
                     static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                     static_cast<const _Float16*>(x), static_cast<_Float16*>(y), partials, N, K,
                     plan.slice_groups);
  return hipGetLastError();
}

template <int MR>
hipError_t launch_waves(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                        const void* zeros, const void* x, void* y, float* partials, hipStream_t stream) {
  switch (plan.waves) {
    case 4: return launch_typed<MR, 4>(N, K, plan, wq, scales, zeros, x, y, partials, stream);
    case 8: return launch_typed<MR, 8>(N, K, plan, wq, scales, zeros, x, y, partials, stream);
    case 16: return launch_typed<MR, 16>(N, K, plan, wq, scales, zeros, x, y, partials, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int max_slice_groups(int M) { return kLdsXBytes / (M * kGroup * 2); }

int launch_gemv(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                const void* zeros, const void* x, void* y, float* partials, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  hipError_t e;
  switch (M) {
    case 1: e = launch_waves<1>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 2: e = launch_waves<2>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 3: e = launch_waves<3>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 4: e = launch_waves<4>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 5: e = launch_waves<5>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 6: e = launch_waves<6>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 7: e = launch_waves<7>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 8: e = launch_waves<8>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    default: e = hipErrorInvalidValue;
  }
  return int(e);
}

int launch_splitk_reduce(int M, int N, int splits, const float* partials, void* y, void* stream_ptr) {
  const int64_t count = int64_t(M) * N;
  const unsigned blocks = unsigned((count + 255) / 256);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream_ptr),
                     partials, static_cast<_Float16*>(y), count, splits);
  return int(hipGetLastError());
}

int launch_dequant(int N, int K, const void* wq, const void* scales, const void* zeros, float* out,
                   void* stream_ptr) {
  const int64_t tiles = (int64_t(N) + kTileRows - 1) / kTileRows * (K / kGroup);
  hipLaunchKernelGGL(dequant_kernel, dim3(unsigned(tiles)), dim3(256), 0, static_cast<hipStream_t>(stream_ptr),
                     static_cast<const uint8_t*>(wq), static_cast<const uint16_t*>(scales),
                     static_cast<const uint8_t*>(zeros), out, N, K);
  return int(hipGetLastError());
}

}  // namespace w4a16

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

// Workgroup barrier that orders LDS only. __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding loads
// (vmcnt(0)) -- including weight tiles requested ahead -- before the barrier.
// No thread here communicates through global memory, so an LDS-scope fence
// (lgkmcnt only) is all the barriers need.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t zero_nibble(const uint8_t* zrow, int g) {
  return (uint32_t(zrow[g >> 1]) >> ((g & 1) * 4)) & 15u;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Inner-product engines. kEngineDot2: v_dot2_f32_f16 on the VALU, lane-private
// partial sums over 8-column pieces. kEngineMfma*: v_mfma_f32_16x16x32_f16
// with the activations as the A operand (row m of A = x[m]; rows >= M repeat
// the last x row and are ignored) and the unpacked weights as the B operand
// (column j of B = weight row j of the tile), so D[m][j] = sum_k x[m][k]
// w[j][k]; the multiply-adds leave the VALU, which then only unpacks. The
// A operand comes from LDS (kEngineMfma) or, when x of the K range does not
// fit in LDS, straight from global memory with the weights of the batch
// (kEngineMfmaGlobalX).
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Workgroup = WAVES waves over row tiles t = blockIdx.x, blockIdx.x +
// gridDim.x, ... (a launch has at most as many workgroups as fit on the GPU at
// once, so there is no second, half-empty round of workgroups) and one K
// range blockIdx.y of gridDim.y. The waves take contiguous shares of the
// range's groups, in rounds of at most SHARE tiles (one round for every shape
// the launch table picks; then a wave stages its x slice in its private LDS
// region once and reuses it for all its row tiles). The waves' partial sums meet in LDS (double-buffered across row tiles, one
// barrier per row tile) and are added in wave order.
// Writes fp16 y[MR][N] when `part` is null, else fp32 part[split][MR][N].
template <int MR, int WAVES, int SHARE, int ENGINE>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(
    const uint8_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const _Float16* __restrict__ x, _Float16* __restrict__ y,
    float* __restrict__ part, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr bool kGlobalX = ENGINE == kEngineMfmaGlobalX;
  constexpr int kAcc = ENGINE == kEngineDot2 ? MR : 4;  // accumulators per lane
  constexpr int kXRow = SHARE * kGroup;                  // halves per staged x row of a wave
  constexpr int kRed = WAVES * MR * 16;                  // floats per reduction buffer
  float* red = reinterpret_cast<float*>(smem);           // [2][WAVES][MR][16]

  const int G = K / kGroup;
  const int GP = (G + 7) & ~7;
  const int64_t row_tiles = (int64_t(N) + kTileRows - 1) / kTileRows;
  const int split = blockIdx.y, splits = gridDim.y;
  const int g_beg = int(int64_t(split) * G / splits);
  const int g_end = int(int64_t(split + 1) * G / splits);
  const int ng = g_end - g_beg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps share bounds scalar
  const int piece = lane >> 4;  // which 8-column piece of each 32 columns
  const int rlane = lane & 15;  // weight row within the tile
  const uint32_t magic = kMagic1024;
  const int share_beg = g_beg + (wave * ng) / WAVES;
  const int share_end = g_beg + ((wave + 1) * ng) / WAVES;
  const int mm = rlane < MR ? rlane : MR - 1;  // activation row feeding A-operand row rlane
  _Float16* xw = reinterpret_cast<_Float16*>(smem + 2 * kRed * sizeof(float)) +
                 (kGlobalX ? 0 : wave * MR * kXRow);  // this wave's x slice [MR][SHARE*128]
  int parity = 0;

  // Copy x[:, 128*g0 : 128*(g0+n)) into this wave's LDS slice (synchronous).
  auto stage_x = [&](int g0, int n) {
    if constexpr (!kGlobalX) {
      const int xchunks = n * (kGroup / 8), xtotal = MR * xchunks;
      for (int c = lane; c < xtotal; c += 64) {
        const int m = c / xchunks, cc = c - m * xchunks;
        *reinterpret_cast<u32x4*>(xw + m * kXRow + cc * 8) =
            *reinterpret_cast<const u32x4*>(x + int64_t(m) * K + int64_t(g0) * kGroup + cc * 8);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
  };

  // A round = SHARE tiles of one row tile. load_round() requests them all
  // (indices past the share's end are clamped to its last tile: always in
  // bounds, discarded later) with their scales and zero bytes as
  // straight-line code; compute_round() then uses them in request order, so
  // each wait is for exactly the tile about to be used (loads retire in
  // order). Every tile is computed -- a branch would let the compiler sink a
  // tile's load next to its use -- and the clamped duplicates are discarded
  // by a select.
  struct Round {
    u32x4 w[SHARE];
    uint32_t sv[SHARE], zb[SHARE];
    half8_t xa[kGlobalX ? SHARE : 1][4];
  };
  auto load_round = [&](Round& r, const u32x4* wlane, const uint16_t* srow, const uint8_t* zrow, int g0, int n) {
#pragma unroll
    for (int u = 0; u < SHARE; ++u) {
      const int gg = g0 + min(u, n - 1);
      r.w[u] = __builtin_nontemporal_load(wlane + int64_t(gg) * (kTileBytes / 16));
      r.sv[u] = srow[gg];
      r.zb[u] = zrow[gg >> 1];
      if constexpr (kGlobalX) {
        const _Float16* xl = x + int64_t(mm) * K + int64_t(gg) * kGroup + 8 * piece;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) r.xa[u][kb] = *reinterpret_cast<const half8_t*>(xl + 32 * kb);
      }
    }
  };
  auto compute_round = [&](const Round& r, int g0, int n, float (&acc)[kAcc]) {
#pragma unroll
    for (int u = 0; u < SHARE; ++u) {
      const bool valid = u < n;
      __builtin_amdgcn_sched_barrier(0);  // keep tiles in request order
      const int g = g0 + min(u, n - 1);
      const ZeroPairs zp = zero_pairs((r.zb[u] >> ((g & 1) * 4)) & 15u);
      const float s = half_bits_to_float(r.sv[u]);
      const _Float16* xg = xw + u * kGroup + 8 * piece;
      if constexpr (ENGINE == kEngineDot2) {
        float dot[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) dot[m] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          half2_t p[4];
          unpack8(r.w[u][kb], magic, zp, p);
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const u32x4 xq = *reinterpret_cast<const u32x4*>(xg + m * kXRow + 32 * kb);
            dot[m] = __builtin_amdgcn_fdot2(p[0], as_h2(xq.x), dot[m], false);
            dot[m] = __builtin_amdgcn_fdot2(p[1], as_h2(xq.y), dot[m], false);
            dot[m] = __builtin_amdgcn_fdot2(p[2], as_h2(xq.z), dot[m], false);
            dot[m] = __builtin_amdgcn_fdot2(p[3], as_h2(xq.w), dot[m], false);
          }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = valid ? __builtin_fmaf(dot[m], s, acc[m]) : acc[m];
      } else {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          half2_t p[4];
          unpack8(r.w[u][kb], magic, zp, p);
          const half8_t bw = {p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
          half8_t ax;
          if constexpr (kGlobalX)
            ax = r.xa[u][kb];
          else
            ax = *reinterpret_cast<const half8_t*>(xg + mm * kXRow + 32 * kb);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, bw, d, 0, 0, 0);
        }
#pragma unroll
        for (int r2 = 0; r2 < 4; ++r2) acc[r2] = valid ? __builtin_fmaf(d[r2], s, acc[r2]) : acc[r2];
      }
    }
  };

  const int share_n = share_end - share_beg;
  const bool one_round = share_n <= SHARE;

  // Cross-wave sum of one row tile and its store. One barrier per row tile:
  // the next tile writes the other buffer, and the tile after that is behind
  // this tile's next barrier.
  auto finish_tile = [&](int64_t t, float (&acc)[kAcc]) {
    float* rb = red + parity * kRed;
    if constexpr (ENGINE == kEngineDot2) {
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
        for (int m = 0; m < MR; ++m) rb[(wave * MR + m) * 16 + lane] = acc[m];
      }
    } else {
      // Lane l holds D[4*(l/16) + r][l%16]: activation row 4*piece + r, weight row rlane.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * piece + r;
        if (m < MR) rb[(wave * MR + m) * 16 + rlane] = acc[r];
      }
    }
    lds_barrier();
    for (int idx = tid; idx < MR * 16; idx += WAVES * 64) {  // one wave has fewer lanes than 8 x 16 outputs
      const int m = idx >> 4, i = idx & 15;
      float sum = rb[m * 16 + i];
#pragma unroll
      for (int w2 = 1; w2 < WAVES; ++w2) sum += rb[(w2 * MR + m) * 16 + i];
      const int64_t nn = t * kTileRows + i;
      if (nn < N) {
        if (part)
          part[(int64_t(split) * MR + m) * N + nn] = sum;
        else
          y[int64_t(m) * N + nn] = (_Float16)sum;
      }
    }
    parity ^= 1;
  };

  struct TilePtrs {
    const u32x4* wlane;
    const uint16_t* srow;
    const uint8_t* zrow;
  };
  auto tile_ptrs = [&](int64_t t) {
    const int64_t row = t * kTileRows + rlane;  // < padded row count: always valid memory
    return TilePtrs{reinterpret_cast<const u32x4*>(wq + t * G * int64_t(kTileBytes)) + lane,
                    scales + row * GP, zeros + row * (GP / 2)};
  };

  int64_t t = blockIdx.x;
  if (one_round && share_n > 0 && !kGlobalX && t < row_tiles) {
    // First row tile of a one-round share: x requests go out just ahead of
    // the weight requests, so the wait before the LDS store is for x alone;
    // the staged slice then serves all of this workgroup's row tiles.
    const TilePtrs p = tile_ptrs(t);
    constexpr int kXSteps = (MR * SHARE * 16 + 63) / 64;
    const int xchunks = share_n * (kGroup / 8), xtotal = MR * xchunks;
    u32x4 xv[kXSteps];
#pragma unroll
    for (int j = 0; j < kXSteps; ++j) {  // clamped: unconditional, in bounds
      const int c = min(lane + 64 * j, xtotal - 1);
      const int m = c / xchunks, cc = c - m * xchunks;
      xv[j] = *reinterpret_cast<const u32x4*>(x + int64_t(m) * K + int64_t(share_beg) * kGroup + cc * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    Round r;
    load_round(r, p.wlane, p.srow, p.zrow, share_beg, share_n);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kXSteps; ++j) {  // clamped steps rewrite the last chunk with its own data
      const int c = min(lane + 64 * j, xtotal - 1);
      const int m = c / xchunks, cc = c - m * xchunks;
      *reinterpret_cast<u32x4*>(xw + m * kXRow + cc * 8) = xv[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    float acc[kAcc];
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = 0.f;
    compute_round(r, share_beg, share_n, acc);
    finish_tile(t, acc);
    t += gridDim.x;
  } else if (one_round && share_n > 0 && !kGlobalX) {
    stage_x(share_beg, share_n);  // (no row tile for this workgroup: unreachable with the host's grids)
  }

  for (; t < row_tiles; t += gridDim.x) {
    const TilePtrs p = tile_ptrs(t);
    float acc[kAcc];
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = 0.f;
    if (one_round) {
      if (share_n > 0) {
        Round r;
        load_round(r, p.wlane, p.srow, p.zrow, share_beg, share_n);
        compute_round(r, share_beg, share_n, acc);
      }
    } else {
      for (int g0 = share_beg; g0 < share_end; g0 += SHARE) {  // long K: x restaged per round
        const int n = min(SHARE, share_end - g0);
        stage_x(g0, n);
        Round r;
        load_round(r, p.wlane, p.srow, p.zrow, g0, n);
        compute_round(r, g0, n, acc);
      }
    }
    finish_tile(t, acc);
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

template <int MR, int WAVES, int SHARE, int ENGINE>
hipError_t launch_typed(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                        const void* zeros, const void* x, void* y, float* partials, hipStream_t stream) {
  const int64_t row_tiles = (int64_t(N) + kTileRows - 1) / kTileRows;
  const int64_t per_wg = plan.tiles_per_wg < 1 ? 1 : plan.tiles_per_wg;
  const int64_t grid = (row_tiles + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((gemv_kernel<MR, WAVES, SHARE, ENGINE>), dim3(unsigned(grid), unsigned(plan.splits)),
                     dim3(WAVES * 64), lds_bytes(MR, K, plan), stream, static_cast<const uint8_t*>(wq),
                     static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                     static_cast<const _Float16*>(x), static_cast<_Float16*>(y), partials, N, K);
  return hipGetLastError();
}

// Instantiated (waves, share) pairs per engine and M: those that fit in
// registers without spilling.
constexpr bool instantiated(int mr, int waves, int share, int engine) {
  if (engine == kEngineMfmaGlobalX) return waves == 16 ? share <= 3 : share <= 4;
  if (engine == kEngineDot2) return mr == 1 ? share <= 10 : (mr == 2 && share <= 5 && waves <= 8);
  return (waves == 16 && mr >= 4) ? share <= 5 : share <= 10;
}

template <int MR, int ENGINE>
hipError_t launch_shape(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                        const void* zeros, const void* x, void* y, float* partials, hipStream_t stream) {
#define W4A16_CASE(W, S)                                                                           \
  if constexpr (instantiated(MR, W, S, ENGINE)) {                                                     \
    if (plan.waves == W && plan.share == S)                                                       \
      return launch_typed<MR, W, S, ENGINE>(N, K, plan, wq, scales, zeros, x, y, partials, stream); \
  }
#define W4A16_SHARES(W) \
  W4A16_CASE(W, 2) W4A16_CASE(W, 3) W4A16_CASE(W, 4) W4A16_CASE(W, 5) W4A16_CASE(W, 7) W4A16_CASE(W, 8) W4A16_CASE(W, 10)
  W4A16_SHARES(1) W4A16_SHARES(2) W4A16_SHARES(4) W4A16_SHARES(8) W4A16_SHARES(16)
#undef W4A16_SHARES
#undef W4A16_CASE
  return hipErrorInvalidValue;
}

template <int MR>
hipError_t launch_engine(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                         const void* zeros, const void* x, void* y, float* partials, hipStream_t stream) {
  switch (plan.engine) {
    case kEngineMfma:
      return launch_shape<MR, kEngineMfma>(N, K, plan, wq, scales, zeros, x, y, partials, stream);
    case kEngineMfmaGlobalX:
      return launch_shape<MR, kEngineMfmaGlobalX>(N, K, plan, wq, scales, zeros, x, y, partials, stream);
    case kEngineDot2:
      if constexpr (MR <= 2)
        return launch_shape<MR, kEngineDot2>(N, K, plan, wq, scales, zeros, x, y, partials, stream);
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

size_t lds_bytes(int M, int K, const LaunchPlan& plan) {
  (void)K;
  const size_t red = 2 * size_t(plan.waves) * M * 16 * sizeof(float);
  if (plan.engine == kEngineMfmaGlobalX) return red;
  return red + size_t(plan.waves) * M * plan.share * kGroup * 2;
}

bool plan_supported(int M, int K, const LaunchPlan& plan) {
  if (M < 1 || M > 8 || plan.splits < 1 || plan.splits > K / kGroup) return false;
  if (plan.engine == kEngineDot2 && M > 2) return false;
  if (plan.engine < kEngineDot2 || plan.engine > kEngineMfmaGlobalX) return false;
  const int w = plan.waves, sh = plan.share;
  if (!(w == 1 || w == 2 || w == 4 || w == 8 || w == 16)) return false;
  if (!(sh == 2 || sh == 3 || sh == 4 || sh == 5 || sh == 7 || sh == 8 || sh == 10)) return false;
  if (!instantiated(M, w, sh, plan.engine)) return false;
  return lds_bytes(M, K, plan) <= kMaxLdsBytes;
}

int launch_gemv(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                const void* zeros, const void* x, void* y, float* partials, void* stream_ptr) {
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  hipError_t e;
  switch (M) {
    case 1: e = launch_engine<1>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 2: e = launch_engine<2>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 3: e = launch_engine<3>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 4: e = launch_engine<4>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 5: e = launch_engine<5>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 6: e = launch_engine<6>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 7: e = launch_engine<7>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
    case 8: e = launch_engine<8>(N, K, plan, wq, scales, zeros, x, y, partials, stream); break;
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

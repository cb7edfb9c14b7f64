// INT8-activation variant for gfx950: the alternative path of "Building an
// LLM Inference Runtime ... on NVIDIA H100", Bug #3 (Path A). The fp16
// activations are first turned into signed 8-bit codes with one fp32 scale
// per group of 128 (a launch of its own, as on that page); the GEMV then
// multiplies weight codes by activation codes as integers and brings each
// group's integer sum back with the weight scale and the activation scale.
//
// On CDNA4 the integer products run on the matrix cores
// (v_mfma_i32_16x16x64_i8, the counterpart of the page's dp4a). The weight
// codes need no arithmetic at all: q is 0..15, already a valid signed byte,
// so masking a packed word's low and high nibbles yields four int8 B-operand
// bytes each. The zero point is applied once per group and row, exactly, in
// integers: sum_k (q - z) xq = sum_k q xq - z * sum_k xq, with sum_k xq
// (one number per activation row and group) produced by the quantizer.
#include "w4a16_device.h"

namespace w4a16 {
namespace dev {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One wave per (activation row m, group g): lane l holds x[m][128g + 2l] and
// the next. sx = absmax / 127 (fp32, correctly rounded); code =
// clamp(rne(x / sx), -127, 127); a group of zeros gets sx = 0 and codes 0.
// xsum = the sum of the group's codes. Groups are numbered i = m * G + g.
__global__ __launch_bounds__(256) void act_quant_i8_kernel(int64_t groups_total, int K, const _Float16* __restrict__ x,
                                                          int8_t* __restrict__ xq, float* __restrict__ sx,
                                                          int32_t* __restrict__ xsum) {
  const int lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (i >= groups_total) return;  // whole waves
  const int G = K / kGroup;
  const int64_t m = int64_t(unsigned(i) / unsigned(G));  // i < M * G <= 8 * 2^24
  const int64_t g = i - m * G;
  const int64_t base = m * K + g * kGroup + 2 * lane;
  const half2_t v = *reinterpret_cast<const half2_t*>(x + base);
  const float a0 = float(v.x), a1 = float(v.y);
  float amax = fmaxf(fabsf(a0), fabsf(a1));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax / 127.0f;
  int c0 = 0, c1 = 0;
  if (scale > 0.0f) {
    c0 = int(fminf(fmaxf(rintf(a0 / scale), -127.0f), 127.0f));
    c1 = int(fminf(fmaxf(rintf(a1 / scale), -127.0f), 127.0f));
  }
  *reinterpret_cast<uint16_t*>(xq + base) = uint16_t((uint32_t(c0) & 0xFFu) | ((uint32_t(c1) & 0xFFu) << 8));
  int sum = c0 + c1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane == 0) {
    sx[i] = scale;
    xsum[i] = sum;
  }
}

// Codes of 8 activations with a group scale computed as in
// act_quant_i8_kernel (the same fp32 operations, so the same bits): packed
// little-endian into two words, four codes each, and their sum.
__device__ __forceinline__ void quantize8(const float (&a)[8], float scale, uint32_t& d0, uint32_t& d1, int& sum) {
  d0 = d1 = 0u;
  sum = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = scale > 0.0f ? int(fminf(fmaxf(rintf(a[k] / scale), -127.0f), 127.0f)) : 0;
    sum += c;
    if (k < 4)
      d0 |= (uint32_t(c) & 0xFFu) << (8 * k);
    else
      d1 |= (uint32_t(c) & 0xFFu) << (8 * (k - 4));
  }
}

// Activation bytes x0..x7 of 8 consecutive columns -> the two words whose
// bytes line up with the masked nibbles of one packed weight word: the
// layout puts weight j of a word at nibble slot {0,4,1,5,2,6,3,7}[j], so
// (w & 0x0F0F0F0F) holds weights (0, 4, 1, 5) in bytes 0..3 and
// ((w >> 4) & 0x0F0F0F0F) weights (2, 6, 3, 7).
__device__ __forceinline__ u32x2 interleave_codes(uint32_t d0, uint32_t d1) {
  const uint32_t lo = (d0 & 0xFFu) | ((d1 & 0xFFu) << 8) | ((d0 & 0xFF00u) << 8) | ((d1 & 0xFF00u) << 16);
  const uint32_t hi = ((d0 >> 16) & 0xFFu) | ((d1 >> 8) & 0xFF00u) | ((d0 & 0xFF000000u) >> 8) | (d1 & 0xFF000000u);
  return {lo, hi};
}

// GEMV with int8 activation codes: one 16-row tile per workgroup; the WAVES
// waves take contiguous shares of the groups, in rounds of at most SHARE
// tiles. Per round a wave stages its activation codes in its private LDS
// slice, in MFMA operand order, with the groups' sx and xsum; requests all
// of the round's weight tiles (straight-line, clamped, as the fp16 GEMV
// does) and then runs, per tile, two integer MFMAs (64 columns each) with
// the codes as A (row m = lane % 16, rows >= M repeat the last) and the
// weight nibbles as B (column = tile row). Lane l then holds the integer
// sums D[4(l/16) + r][l % 16], corrects them by the zero point, and adds
// float(D - z xsum) * (s * sx) to its fp32 accumulators. The waves' sums
// meet in LDS and are added in wave order, so results are bit-identical run
// to run and do not depend on M.
//
// LDS: [WAVES][4][rows][16] floats for the reduction, then per wave
// [M][SHARE][128] code bytes and [SHARE][16] sx and xsum values (activation
// rows 0..15 of each group, zero past M).
//
// FQ (fused quantization): x is the fp16 activations, and each round
// quantizes its own slice while the weights are in flight, 16 lanes per
// group of 128, with the arithmetic of act_quant_i8_kernel: the codes, sx
// and xsum are those the separate launch would have produced, bit for bit,
// and so is y. sx and xsum are then unused.
template <int MR, int WAVES, int SHARE, bool FQ>
__global__ __launch_bounds__(WAVES * 64) void gemv_a8_kernel(
    int N, int K, const uint8_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const void* __restrict__ xin, const float* __restrict__ sx,
    const int32_t* __restrict__ xsum, _Float16* __restrict__ y) {
  const int8_t* xq = static_cast<const int8_t*>(xin);
  const _Float16* xf = static_cast<const _Float16*>(xin);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int kRows = MR < 4 ? MR : 4;                      // D rows of a lane that are activation rows
  constexpr int kRedWave = 4 * kRows * 16;
  constexpr int kSlice = MR * SHARE * kGroup + 2 * SHARE * 16 * 4;  // bytes per wave
  float* red = reinterpret_cast<float*>(smem);
  const int G = K / kGroup;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int piece = lane >> 4, rlane = lane & 15;
  const int mm = rlane < MR ? rlane : MR - 1;
  unsigned char* slice = smem + WAVES * kRedWave * sizeof(float) + wave * kSlice;
  float* ssx = reinterpret_cast<float*>(slice + MR * SHARE * kGroup);  // [SHARE][16]
  int32_t* ssum = reinterpret_cast<int32_t*>(ssx + SHARE * 16);      // [SHARE][16]
  const int share_beg = (wave * G) / WAVES, share_end = ((wave + 1) * G) / WAVES;

  const int64_t t = blockIdx.x;
  const int64_t q0 = t * G;  // tile (t, 0)
  const u32x4* wlane = reinterpret_cast<const u32x4*>(wq + q0 * kTileBytes) + lane;
  const uint32_t* sword = reinterpret_cast<const uint32_t*>(scales) + q0 * (kTileRows / 2) + (rlane >> 1);
  const uint32_t* zword = reinterpret_cast<const uint32_t*>(zeros) + q0 * (kTileRows / 8) + (rlane >> 3);

  float acc[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) acc[r] = 0.f;

  for (int g0 = share_beg; g0 < share_end; g0 += SHARE) {
    const int n = min(SHARE, share_end - g0);
    u32x4 w[SHARE];
    uint32_t sw[SHARE], zw[SHARE];
    auto request_weights = [&]() {
#pragma unroll
      for (int u = 0; u < SHARE; ++u) {
        const int gg = g0 + min(u, n - 1);
        w[u] = __builtin_nontemporal_load(wlane + int64_t(gg) * (kTileBytes / 16));
        sw[u] = sword[gg * (kTileRows / 2)];
        zw[u] = zword[gg * (kTileRows / 8)];
      }
    };
    if constexpr (!FQ) {
      // Activation codes first (their wait then covers them alone): 16-byte
      // chunks c = (m, group u, 16 columns h), clamped to the last real chunk.
      // Chunk c is row c / (8 SHARE), a division by a constant (a division by
      // the round's own chunk count costs some 20 vector instructions per
      // chunk); chunks past a short round's groups take a copy of the row's
      // last chunk.
      constexpr int kRowChunks = SHARE * 8;
      constexpr int kXSteps = (MR * kRowChunks + 63) / 64;
      const int xlast = n * 8 - 1;
      auto chunk = [&](int ln, int j, int& m, int& cc) {
        const int c = min(ln + 64 * j, MR * kRowChunks - 1);
        m = MR == 1 ? 0 : c / kRowChunks;
        cc = min(c - m * kRowChunks, xlast);
      };
      u32x4 xv[kXSteps];
#pragma unroll
      for (int j = 0; j < kXSteps; ++j) {
        int m, cc;
        chunk(lane, j, m, cc);
        xv[j] = *reinterpret_cast<const u32x4*>(xq + int64_t(m) * K + int64_t(g0) * kGroup + cc * 16);
      }
      constexpr int kMSteps = (SHARE * 16 + 63) / 64;
      float mv[kMSteps];
      int32_t sv[kMSteps];
#pragma unroll
      for (int j = 0; j < kMSteps; ++j) {
        const int c = min(lane + 64 * j, n * 16 - 1);
        const int u = c >> 4, m = c & 15;
        const int64_t e = int64_t(m < MR ? m : 0) * G + g0 + u;
        mv[j] = m < MR ? sx[e] : 0.f;
        sv[j] = m < MR ? xsum[e] : 0;
      }
      __builtin_amdgcn_sched_barrier(0);
      request_weights();
      __builtin_amdgcn_sched_barrier(0);
      // Stage: chunk (m, u, h) covers columns 16h .. 16h+15 of group u, i.e.
      // 8-column blocks b = 2h, 2h+1 with b = 4 kb + piece; block b goes to
      // byte (kb / 2) * 64 + piece * 16 + (kb % 2) * 8 of the group's 128.
      // The chunk indices again, from an opaque copy of the lane: kept from
      // the loads instead, they stay live across the weight requests and
      // spill at 16 waves.
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
#pragma unroll
      for (int j = 0; j < kXSteps; ++j) {
        int m, cc;
        chunk(lane_o, j, m, cc);
        const int u = cc >> 3, h = cc & 7;
        unsigned char* dst = slice + (m * SHARE + u) * kGroup;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int b = 2 * h + half, kb = b >> 2, pc = b & 3;
          const u32x2 v = interleave_codes(xv[j][2 * half], xv[j][2 * half + 1]);
          *reinterpret_cast<u32x2*>(dst + (kb >> 1) * 64 + pc * 16 + (kb & 1) * 8) = v;
        }
      }
#pragma unroll
      for (int j = 0; j < kMSteps; ++j) {
        const int c = min(lane + 64 * j, n * 16 - 1);
        ssx[c] = mv[j];
        ssum[c] = sv[j];
      }
    } else {
      // fp16 x of the round first: pass j, lane l takes 8 halves (l % 16)
      // of group 4 j + l / 16 of the [MR][SHARE] slice, row gi / SHARE,
      // group gi % SHARE (clamped to the round's last group and to the last
      // row: duplicates recompute the same values).
      constexpr int kPasses = (MR * SHARE + 3) / 4;
      auto group_of = [&](int ln, int j, int& m, int& u) {
        const int gi = min(4 * j + (ln >> 4), MR * SHARE - 1);
        m = MR == 1 ? 0 : gi / SHARE;
        u = min(gi - m * SHARE, n - 1);
      };
      u32x4 xh[kPasses];
#pragma unroll
      for (int j = 0; j < kPasses; ++j) {
        int m, u;
        group_of(lane, j, m, u);
        xh[j] = *reinterpret_cast<const u32x4*>(xf + int64_t(m) * K + int64_t(g0 + u) * kGroup + (lane & 15) * 8);
      }
      __builtin_amdgcn_sched_barrier(0);
      request_weights();
      __builtin_amdgcn_sched_barrier(0);
      // Rows past M: scale and code sum 0.
#pragma unroll
      for (int jj = 0; jj < (SHARE * 16 + 63) / 64; ++jj) {
        const int c = lane + 64 * jj;
        if (c < SHARE * 16 && (c & 15) >= MR) {
          ssx[c] = 0.f;
          ssum[c] = 0;
        }
      }
      int lane_o = lane;
      asm volatile("" : "+v"(lane_o));
      const int h8 = lane & 15;  // 8-column block of the group
#pragma unroll
      for (int j = 0; j < kPasses; ++j) {
        int m, u;
        group_of(lane_o, j, m, u);
        float a[8];
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const half2_t h2 = as_h2(xh[j][k]);
          a[2 * k] = float(h2.x);
          a[2 * k + 1] = float(h2.y);
          amax = fmaxf(amax, fmaxf(fabsf(a[2 * k]), fabsf(a[2 * k + 1])));
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const float scale = amax / 127.0f;
        uint32_t d0, d1;
        int sum;
        quantize8(a, scale, d0, d1, sum);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
        const int kb = h8 >> 2, pc = h8 & 3;
        *reinterpret_cast<u32x2*>(slice + (m * SHARE + u) * kGroup + (kb >> 1) * 64 + pc * 16 + (kb & 1) * 8) =
            interleave_codes(d0, d1);
        if (h8 == 0) {
          ssx[u * 16 + m] = scale;
          ssum[u * 16 + m] = sum;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");

    int xoff = mm * SHARE * kGroup + piece * 16;
    asm volatile("" : "+v"(xoff));
#pragma unroll
    for (int u = 0; u < SHARE; ++u) {
      __builtin_amdgcn_sched_barrier(0);
      u32x4 wt = w[u];
      uint32_t zt = zw[u], st = sw[u];
      asm volatile("" : "+v"(wt), "+v"(zt), "+v"(st));
      const unsigned char* xg = slice + xoff + u * kGroup;
      const i32x4 a0 = *reinterpret_cast<const i32x4*>(xg);
      const i32x4 a1 = *reinterpret_cast<const i32x4*>(xg + 64);
      const i32x4 b0 = {int32_t(wt[0] & 0x0F0F0F0Fu), int32_t((wt[0] >> 4) & 0x0F0F0F0Fu),
                        int32_t(wt[1] & 0x0F0F0F0Fu), int32_t((wt[1] >> 4) & 0x0F0F0F0Fu)};
      const i32x4 b1 = {int32_t(wt[2] & 0x0F0F0F0Fu), int32_t((wt[2] >> 4) & 0x0F0F0F0Fu),
                        int32_t(wt[3] & 0x0F0F0F0Fu), int32_t((wt[3] >> 4) & 0x0F0F0F0Fu)};
      i32x4 d = {0, 0, 0, 0};
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, d, 0, 0, 0);
      const int z = int((zt >> ((rlane & 7) * 4)) & 15u);
      const float s = half_bits_to_float((st >> ((rlane & 1) * 16)) & 0xFFFFu);
      const f32x4 gsx = *reinterpret_cast<const f32x4*>(ssx + u * 16 + 4 * piece);
      const i32x4 gsum = *reinterpret_cast<const i32x4*>(ssum + u * 16 + 4 * piece);
      const bool valid = u < n;
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const float term = float(d[r] - __mul24(z, gsum[r]));  // |xsum| <= 128 * 127 < 2^23
        acc[r] = valid ? __builtin_fmaf(term, s * gsx[r], acc[r]) : acc[r];
      }
    }
    // The next round restages the slice: every lane's reads are done first.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }

  // Cross-wave sum in wave order; lane l holds activation rows 4 piece + r.
#pragma unroll
  for (int r = 0; r < kRows; ++r) red[wave * kRedWave + (piece * kRows + r) * 16 + rlane] = acc[r];
  lds_barrier();
  constexpr int kOut = (MR * 16 + WAVES * 64 - 1) / (WAVES * 64);
#pragma unroll
  for (int j = 0; j < kOut; ++j) {
    const int idx = tid + j * WAVES * 64;
    const int m = idx >> 4, i = idx & 15;
    const int64_t nn = t * kTileRows + i;
    if (idx < MR * 16 && nn < N) {
      const int slot = ((m >> 2) * kRows + (m & 3)) * 16 + i;
      float sum = red[slot];
#pragma unroll
      for (int w2 = 1; w2 < WAVES; ++w2) sum += red[w2 * kRedWave + slot];
      y[int64_t(m) * N + nn] = (_Float16)sum;
    }
  }
}

template <int MR, int WAVES, int SHARE, bool FQ>
hipError_t launch_a8_typed(int N, int K, const void* wq, const void* scales, const void* zeros, const void* xq,
                           const void* sx, const void* xsum, void* y, hipStream_t stream) {
  constexpr size_t lds = gemv_a8_lds_bytes(MR, WAVES, SHARE);
  static_assert(lds <= kMaxLdsBytes, "instantiation beyond the LDS of a workgroup");
  auto* kernel = &gemv_a8_kernel<MR, WAVES, SHARE, FQ>;
  if constexpr (lds > kDefaultLdsLimit) {
    static std::atomic<uint64_t> raised{0};  // devices on which this instantiation's limit is raised
    const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kernel), lds, raised);
    if (e != hipSuccess) return e;
  }
  const int64_t row_tiles = (int64_t(N) + kTileRows - 1) / kTileRows;
  return launch_kernel(kernel, dim3(unsigned(row_tiles)), dim3(WAVES * 64), lds, stream, N, K,
                       static_cast<const uint8_t*>(wq), static_cast<const uint16_t*>(scales),
                       static_cast<const uint8_t*>(zeros), xq,
                       static_cast<const float*>(sx), static_cast<const int32_t*>(xsum), static_cast<_Float16*>(y));
}

template <int MR, bool FQ>
hipError_t launch_a8_m(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales, const void* zeros,
                       const void* xq, const void* sx, const void* xsum, void* y, hipStream_t stream) {
#define W4A16_A8_CASE(W, S)                                                                      \
  if constexpr (FQ ? a8_fused_instantiated(MR, W, S) : a8_instantiated(MR, W, S)) {              \
    if (plan.waves == W && plan.share == S)                                                      \
      return launch_a8_typed<MR, W, S, FQ>(N, K, wq, scales, zeros, xq, sx, xsum, y, stream);    \
  }
#define W4A16_A8_SHARES(W) W4A16_A8_CASE(W, 4) W4A16_A8_CASE(W, 7) W4A16_A8_CASE(W, 10)
  W4A16_A8_SHARES(1) W4A16_A8_SHARES(2) W4A16_A8_SHARES(4) W4A16_A8_SHARES(8) W4A16_A8_SHARES(16)
#undef W4A16_A8_SHARES
#undef W4A16_A8_CASE
  return hipErrorInvalidValue;
}

}  // namespace dev

int launch_act_quant_i8(int M, int K, const void* x, void* xq, void* sx, void* xsum, void* stream) {
  const int64_t groups_total = int64_t(M) * (K / kGroup);
  return int(dev::launch_kernel(&dev::act_quant_i8_kernel, dim3(unsigned((groups_total + 3) / 4)), dim3(256), 0,
                                static_cast<hipStream_t>(stream), groups_total, K, static_cast<const _Float16*>(x),
                                static_cast<int8_t*>(xq), static_cast<float*>(sx), static_cast<int32_t*>(xsum)));
}

int launch_gemv_a8(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                   const void* zeros, const void* xq, const void* sx, const void* xsum, void* y, void* stream_ptr) {
  const hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  switch (M) {
    case 1: return int(dev::launch_a8_m<1, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 2: return int(dev::launch_a8_m<2, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 3: return int(dev::launch_a8_m<3, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 4: return int(dev::launch_a8_m<4, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 5: return int(dev::launch_a8_m<5, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 6: return int(dev::launch_a8_m<6, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 7: return int(dev::launch_a8_m<7, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    case 8: return int(dev::launch_a8_m<8, false>(N, K, plan, wq, scales, zeros, xq, sx, xsum, y, stream));
    default: return int(hipErrorInvalidValue);
  }
}

int launch_gemv_a8_fused(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                         const void* zeros, const void* x, void* y, void* stream_ptr) {
  const hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  switch (M) {
    case 1: return int(dev::launch_a8_m<1, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 2: return int(dev::launch_a8_m<2, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 3: return int(dev::launch_a8_m<3, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 4: return int(dev::launch_a8_m<4, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 5: return int(dev::launch_a8_m<5, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 6: return int(dev::launch_a8_m<6, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 7: return int(dev::launch_a8_m<7, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    case 8: return int(dev::launch_a8_m<8, true>(N, K, plan, wq, scales, zeros, x, nullptr, nullptr, y, stream));
    default: return int(hipErrorInvalidValue);
  }
}

}  // namespace w4a16

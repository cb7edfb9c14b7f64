// W4A16 GEMM for many activation rows (prefill-sized M), on the matrix
// cores: y[M][N] = x[M][K] W^T with W in layout ID 2, dequantized in
// registers. A 256-thread workgroup computes a 128 (m) x 128 (n) tile of y
// as four 64 x 64 wave tiles (2 x 2), each 4 x 4 blocks of
// v_mfma_f32_16x16x32_f16 with fp32 accumulators, over K one 128-column
// group at a time. (Wave tiles of 128 x 64, which dequantize each weight
// tile once instead of twice, need 424 registers, one wave per SIMD, and
// measured 20-50% slower.)
//  - x[m0 .. m0+127][group] is staged in LDS (double-buffered, rows padded
//    by 16 bytes against bank conflicts) and read as the A operand;
//  - each wave streams its four weight tiles (16 rows x 128 columns, 1 KiB
//    each; a lane's 16 bytes are exactly its B operand for the four 32-column
//    blocks) and dequantizes them to fp16 (q - z) * s, rounded once to
//    nearest even -- the values w4a16_dequant_f16 writes;
//  - the next group's x and weight requests go out before the current group
//    is multiplied.
#include "w4a16_device.h"

namespace w4a16 {
namespace dev {

constexpr int kGemmBM = 128;                // activation rows per workgroup
constexpr int kGemmBN = 128;                // weight rows per workgroup (8 row tiles)
constexpr int kGemmMB = 4;                  // 16-row m blocks per wave (64 rows)
constexpr int kXStride = kGroup + 8;        // halves per LDS row of x (272 bytes)
constexpr size_t kGemmLds = size_t(2) * kGemmBM * kXStride * 2;

__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ wq,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros,
                                                   const _Float16* __restrict__ x, _Float16* __restrict__ y,
                                                   int M, int N, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* xs = reinterpret_cast<_Float16*>(smem);  // [2][kGemmBM][kXStride]
  const int G = K / kGroup;
  const int64_t NT = (int64_t(N) + kTileRows - 1) / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // this wave's 64 x 64 quarter
  const int rlane = lane & 15, piece = lane >> 4;
  // m fastest: the workgroups resident at once share weight tiles in L2
  // (making n fastest instead, to share x, measured no faster).
  const int64_t m0 = int64_t(blockIdx.x) * kGemmBM;
  const int64_t tw = int64_t(blockIdx.y) * (kGemmBN / kTileRows) + wn * 4;  // wave's first row tile

  // The wave's four row tiles (clamped past the end: valid memory, never stored).
  const u32x4* wl[4];
  const uint32_t* swp[4];
  const uint32_t* zwp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = tw + j < NT ? tw + j : NT - 1;
    const int64_t q0 = t * G;
    wl[j] = reinterpret_cast<const u32x4*>(wq + q0 * kTileBytes) + lane;
    swp[j] = reinterpret_cast<const uint32_t*>(scales) + q0 * (kTileRows / 2) + (rlane >> 1);
    zwp[j] = reinterpret_cast<const uint32_t*>(zeros) + q0 * (kTileRows / 8) + (rlane >> 3);
  }
  // x chunks of this thread: 8 x 16 bytes of the 128 x 128 group tile (rows
  // past M read row M - 1: valid memory, never stored).
  auto load_x = [&](int g, u32x4 (&xv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = c & 15;
      const int64_t mr = m0 + row < M ? m0 + row : M - 1;
      xv[i] = *reinterpret_cast<const u32x4*>(x + mr * K + int64_t(g) * kGroup + col * 8);
    }
  };
  auto store_x = [&](int buf, const u32x4 (&xv)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 256 * i, row = c >> 4, col = c & 15;
      *reinterpret_cast<u32x4*>(xs + (buf * kGemmBM + row) * kXStride + col * 8) = xv[i];
    }
  };
  struct W {
    u32x4 w[4];
    uint32_t s[4], z[4];
  };
  auto load_w = [&](int g, W& r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.w[j] = __builtin_nontemporal_load(wl[j] + int64_t(g) * (kTileBytes / 16));
      r.s[j] = swp[j][g * (kTileRows / 2)];
      r.z[j] = zwp[j][g * (kTileRows / 8)];
    }
  };

  f32x4 acc[kGemmMB][4];
#pragma unroll
  for (int a = 0; a < kGemmMB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xv[8];
  W cur, nxt;
  load_x(0, xv);
  load_w(0, cur);
  store_x(0, xv);
  __syncthreads();
  const uint32_t magic = kMagic1024;
  for (int g = 0; g < G; ++g) {
    const int buf = g & 1;
    const bool more = g + 1 < G;
    if (more) {
      load_x(g + 1, xv);
      load_w(g + 1, nxt);
    }
    // Per tile: the fp16 scale pair and the zero-point pairs of row rlane.
    half2_t s2[4];
    ZeroPairs zp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t sb = uint16_t((cur.s[j] >> ((rlane & 1) * 16)) & 0xFFFFu);
      s2[j] = as_h2(uint32_t(sb) * 0x00010001u);
      zp[j] = zero_pairs((cur.z[j] >> ((rlane & 7) * 4)) & 15u);
    }
    const _Float16* xa = xs + (buf * kGemmBM + wm * 64 + rlane) * kXStride + piece * 8;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      half8_t bw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        half2_t p[4];
        unpack8(cur.w[j][kb], magic, zp[j], p);
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = p[i] * s2[j];  // (q - z) * s, rounded once
        bw[j] = half8_t{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
      }
      half8_t af[kGemmMB];
#pragma unroll
      for (int mb = 0; mb < kGemmMB; ++mb) af[mb] = *reinterpret_cast<const half8_t*>(xa + mb * 16 * kXStride + kb * 32);
#pragma unroll
      for (int mb = 0; mb < kGemmMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bw[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      store_x(buf ^ 1, xv);  // buffer buf ^ 1 was last read before the previous barrier
      cur = nxt;
    }
    __syncthreads();
  }

  // D layout: lane l holds D[4 * (l / 16) + r][l % 16] of each 16 x 16 block.
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t t = tw + nb;
    const int64_t n = t * kTileRows + rlane;
    if (t >= NT || n >= N) continue;
#pragma unroll
    for (int mb = 0; mb < kGemmMB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 64 + mb * 16 + piece * 4 + r;
        if (m < M) y[m * N + n] = (_Float16)acc[mb][nb][r];
      }
  }
}

}  // namespace dev

int launch_gemm(int M, int N, int K, const void* wq, const void* scales, const void* zeros, const void* x, void* y,
                void* stream) {
  static const hipError_t raised = hipFuncSetAttribute(reinterpret_cast<const void*>(&dev::gemm_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       int(dev::kGemmLds));
  if (raised != hipSuccess) return int(raised);
  const int64_t NT = (int64_t(N) + kTileRows - 1) / kTileRows;
  const dim3 grid(unsigned((M + dev::kGemmBM - 1) / dev::kGemmBM),
                  unsigned((NT + dev::kGemmBN / kTileRows - 1) / (dev::kGemmBN / kTileRows)));
  return int(dev::launch_kernel(&dev::gemm_kernel, grid, dim3(256), dev::kGemmLds, static_cast<hipStream_t>(stream),
                                static_cast<const uint8_t*>(wq), static_cast<const uint16_t*>(scales),
                                static_cast<const uint8_t*>(zeros), static_cast<const _Float16*>(x),
                                static_cast<_Float16*>(y), M, N, K));
}

}  // namespace w4a16

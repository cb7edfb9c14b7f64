// Internal declarations shared by the host packer, the C-ABI front end and the
// HIP kernels of libw4a16.so (not part of the public ABI).
#pragma once

#include <cstddef>
#include <cstdint>

namespace w4a16 {

constexpr int kLayoutId = 1;
constexpr int kGroup = 128;
constexpr int kTileRows = 16;
constexpr int kTileBytes = 1024;  // 16 rows x 128 weights x 4 bits

// Geometry of the layout-ID-1 buffers of an N x K matrix.
struct Geometry {
  int64_t rows, cols, row_tiles, groups, groups_padded;
  Geometry(int64_t N, int64_t K)
      : rows(N),
        cols(K),
        row_tiles((N + kTileRows - 1) / kTileRows),
        groups(K / kGroup),
        groups_padded((K / kGroup + 7) / 8 * 8) {}
  size_t wq_bytes() const { return size_t(row_tiles) * size_t(groups) * kTileBytes; }
  size_t s_bytes() const { return size_t(row_tiles) * kTileRows * size_t(groups_padded) * 2; }
  size_t z_bytes() const { return size_t(row_tiles) * kTileRows * size_t(groups_padded) / 2; }
};

// Inner-product engine of the GEMV kernel.
enum Engine : int {
  kEngineDot2 = 0,      // v_dot2_f32_f16 on the VALU (M <= 2), x staged in LDS
  kEngineMfma = 1,      // v_mfma_f32_16x16x32_f16, x staged in LDS
  kEngineMfmaGlobalX = 2  // v_mfma_f32_16x16x32_f16, x read straight from global memory
};

// Launch parameters chosen by the front end for one GEMV shape.
struct LaunchPlan {
  int engine;  // Engine
  int waves;   // waves per workgroup: 1, 2, 4, 8 or 16
  int share;   // tiles a wave requests at once (2, 4, 8 or 12); longer shares take several rounds
  int splits;  // K ranges (gridDim.y); 1 for the plain GEMV
  int tiles_per_wg;  // row tiles per workgroup (gridDim.x = ceil(row tiles / this))
};

// Largest dynamic LDS a GEMV workgroup may use.
constexpr size_t kMaxLdsBytes = 64 * 1024;

// Dynamic LDS bytes of a GEMV launch (0 for kEngineMfmaGlobalX).
size_t lds_bytes(int M, int K, const LaunchPlan& plan);

// Whether the kernel set has an instantiation for this plan, within the LDS limit.
bool plan_supported(int M, int K, const LaunchPlan& plan);

// Kernel launchers (w4a16_kernels.hip). They return a hipError_t value as int.
int launch_gemv(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                const void* zeros, const void* x, void* y, float* partials, void* stream);
int launch_splitk_reduce(int M, int N, int splits, const float* partials, void* y, void* stream);
int launch_dequant(int N, int K, const void* wq, const void* scales, const void* zeros, float* out,
                   void* stream);

}  // namespace w4a16

// Internal declarations shared by the host packer, the C-ABI front end and the
// HIP kernels of libw4a16.so (not part of the public ABI).
#pragma once

#include <cstddef>
#include <cstdint>

namespace w4a16 {

constexpr int kLayoutId = 2;
constexpr int kGroup = 128;
constexpr int kTileRows = 16;
constexpr int kTileBytes = 1024;  // 16 rows x 128 weights x 4 bits

// Geometry of the layout-ID-2 buffers of an N x K matrix. Tile (t, g) is
// rows 16t..16t+15 of group g; all three buffers list tiles in the order
// t*G + g: 1024 weight bytes, 16 fp16 scales and 8 zero-point bytes each.
struct Geometry {
  int64_t rows, cols, row_tiles, groups;
  Geometry(int64_t N, int64_t K)
      : rows(N), cols(K), row_tiles((N + kTileRows - 1) / kTileRows), groups(K / kGroup) {}
  size_t wq_bytes() const { return size_t(row_tiles) * size_t(groups) * kTileBytes; }
  size_t s_bytes() const { return size_t(row_tiles) * kTileRows * size_t(groups) * 2; }
  size_t z_bytes() const { return size_t(row_tiles) * kTileRows * size_t(groups) / 2; }
  // Scale element of row n, group g (the zero point is nibble n&1 of byte
  // meta_index/2).
  int64_t meta_index(int64_t n, int64_t g) const {
    return ((n / kTileRows) * groups + g) * kTileRows + n % kTileRows;
  }
};

// Inner-product engine of the GEMV kernel.
enum Engine : int {
  kEngineMfma = 1,      // v_mfma_f32_16x16x32_f16, x staged in LDS
  kEngineMfmaGlobalX = 2  // v_mfma_f32_16x16x32_f16, x read straight from global memory
};

// What the GEMV kernel does with its sums.
enum Epilogue : int {
  kEpiStore = 0,   // y = fp16(sum) (or the split-K atomic accumulation)
  kEpiSwiglu = 1,  // row tile j: rows 0-7 gate, 8-15 up of outputs 8j..8j+7 -> y = fp16(silu(gate) * up)
};

// Launch parameters chosen by the front end for one GEMV shape.
struct LaunchPlan {
  int engine;  // Engine
  int waves;   // waves per workgroup: 1, 2, 4, 8 or 16
  int share;   // tiles a wave requests at once (2 .. 10); longer shares take several rounds
  int splits;  // K ranges (gridDim.y); 1 for the plain GEMV
  int tiles_per_wg;  // row tiles per workgroup: 1 (gridDim.x = row tiles)
  int epilogue;      // Epilogue (kEpiSwiglu: splits 1)
};

// Instantiated (waves, share) per engine and M: those that fit in registers
// without spilling, one row tile per workgroup; the SwiGLU epilogue for the
// same set. (Several row tiles per workgroup and a VALU dot2 engine were
// measured and dropped: the plans never chose them.)
constexpr bool instantiated(int mr, int waves, int share, int engine, int r, int epi = kEpiStore) {
  if (r != 1) return false;
  if (epi != kEpiStore && epi != kEpiSwiglu) return false;
  if (engine == kEngineMfmaGlobalX) return waves == 16 ? share <= 3 : share <= 4;
  if (engine != kEngineMfma) return false;
  if (waves == 16) return mr <= 2 ? share <= 10 : share <= 5;
  return !(waves == 8 && mr >= 3 && share >= 8);
}

// LDS of the cross-wave reduction: two buffers of [waves][4 pieces][rows][16]
// floats, rows = the MFMA D rows a lane holds that are activation rows.
constexpr size_t reduction_lds_bytes(int mr, int waves, int engine) {
  (void)engine;
  return 2 * size_t(waves) * 4 * (mr < 4 ? mr : 4) * 16 * sizeof(float);
}

// Halves per row of a wave's staged x slice: share * 128, plus 32 when
// there are several rows. An MFMA A-operand read takes rows 0 .. M-1 at
// four 16-byte column pieces; at an unpadded stride (a multiple of 256
// bytes, the span of the 64 banks) every row falls in the same banks, an
// up-to-8-way conflict on every read. A 64-byte pad puts row r's pieces at
// bank offset 64 r + 16 piece, at most 2-way for 8 rows (512 bytes take
// two passes anyway). One row is a broadcast and needs no padding.
constexpr int gemv_x_row(int mr, int share) { return share * kGroup + (mr > 1 ? 32 : 0); }

// Dynamic LDS of a GEMV workgroup: the reduction buffers, then one x slice
// [M][gemv_x_row] fp16 per wave (none when x is read from global memory).
constexpr size_t gemv_lds_bytes(int mr, int waves, int share, int engine, int epi) {
  (void)epi;
  return reduction_lds_bytes(mr, waves, engine) +
         (engine == kEngineMfmaGlobalX ? 0 : size_t(waves) * mr * gemv_x_row(mr, share) * 2);
}

// Largest dynamic LDS a GEMV workgroup may use: gfx950's 160 KiB per
// workgroup (a launch above 64 KiB first raises the kernel's limit).
constexpr size_t kMaxLdsBytes = 160 * 1024;
constexpr size_t kDefaultLdsLimit = 64 * 1024;

// Dynamic LDS bytes of a GEMV launch (0 for kEngineMfmaGlobalX).
size_t lds_bytes(int M, int K, const LaunchPlan& plan);

// Whether the kernel set has an instantiation for this plan, within the LDS limit.
bool plan_supported(int M, int K, const LaunchPlan& plan);

// Split-K: at most this many splits (the 5-bit arrival count of the
// accumulation word, see splitk_addend in w4a16_device.h), and a workspace of
// one uint64 accumulation word per output, zero between calls.
constexpr int kMaxSplits = 31;
constexpr size_t splitk_workspace_bytes(int M, int N) {
  return (size_t(8) * size_t(M) * size_t(N) + 15) / 16 * 16;
}

// Plans and launches a split-K GEMV (splits > 1) with accumulation words
// `acc` (all zero; left zero). Arguments already checked. Returns a W4A16
// status (api.cpp).
int gemv_splitk_status(int M, int N, int K, int splits, const void* wq, const void* scales, const void* zeros,
                       const void* x, void* y, unsigned long long* acc, void* stream);

// Kernel launchers (w4a16_kernels.hip). They return a hipError_t value as int.
// `acc` non-null selects split-K: it is the workspace above, all zero.
int launch_gemv(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                const void* zeros, const void* x, void* y, unsigned long long* acc, void* stream);
#define W4A16_DECLARE_M(MR)                                                                            \
  int launch_gemv_m##MR(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales, \
                        const void* zeros, const void* x, void* y, unsigned long long* acc, void* stream);
W4A16_DECLARE_M(1) W4A16_DECLARE_M(2) W4A16_DECLARE_M(3) W4A16_DECLARE_M(4)
W4A16_DECLARE_M(5) W4A16_DECLARE_M(6) W4A16_DECLARE_M(7) W4A16_DECLARE_M(8)
#undef W4A16_DECLARE_M
// INT8-activation variant (a8_kernels.hip). LDS of a GEMV workgroup: the
// reduction buffers [waves][4][min(M, 4)][16] floats, then per wave the
// activation codes [M][share][128] bytes and [share][16] fp32 scales and
// int32 code sums.
constexpr size_t gemv_a8_lds_bytes(int mr, int waves, int share) {
  return size_t(waves) * 4 * (mr < 4 ? mr : 4) * 16 * sizeof(float) +
         size_t(waves) * (size_t(mr) * share * kGroup + size_t(share) * 16 * 8);
}
// Instantiated (waves, share): waves 1..16 (powers of two), shares 4, 7, 10,
// within the LDS of a workgroup; not 16 waves of 10-tile shares for 4 or
// more rows, whose registers (at most 128 per lane in a 1024-thread
// workgroup) cannot hold the staged codes of a round without spilling:
// those take 7-tile shares in two rounds.
constexpr bool a8_instantiated(int mr, int waves, int share) {
  return (waves == 1 || waves == 2 || waves == 4 || waves == 8 || waves == 16) &&
         (share == 4 || share == 7 || share == 10) && !(waves == 16 && share == 10 && mr >= 4) &&
         gemv_a8_lds_bytes(mr, waves, share) <= kMaxLdsBytes;
}
// The fused-quantization variant holds a round's fp16 x in registers (one
// 16-byte load per lane per 4 groups of the [M][share] slice): built where
// M * share <= 40; in 1024-thread workgroups (128 registers per lane), for
// two or more rows, with 4-tile shares, or 7-tile shares up to 3 rows
// (beyond that the compiler spills).
constexpr bool a8_fused_instantiated(int mr, int waves, int share) {
  return a8_instantiated(mr, waves, share) && mr * share <= 40 &&
         !(waves == 16 && mr >= 2 && (share == 10 || (share == 7 && mr >= 4)));
}
int launch_act_quant_i8(int M, int K, const void* x, void* xq, void* sx, void* xsum, void* stream);
int launch_gemv_a8(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                   const void* zeros, const void* xq, const void* sx, const void* xsum, void* y, void* stream);
int launch_gemv_a8_fused(int M, int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                         const void* zeros, const void* x, void* y, void* stream);
// The GEMM addresses a workgroup's (at most 128) rows of x with 32-bit
// element offsets (below 128 K), so K stays under 2^25.
constexpr int kGemmMaxK = 1 << 25;
// 16-row m blocks per GEMM wave (the workgroup's rows / 16): the fewest that
// cover M, up to 8. A 128-row tile at M = 16 spends 7/8 of its matrix-core
// work on padding rows.
constexpr int gemm_m_blocks(int M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8; }
// An unsplit launch above 64 rows takes 64-row tiles where their grid still
// fits one workgroup per CU (ceil(M/64) x 128-column strips <= 256: a narrow
// matrix, whose 128-row grid leaves most CUs idle), or where the second of
// two 128-row tiles would be at most half used (128 < M <= 192); 128-row
// tiles otherwise. Measured on MI355X (7B shapes, unsplit, µs): 3584x18944 at
// M = 192 124.0 against 146.7, at M = 512 122.1 against 147.0; 4608x3584 at
// M = 448 29.3 against 31.3 (at M = 512, 288 workgroups: 33.7 against 31.6);
// 37888x3584 at M = 160 79.1 against 88.7, at M = 320 114.2 against 110.4.
// Split launches keep gemm_m_blocks, to which their split rules are fitted.
// Each output's sum is the same sequence of MFMAs for every tile height.
constexpr int gemm_m_blocks_unsplit(int M, int N) {
  if (M <= 64) return gemm_m_blocks(M);
  const long long strips = (static_cast<long long>(N) + 127) / 128;
  return ((static_cast<long long>(M) + 63) / 64 * strips <= 256 || (M > 128 && M <= 192)) ? 4 : 8;
}
// splits > 1 takes `ws`, the split-K workspace above (all zero), or, when
// `part` is non-null, fp32 partials part[splits][M][N] summed by a second
// launch; 1 ignores both.
int launch_gemm(int M, int N, int K, int splits, const void* wq, const void* scales, const void* zeros,
                const void* x, void* y, unsigned long long* ws, void* stream, float* part = nullptr);
// Bytes of the fp32 partials of w4a16_gemm_splitk_partials: 4 * splits * M * N,
// rounded up to 16.
constexpr size_t gemm_partials_bytes(int M, int N, int splits) {
  return (size_t(4) * size_t(splits) * size_t(M) * size_t(N) + 15) / 16 * 16;
}
int launch_dequant_f16(int N, int K, const void* wq, const void* scales, const void* zeros, void* out,
                       void* stream);
int launch_read_probe(const void* buf, size_t bytes, int grid, void* sink, void* stream);
int launch_dequant(int N, int K, const void* wq, const void* scales, const void* zeros, float* out,
                   void* stream);

}  // namespace w4a16

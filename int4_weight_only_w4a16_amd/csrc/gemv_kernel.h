// The GEMV kernel template and its launchers (included by one translation
// unit per activation-row count M, so the instantiations compile in parallel).
//
// GEMV y = W x with W in layout ID 2 (16-row x 128-column tiles of 1 KiB,
// each with 32 bytes of scales and 8 bytes of zero points).
// Per tile a lane issues one 16-byte non-temporal load (32 weights of its
// row), turns the nibbles into exact fp16 (q - z) pairs in registers and
// feeds them to the inner product; each group's fp32 sum is scaled once by s.
// All sums run in a fixed order, so results are bit-identical run to run
// (the determinism rule of the qengine page, "Learnings").
#pragma once

#include "w4a16_device.h"

namespace w4a16 {
namespace dev {

// Workgroup = WAVES waves over R row tiles, t = blockIdx.x + r * gridDim.x
// (r < R), and one K range blockIdx.y of gridDim.y. The waves take
// contiguous shares of the range's groups, in rounds of at most SHARE tiles
// (one round for every shape the launch table picks: a wave then stages its
// x slice in its private LDS region once and reuses it for all R row tiles,
// and requests the next row tile's round before computing the current one).
// The waves' partial sums meet in LDS (double-buffered across row tiles, one
// barrier per row tile) and are added in wave order.
// EPI == kEpiSwiglu: row tile j of the matrix holds the gate rows of
// outputs 8j .. 8j+7 in its rows 0-7 and their up rows in rows 8-15, so a
// workgroup runs exactly the plain GEMV's waves and shares, and its
// cross-wave sum holds both projections of 8 outputs: y[m][8j + i] =
// fp16(silu(g) * u) with g the sum of row i, u that of row i + 8 and
// silu(g) = g / (1 + e^-g) in fp32. N is the output width (the matrix has
// ceil(N/8) row tiles); never with split K.
// Writes fp16 y[MR][N] directly when `acc` is null. Otherwise (split-K,
// gridDim.y splits) each workgroup adds its fp32 partial sums, in the
// fixed-point word format of splitk_addend(), to acc[MR][N] (one uint64 per
// output) with a relaxed device-scope atomic add. The word also counts the
// arrivals, so the workgroup whose add completes the count finds the whole
// sum in the value its atomic returned: it writes y and resets the word to
// zero for the next call. Integer addition is exact and order-free, so y
// does not depend on the order in which the splits arrive; and each output
// lives in one atomic location, so no fence is needed.
// The sizes and the split count come first among the arguments, and the
// split count is an argument rather than gridDim.y, so that everything the
// kernel needs at entry arrives in preloaded SGPRs (no scalar load).
template <int MR, int WAVES, int SHARE, int ENGINE, int R, int EPI>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(
    int N, int K, int splits, const uint8_t* __restrict__ wq, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const _Float16* __restrict__ x, _Float16* __restrict__ y,
    unsigned long long* __restrict__ acc) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr bool kGlobalX = ENGINE == kEngineMfmaGlobalX;
  // Accumulators per lane: the MFMA D rows a lane can hold (4*piece + r)
  // that are activation rows, at most 4.
  constexpr int kAcc = MR < 4 ? MR : 4;
  constexpr int kXRow = gemv_x_row(MR, SHARE);          // halves per staged x row of a wave (padded)
  // Per-wave partial sums in LDS: every lane writes its kRows accumulators
  // (no lane-dependent branch, which would let the compiler move the whole
  // scale chain, and the scale loads with it, behind the barrier).
  constexpr int kRows = kAcc;
  constexpr int kRedWave = 4 * kRows * 16;               // floats per wave: [piece][kRows][16]
  constexpr int kRed = WAVES * kRedWave;                 // floats per reduction buffer
  float* red = reinterpret_cast<float*>(smem);           // [2][WAVES][4][kRows][16]

  const int G = K / kGroup;
  constexpr bool kRows8 = EPI == kEpiSwiglu;  // 8 outputs per row tile: gate rows 0-7, up rows 8-15
  const int64_t row_tiles = kRows8 ? (int64_t(N) + 7) / 8 : (int64_t(N) + kTileRows - 1) / kTileRows;
  const int split = blockIdx.y;  // splits == gridDim.y, passed as an argument
  // The split's groups. No division for the usual unsplit launch; else a
  // 32-bit one (split * G < 31 * 2^24): the 64-bit division compiled to
  // some 130 instructions per wave before the first request.
  const int g_beg = splits == 1 ? 0 : int(unsigned(split) * unsigned(G) / unsigned(splits));
  const int g_end = splits == 1 ? G : int(unsigned(split + 1) * unsigned(G) / unsigned(splits));
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
                 (kGlobalX ? 0 : wave * MR * kXRow);  // x slice [MR][kXRow]
  int parity = 0;

  // Copy x[:, 128*g0 : 128*(g0+n)) into this wave's LDS slice (synchronous).
  auto stage_x = [&](int g0, int n) {
    if constexpr (!kGlobalX) {
      const int xchunks = n * (kGroup / 8), xtotal = MR * xchunks;
      for (int c = lane; c < xtotal; c += 64) {
        const int m = row_of_chunk<MR>(c, xchunks), cc = c - m * xchunks;
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
    // The aligned 32-bit words holding the lane's fp16 scale and zero
    // nibble. Whole words need no widening after the load: a widening is
    // placed where the value is used, and when a branch separates loads and
    // uses the compiler puts all of them, and so all the waits, before the
    // first tile. The fields are cut out inside each tile, after its wait.
    uint32_t sw[SHARE], zw[SHARE];
    half8_t xa[kGlobalX ? SHARE : 1][4];
  };
  auto load_round = [&](Round& r, const u32x4* wlane, const uint32_t* sword, const uint32_t* zword, int g0,
                        int n) {
#pragma unroll
    for (int u = 0; u < SHARE; ++u) {
      const int gg = g0 + min(u, n - 1);
      r.w[u] = __builtin_nontemporal_load(wlane + int64_t(gg) * (kTileBytes / 16));
      r.sw[u] = sword[gg * (kTileRows / 2)];  // 16 scales = 8 words per tile
      r.zw[u] = zword[gg * (kTileRows / 8)];  // 16 nibbles = 2 words per tile
      if constexpr (kGlobalX) {
        const _Float16* xl = x + int64_t(mm) * K + int64_t(gg) * kGroup + 8 * piece;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) r.xa[u][kb] = *reinterpret_cast<const half8_t*>(xl + 32 * kb);
      }
    }
  };
  auto compute_round = [&](const Round& r, int g0, int n, float (&acc)[kAcc]) {
    // The staged x slice does not change between row tiles, so the compiler
    // would reuse every x read across row tiles and keep the whole slice in
    // registers (100+ VGPRs, a quarter of the occupancy). An opaque copy of
    // the lane's offset keeps the reads next to their use. (The offset, not
    // the pointer: an opaque pointer would lose its LDS address space.)
    int xoff = 8 * piece;
    asm volatile("" : "+v"(xoff));
    const _Float16* xbase = xw + xoff;
    // MFMA: each tile's group sums stay in their own registers and are scaled
    // after the last tile, so a tile's unpack never waits for the previous
    // tile's MFMA chain to finish (same fp32 operations, same order).
    f32x4 dsave[SHARE];
    float ssave[SHARE];
#pragma unroll
    for (int u = 0; u < SHARE; ++u) {
      __builtin_amdgcn_sched_barrier(0);  // keep tiles in request order
      // Pass this tile's registers through an (empty) volatile asm: the
      // asm statements stay in program order, and nothing computed from the
      // tile can move above its asm, so no tile's unpack is hoisted ahead of
      // earlier tiles (which would wait for every load at once).
      u32x4 wt = r.w[u];
      uint32_t zt = r.zw[u], st = r.sw[u];
      asm volatile("" : "+v"(wt), "+v"(zt), "+v"(st));
      // Row rlane's zero nibble is nibble rlane % 8 of its word; its scale
      // the half rlane % 2 of its word.
      const ZeroPairs zp = zero_pairs((zt >> ((rlane & 7) * 4)) & 15u);
      const float s = half_bits_to_float((st >> ((rlane & 1) * 16)) & 0xFFFFu);
      const _Float16* xg = xbase + u * kGroup;
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        half2_t p[4];
        unpack8(wt[kb], magic, zp, p);
        const half8_t bw = {p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
        half8_t ax;
        if constexpr (kGlobalX)
          ax = r.xa[u][kb];
        else
          ax = *reinterpret_cast<const half8_t*>(xg + mm * kXRow + 32 * kb);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, bw, d, 0, 0, 0);
      }
      dsave[u] = d;
      ssave[u] = s;
    }
#pragma unroll
    for (int u = 0; u < SHARE; ++u) {
      const bool valid = u < n;
#pragma unroll
      for (int r2 = 0; r2 < kAcc; ++r2) acc[r2] = valid ? __builtin_fmaf(dsave[u][r2], ssave[u], acc[r2]) : acc[r2];
    }
  };

  const int share_n = share_end - share_beg;
  const bool one_round = share_n <= SHARE;

  // Cross-wave sum of one row tile: each wave's partials go to LDS and the
  // first threads add them in wave order. One barrier per row tile: the next
  // tile writes the other buffer, and the tile after that is behind this
  // tile's next barrier. The sums stay in registers and are stored after the
  // last tile, so no store sits between a weight request and its use.
  constexpr int kOut = (MR * 16 + WAVES * 64 - 1) / (WAVES * 64);  // outputs per thread per tile
  auto reduce_tile = [&](float (&acc)[kAcc], float (&out)[kOut]) {
    float* rb = red + parity * kRed;
    // Lane l holds D[4*(l/16) + r][l%16], i.e. activation row 4*piece + r of
    // weight row rlane.
#pragma unroll
    for (int r = 0; r < kRows; ++r) rb[wave * kRedWave + (piece * kRows + r) * 16 + rlane] = acc[r];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      if constexpr (kRows8) {
        // Output (m, i) of the tile: gate row i, up row i + 8.
        const int idx = min(tid + j * WAVES * 64, MR * 8 - 1);
        const int m = idx >> 3, i = idx & 7;
        const int slot = ((m >> 2) * kRows + (m & 3)) * 16 + i;
        float g = rb[slot], u = rb[slot + 8];
#pragma unroll
        for (int w2 = 1; w2 < WAVES; ++w2) {
          g += rb[w2 * kRedWave + slot];
          u += rb[w2 * kRedWave + slot + 8];
        }
        // silu(gate) * up, rounded to fp32 before the fp16 store rounds it
        // again: held in a register, the product cannot be fused into the
        // store's conversion (a single-rounding v_fma_mix, which the compiler
        // picks for some code shapes only), so every kernel computing this
        // epilogue rounds the same way.
        float su = g / (1.f + expf(-g)) * u;
        asm volatile("" : "+v"(su));
        out[j] = su;
        continue;
      }
      const int idx = min(tid + j * WAVES * 64, MR * 16 - 1);  // one wave has fewer lanes than 8 x 16 outputs
      const int m = idx >> 4, i = idx & 15;
      const int slot = ((m >> 2) * kRows + (m & 3)) * 16 + i;
      float sum = rb[slot];
#pragma unroll
      for (int w2 = 1; w2 < WAVES; ++w2) sum += rb[w2 * kRedWave + slot];
      out[j] = sum;
    }
    parity ^= 1;
  };
  auto store_tile = [&](int64_t t, const float (&out)[kOut]) {
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      if constexpr (kRows8) {
        const int idx = tid + j * WAVES * 64;
        const int m = idx >> 3, i = idx & 7;
        const int64_t nn = t * 8 + i;
        if (idx < MR * 8 && nn < N) y[int64_t(m) * N + nn] = (_Float16)out[j];
        continue;
      }
      const int idx = tid + j * WAVES * 64;
      const int m = idx >> 4, i = idx & 15;
      const int64_t nn = t * kTileRows + i;
      if (idx < MR * 16 && nn < N) y[int64_t(m) * N + nn] = (_Float16)out[j];
    }
  };
  struct TilePtrs {
    const u32x4* wlane;
    const uint32_t* sword;  // word of tile (t, 0)'s scale block holding row rlane's scale
    const uint32_t* zword;  // word of tile (t, 0)'s zero block holding row rlane's nibble
  };
  auto tile_ptrs = [&](int64_t t) {  // t < row tiles: always valid memory
    const int64_t q0 = t * G;           // index of tile (t, 0)
    return TilePtrs{reinterpret_cast<const u32x4*>(wq + q0 * kTileBytes) + lane,
                    reinterpret_cast<const uint32_t*>(scales) + q0 * (kTileRows / 2) + (rlane >> 1),
                    reinterpret_cast<const uint32_t*>(zeros) + q0 * (kTileRows / 8) + (rlane >> 3)};
  };

  // This workgroup's row tiles: t0 + r * gridDim.x for r < R (the host
  // launches ceil(row tiles / R) workgroups, so t0 is in range). Tiles past
  // the end are computed on a clamped (valid) tile and never stored.
  const int64_t t0 = blockIdx.x;
  auto tile_of = [&](int r) { return t0 + int64_t(r) * gridDim.x; };
  auto clamp_tile = [&](int64_t t) { return t < row_tiles ? t : row_tiles - 1; };
  float sums[R][kOut];

  if (one_round && share_n > 0) {
    // Straight-line software pipeline over the R row tiles: the next tile's
    // round is requested before the current one is computed, in two register
    // sets. No branch and no store on this path, so every wait is exact.
    Round rr[2];
    {
      const TilePtrs p = tile_ptrs(tile_of(0));
      if constexpr (!kGlobalX) {
        // x requests go out just ahead of the first weight requests, so the
        // wait before the LDS store is for x alone; the staged slice then
        // serves all of this workgroup's row tiles. Chunk c of the slice is
        // row c / kRowChunks, a division by a constant (one row: none); in a
        // short share the chunks past its groups take a copy of the row's
        // last chunk. (Dividing by the share's own chunk count cost some
        // 20 vector instructions per chunk, 380 per wave at M = 8, all ahead
        // of the first weight request. Direct global-to-LDS requests, which
        // need no registers, measured slower than this from two rows on:
        // before the first LDS read the compiler waits for every
        // outstanding load, the whole round of weights included.)
        constexpr int kRowChunks = SHARE * (kGroup / 8);
        constexpr int kXSteps = (MR * kRowChunks + 63) / 64;
        const int xlast = share_n * (kGroup / 8) - 1;
        auto chunk = [&](int j, int& m, int& cc) {  // clamped: unconditional, in bounds
          const int c = min(lane + 64 * j, MR * kRowChunks - 1);
          m = MR == 1 ? 0 : c / kRowChunks;
          cc = min(c - m * kRowChunks, xlast);
        };
        u32x4 xv[kXSteps];
#pragma unroll
        for (int j = 0; j < kXSteps; ++j) {
          int m, cc;
          chunk(j, m, cc);
          xv[j] = *reinterpret_cast<const u32x4*>(x + int64_t(m) * K + int64_t(share_beg) * kGroup + cc * 8);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_round(rr[0], p.wlane, p.sword, p.zword, share_beg, share_n);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kXSteps; ++j) {  // clamped chunks rewrite a chunk with its own data
          int m, cc;
          chunk(j, m, cc);
          *reinterpret_cast<u32x4*>(xw + m * kXRow + cc * 8) = xv[j];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
      } else {
        load_round(rr[0], p.wlane, p.sword, p.zword, share_beg, share_n);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r + 1 < R) {
        const TilePtrs p = tile_ptrs(clamp_tile(tile_of(r + 1)));
        load_round(rr[(r + 1) & 1], p.wlane, p.sword, p.zword, share_beg, share_n);
      }
      float acc[kAcc];
#pragma unroll
      for (int i = 0; i < kAcc; ++i) acc[i] = 0.f;
      compute_round(rr[r & 1], share_beg, share_n, acc);
      reduce_tile(acc, sums[r]);
    }
  } else {
    // Long K (several rounds per share, x restaged per round) or an empty
    // share (a K range with fewer groups than waves): plain loop.
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const TilePtrs p = tile_ptrs(clamp_tile(tile_of(r)));
      float acc[kAcc];
#pragma unroll
      for (int i = 0; i < kAcc; ++i) acc[i] = 0.f;
      for (int g0 = share_beg; g0 < share_end; g0 += SHARE) {
        const int n = min(SHARE, share_end - g0);
        stage_x(g0, n);
        Round rd;
        load_round(rd, p.wlane, p.sword, p.zword, g0, n);
        compute_round(rd, g0, n, acc);
      }
      reduce_tile(acc, sums[r]);
    }
  }
  if (!acc || kRows8) {  // (the host never pairs kEpiSwiglu with split K)
#pragma unroll
    for (int r = 0; r < R; ++r) store_tile(tile_of(r), sums[r]);
    return;
  }
  // Split-K: one relaxed device-scope atomic add per output and row tile.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t t = tile_of(r);
#pragma unroll
    for (int j = 0; j < kOut; ++j) {
      const int idx = tid + j * WAVES * 64;
      const int m = idx >> 4, i = idx & 15;
      const int64_t nn = t * kTileRows + i;
      if (idx < MR * 16 && nn < N && t < row_tiles) {
        unsigned long long* word = acc + int64_t(m) * N + nn;
        const unsigned long long add = splitk_addend(sums[r][j]);
        const unsigned long long now =
            __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
        if (splitk_count(now) == unsigned(splits)) {
          y[int64_t(m) * N + nn] = splitk_value(now, splits);
          // Every split has added: nothing else touches the word in this call.
          __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

template <int MR, int WAVES, int SHARE, int ENGINE, int EPI>
constexpr size_t lds_for() {
  return gemv_lds_bytes(MR, WAVES, SHARE, ENGINE, EPI);
}

template <int MR, int WAVES, int SHARE, int ENGINE, int R, int EPI>
hipError_t launch_typed(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                        const void* zeros, const void* x, void* y, unsigned long long* acc, hipStream_t stream) {
  const int64_t row_tiles = EPI == kEpiSwiglu ? (int64_t(N) + 7) / 8  // 8 outputs per tile
                                                  : (int64_t(N) + kTileRows - 1) / kTileRows;
  const int64_t grid = (row_tiles + R - 1) / R;
  constexpr size_t lds = lds_for<MR, WAVES, SHARE, ENGINE, EPI>();
  if constexpr (lds > kDefaultLdsLimit) {
    static std::atomic<uint64_t> raised{0};  // devices on which this instantiation's limit is raised
    const hipError_t e = raise_lds_limit(
        reinterpret_cast<const void*>(&gemv_kernel<MR, WAVES, SHARE, ENGINE, R, EPI>), lds, raised);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(&gemv_kernel<MR, WAVES, SHARE, ENGINE, R, EPI>, dim3(unsigned(grid), unsigned(plan.splits)),
                       dim3(WAVES * 64), lds, stream, N, K, plan.splits, static_cast<const uint8_t*>(wq),
                       static_cast<const uint16_t*>(scales), static_cast<const uint8_t*>(zeros),
                       static_cast<const _Float16*>(x), static_cast<_Float16*>(y), acc);
}

template <int MR, int ENGINE>
hipError_t launch_shape(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                        const void* zeros, const void* x, void* y, unsigned long long* acc, hipStream_t stream) {
#define W4A16_CASE(W, S, RR, EP)                                                                            \
  if constexpr (instantiated(MR, W, S, ENGINE, RR, EP)) {                                                  \
    if (plan.waves == W && plan.share == S && plan.tiles_per_wg == RR && plan.epilogue == EP)              \
      return launch_typed<MR, W, S, ENGINE, RR, EP>(N, K, plan, wq, scales, zeros, x, y, acc, stream); \
  }
#define W4A16_SHARES(W, EP)                                                                             \
  W4A16_CASE(W, 2, 1, EP) W4A16_CASE(W, 3, 1, EP) W4A16_CASE(W, 4, 1, EP) W4A16_CASE(W, 5, 1, EP)        \
  W4A16_CASE(W, 7, 1, EP) W4A16_CASE(W, 8, 1, EP) W4A16_CASE(W, 10, 1, EP)
#define W4A16_WAVES(EP) \
  W4A16_SHARES(1, EP) W4A16_SHARES(2, EP) W4A16_SHARES(4, EP) W4A16_SHARES(8, EP) W4A16_SHARES(16, EP)
  W4A16_WAVES(kEpiStore) W4A16_WAVES(kEpiSwiglu)
#undef W4A16_WAVES
#undef W4A16_SHARES
#undef W4A16_CASE
  return hipErrorInvalidValue;
}

template <int MR>
hipError_t launch_engine(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                         const void* zeros, const void* x, void* y, unsigned long long* acc, hipStream_t stream) {
  switch (plan.engine) {
    case kEngineMfma:
      return launch_shape<MR, kEngineMfma>(N, K, plan, wq, scales, zeros, x, y, acc, stream);
    case kEngineMfmaGlobalX:
      return launch_shape<MR, kEngineMfmaGlobalX>(N, K, plan, wq, scales, zeros, x, y, acc, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dev
}  // namespace w4a16

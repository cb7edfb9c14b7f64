// A chain of dependent W4A16 GEMVs in one persistent launch (w4a16_chain_plan,
// w4a16_chain_run): a whole decode step of GEMVs, each reading its input from
// an earlier GEMV's output, without a launch boundary between them.
//
// Why: between two dependent GEMV launches the GPU streams no weights. The
// qengine page gets its matrix kernels to 94.9% of bandwidth inside the
// decode loop by letting each kernel start loading while the previous one
// finishes ("Why speed is a byte count", "How it works": programmatic
// dependent launch, the DeltaNet kernel started ahead of its wait). Here a
// workgroup requests the weights of its next work items before it waits for
// their input, so the weight stream goes on across every dependency.
//
// Structure. Two workgroups of 8 waves per compute unit, all resident at
// once (checked at launch). The chain's work items -- (GEMV, 16-row tile or
// tile pair, K range) -- are numbered in chain order, and workgroup w takes
// items w, w + P, w + 2P, ... (P workgroups). A wave takes a fixed share of
// every item's K range (as the standalone kernels' waves do), in rounds of
// at most 7 tiles when the share is longer. Per round it (1) requests the
// weights of the round NBUF - 1 rounds on, (2) multiplies the round whose
// weights were requested a round ago, with x from LDS, and, at an item's last
// round, (3) hands its fp32 partial sums in through an LDS slot. At the
// first round of a GEMV the waves first stage the GEMV's whole input into
// LDS -- wave 0 polls the producer's last output word, the others wait in
// LDS -- while that round's weights are already in flight.
// The epilogue of an item (its partial sums added in wave order, then the
// fp16 store, SwiGLU, or the split-K fixed-point atomics) rotates over the
// waves: wave o % 8 does item o's one item later, when every wave has
// almost always handed it in, or at once for the workgroup's last item of a
// GEMV, whose consumers wait for it.
//
// Handoff between GEMVs. A GEMV whose output feeds another also writes each
// output as a 32-bit word (fp16 bits | tag << 16) with device-scope stores,
// tag = a 16-bit number of this launch, never 0 (it comes from the
// workspace and the last workgroup to finish advances it). A consumer
// accepts a word only when its tag is this launch's: no word from an
// earlier launch or an unfinished producer is ever used, whatever order the
// stores become visible in, and no fence or counter is needed. Stale words
// are requested again with device-scope loads until they carry the tag.
//
// Progress. Item k waits only for GEMVs of smaller item numbers, every
// workgroup takes its items in increasing order, and all workgroups are
// resident, so the smallest unfinished item can always finish. Inside a
// workgroup every wait is for an earlier item (a slot is reused once the
// epilogue of the item 4 before has run; an epilogue waits for the item's
// hand-ins; a deferred epilogue never crosses into the next GEMV). Every
// wait is bounded (kWaitTicks of the 100 MHz real-time counter); a wait that
// runs out sets the workspace error word and every workgroup leaves.
//
// The arithmetic of an item is that of the standalone kernels with the same
// waves and shares (w4a16_gemv and w4a16_gemv_swiglu: 4 waves per tile at
// 28 groups; w4a16_gemv_splitk: 8 waves of the split's range), so each output
// equals theirs bit for bit where the plans coincide.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <vector>

#include "w4a16.h"
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace w4a16 {
namespace chain {

using dev::f32x4;
using dev::u32x4;

constexpr int kWaves = 8;   // waves per workgroup, all computing
constexpr int kThreads = kWaves * 64;
constexpr int kShare = 7;   // tiles per wave and round, at most
constexpr int kSlots = 4;   // partial-sum slots of a workgroup (items a wave may run ahead)
constexpr uint32_t kMagic = 0x57344348u;  // "W4CH"
constexpr uint64_t kWaitTicks = 100000000ull;  // 1 s of the 100 MHz counter

// Workspace control words (uint32, first 256 bytes): launch number, finished
// workgroups, error.
enum : int { kWsEpoch = 0, kWsFinished = 1, kWsError = 2 };
constexpr size_t kWsHeader = 256;

// Device addresses are kept as integers and read back as global-memory
// pointers: a pointer loaded from memory would otherwise be a generic (flat)
// one, and flat loads also count against the LDS wait counter.
#define W4A16_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ W4A16_GLOBAL T* gptr(uint64_t a) {
  return reinterpret_cast<W4A16_GLOBAL T*>(a);
}

struct alignas(16) OpDev {
  uint64_t wq;
  uint64_t sw;           // scales, as 32-bit words
  uint64_t zw;           // zero points, as 32-bit words
  uint64_t x_ext;        // external fp16 input [M][K] when x_src < 0
  uint64_t y;            // fp16 output [M][N]
  uint64_t yt_off;       // workspace offset of this GEMV's tagged output [M][N] (0: nobody reads it)
  uint64_t xt_off;       // workspace offset of the producer's tagged output (x_src >= 0)
  uint64_t acc_off;      // workspace offset of the split-K words [M][N] (splits > 1)
  int32_t N, K, G, kind;
  int32_t splits, tp, wpt, row_tiles;       // tiles per item, waves per tile, matrix row tiles
  int32_t per_split, items, item_begin, x_shift;
  int32_t x_stride;   // producer's N: row stride of its tagged output, in words
  int32_t sentinel;   // word of the producer's tagged output polled before staging
  int32_t x_src;
  int32_t split_q;    // G / splits
  int32_t rounds;     // rounds of at most kShare tiles per wave and item
  int32_t pad[3];
};
static_assert(sizeof(OpDev) == 144, "descriptor size");

struct alignas(16) Header {
  uint32_t magic;
  int32_t M, n_ops, total_items;
  uint64_t plan_bytes, ws_bytes;
  int32_t reserved[8];
};
static_assert(sizeof(Header) == 64, "header size");

// LDS control block.
struct LdsCtl {
  int ready;             // highest GEMV index whose producer wave 0 has seen finish
  int abort;             // nonzero: leave
  int cnt[kSlots];       // waves that have written the slot's partial sums
  int gen[kSlots];       // times the slot has been consumed
  int xstaged;           // waves that have staged their part of the x buffer, over all its uses
  int xfreed;            // waves that are done with the x buffer, over all its uses
  int pad[4];
};
static_assert(sizeof(LdsCtl) == 64, "LDS control block");

// Control words are read the same by every lane: reading the value back from
// the first lane tells the compiler so, and keeps every decision made on it
// (and all the walk state behind it) in scalar registers.
__device__ __forceinline__ uint32_t ld_dev(const W4A16_GLOBAL uint32_t* p) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_dev(W4A16_GLOBAL uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int lds_ld(const int* p) {
  return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
}
__device__ __forceinline__ void lds_st(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local"); }
__device__ __forceinline__ void lds_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local"); }

// Bounded waiting: a wait gives up after kWaitTicks without progress
// (setting the workspace error word and the workgroup's abort flag), or at
// once when another wave of the workgroup has given up; a wait for another
// workgroup also gives up when some workgroup has reported an error.
struct Waiter {
  LdsCtl* lc;
  W4A16_GLOBAL uint32_t* ctl;
  bool failed = false;

  __device__ __forceinline__ void fail(uint32_t code) {
    st_dev(ctl + kWsError, code);
    lds_st(&lc->abort, 1);
    failed = true;
  }
  // True while the wait that began at t0 may go on.
  __device__ __forceinline__ bool may_wait(uint64_t t0, bool global) {
    if (lds_ld(&lc->abort) || (global && ld_dev(ctl + kWsError))) {
      lds_st(&lc->abort, 1);
      failed = true;
      return false;
    }
    if (wall_clock64() - t0 > kWaitTicks) {
      fail(1u);
      return false;
    }
    return true;
  }
  // Waits until the LDS word reaches `target`; false if the wait gave up.
  __device__ __forceinline__ bool wait_lds(int* word, int target) {
    const uint64_t t0 = wall_clock64();
    while (lds_ld(word) < target) {
      if (!may_wait(t0, false)) return false;
      __builtin_amdgcn_s_sleep(1);
    }
    lds_acquire();
    return true;
  }
};

// A workgroup's walk over its items (every P-th item of the chain) and over
// each item's rounds, kept in scalar registers: the item, its GEMV's
// fields, its split and tile group, and the round. Advancing by P costs no
// division: a split boundary is crossed by subtraction, and the split's
// groups [floor(s G / S), floor((s+1) G / S)) are tracked incrementally as s
// grows. Divisions happen only when the walk enters a new GEMV.
struct Walk {
  int k, op, end, rd;      // item, its GEMV, first item past that GEMV, round
  int split, tg;           // split and tile group of item k
  int g_beg, g_end, r_end; // the split's groups; r_end = (split + 1) G mod S
  int splits, per_split, row_tiles;
  int shape;               // kind | log2(waves per tile) << 1 | tiles per item << 3 | rounds << 6
  __device__ int kind() const { return shape & 1; }
  __device__ int wpt_log2() const { return (shape >> 1) & 3; }
  __device__ int tp() const { return (shape >> 3) & 7; }
  __device__ int rounds() const { return shape >> 6; }
};

__device__ __forceinline__ void walk_enter(Walk& w, const OpDev* ops) {
  while (w.k >= ops[w.op].item_begin + ops[w.op].items) ++w.op;
  const OpDev& d = ops[w.op];
  w.end = d.item_begin + d.items;
  w.rd = 0;
  w.splits = d.splits, w.per_split = d.per_split, w.row_tiles = d.row_tiles;
  w.shape = d.kind | (d.wpt == 8 ? 3 : 2) << 1 | d.tp << 3 | d.rounds << 6;
  const int i = w.k - d.item_begin;
  w.split = i / w.per_split;
  w.tg = i - w.split * w.per_split;
  w.g_beg = w.split * d.G / w.splits;
  const int next = (w.split + 1) * d.G;
  w.g_end = next / w.splits;
  w.r_end = next - w.g_end * w.splits;
}

// Moves the walk one round on: to the item's next round, or P items on
// (within `total`).
__device__ __forceinline__ void walk_advance(Walk& w, const OpDev* ops, int P, int total) {
  if (++w.rd < w.rounds()) return;
  w.rd = 0;
  w.k += P;
  if (w.k >= total) return;
  if (w.k >= w.end) {
    walk_enter(w, ops);
    return;
  }
  w.tg += P;
  while (w.tg >= w.per_split) {
    const OpDev& d = ops[w.op];
    w.tg -= w.per_split;
    ++w.split;
    w.g_beg = w.g_end;
    w.g_end += d.split_q;
    w.r_end += d.G - d.split_q * w.splits;
    if (w.r_end >= w.splits) {
      ++w.g_end;
      w.r_end -= w.splits;
    }
  }
}

// Where a wave works in a round of an item: the matrix row tile it reads and
// the round's part of its share of the item's K range (waves per tile: 4 or
// 8; up to kShare tiles per round, possibly none).
struct Share {
  int64_t tile;
  int beg, n;
};

__device__ __forceinline__ Share share_of(const Walk& w, int wave) {
  const int sh = w.wpt_log2();
  const int lt = wave >> sh, wi = wave & ((1 << sh) - 1);
  int64_t tile = int64_t(w.tg) * w.tp() + lt;
  if (tile >= w.row_tiles) tile = w.row_tiles - 1;  // a pair's missing second tile: valid, never stored
  const int ng = w.g_end - w.g_beg;
  const int beg = w.g_beg + ((wi * ng) >> sh) + w.rd * kShare;
  const int end = w.g_beg + (((wi + 1) * ng) >> sh);
  return Share{tile, beg, min(end - beg, kShare)};
}

// The longest K a GEMV of the chain may have: each workgroup keeps a GEMV's
// whole input in LDS (kMaxK halves per activation row).
constexpr int kMaxK = 32768;

template <int MR>
struct Geo {
  static constexpr int kRows = MR < 4 ? MR : 4;          // accumulators per lane (MFMA D rows used)
  static constexpr int kRedWave = 4 * kRows * 16;        // floats of one wave's partial sums
  static constexpr int kXRow = kMaxK + (MR > 1 ? 32 : 0);  // halves per x row
  static constexpr size_t kCtlBytes = sizeof(LdsCtl);
  static constexpr size_t kPartBytes = size_t(kSlots) * kWaves * kRedWave * 4;
  static constexpr size_t kXBytes = size_t(MR) * kXRow * 2;
  static constexpr size_t kLds = kCtlBytes + kPartBytes + kXBytes;
};

// One round's requests: the weight tiles (16 bytes per lane each), and the
// round's scale and zero words gathered one per lane -- lane 8u + i holds
// the scale word i of tile u (rows 2i, 2i + 1), lane 2u + i its zero word i
// (rows 8i .. 8i + 7) -- handed to the lanes that need them by a cross-lane
// read at use.
struct Buf {
  u32x4 w[kShare];
  uint32_t sw, zw;
};

template <int MR, int NBUF>
__global__ __launch_bounds__(kThreads, 4) void chain_kernel(const Header* __restrict__ plan, uint8_t* __restrict__ ws,
                                                             uint64_t ws_bytes) {
  using GG = Geo<MR>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  LdsCtl* lc = reinterpret_cast<LdsCtl*>(smem);
  float* part = reinterpret_cast<float*>(smem + GG::kCtlBytes);  // [kSlots][waves][kRedWave]
  _Float16* xs = reinterpret_cast<_Float16*>(smem + GG::kCtlBytes + GG::kPartBytes);
  const uint64_t wsa = reinterpret_cast<uint64_t>(ws);
  W4A16_GLOBAL uint32_t* ctl = gptr<uint32_t>(wsa);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = gridDim.x, wg = blockIdx.x;
  if (tid == 0) {
    lc->ready = -1;
    lc->abort = 0;
    for (int s = 0; s < kSlots; ++s) lc->cnt[s] = 0, lc->gen[s] = 0;
    lc->xstaged = lc->xfreed = 0;
  }
  const bool plan_ok = plan->magic == kMagic && plan->M == MR && plan->ws_bytes <= ws_bytes;
  const uint32_t err0 = ld_dev(ctl + kWsError);
  const uint32_t epoch = ld_dev(ctl + kWsEpoch);
  __syncthreads();
  if (!plan_ok) {
    if (tid == 0) st_dev(ctl + kWsError, 2u);
    return;
  }
  if (err0 != 0) return;  // a failed earlier run: the caller clears the workspace first
  const uint32_t tag = epoch % 65535u + 1u;
  const int total = plan->total_items;
  const OpDev* ops = reinterpret_cast<const OpDev*>(plan + 1);

  const int piece = lane >> 4, rlane = lane & 15;
  const int mm = rlane < MR ? rlane : MR - 1;
  const uint32_t magic = dev::kMagic1024;
  Waiter wt{lc, ctl};
  bool& failed = wt.failed;

  // A round's weight tiles, scales and zero words as buffer loads: the row
  // tile's base goes into the (scalar) resource, the group into the scalar
  // offset, and the lane's constant offset is the only vector operand, so
  // no 64-bit addresses occupy vector registers. Indices past the round are
  // clamped to its last tile (in bounds, discarded in compute()). `live`
  // false gives the resources 0 records: the same requests go out and come
  // back as zeros without touching memory, so every path issues the same
  // number of requests and every wait count stays exact.
  const int w_voff = lane * 16;
  const int s_tile = min(lane >> 3, kShare - 1), s_word = lane & 7;  // scale word gathered by this lane
  const int z_tile = min(lane >> 1, kShare - 1), z_word = lane & 1;  // zero word gathered by this lane
  auto load = [&](Buf& b, const OpDev& d, const Share& s, bool live) {
    const uint64_t q0 = uint64_t(s.tile) * uint64_t(d.G);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(d.wq + q0 * kTileBytes), (short)0, live ? d.G * kTileBytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(d.sw + q0 * 32), (short)0, live ? d.G * 32 : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(d.zw + q0 * 8), (short)0, live ? d.G * 8 : 0, 0x00020000);
#pragma unroll
    for (int u = 0; u < kShare; ++u) {
      const int gg = max(s.beg + min(u, s.n - 1), 0);
      b.w[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_voff, gg * kTileBytes, 2 /* nt */);
    }
    const int gs = max(s.beg + min(s_tile, s.n - 1), 0), gz = max(s.beg + min(z_tile, s.n - 1), 0);
    b.sw = __builtin_amdgcn_raw_buffer_load_b32(rsc, gs * 32 + s_word * 4, 0, 0);
    b.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, gz * 8 + z_word * 4, 0, 0);
  };

  // Staging of a GEMV's whole input (all M rows, all K) into the x buffer,
  // the waves taking 64-chunk blocks in turn: this wave's blocks are wave,
  // wave + 8, ... A chunk is 16 bytes: four tagged words (x from a producer:
  // tag checked, fp16 value scaled by 2^-x_shift and rounded to fp16) or
  // eight fp16 values (external x). Requests go out in batches of kBatch
  // chunks per lane; chunks past the end repeat the last one (in bounds;
  // they rewrite the same values). Stale words are requested again with
  // device-scope loads until they carry the launch's tag.
  constexpr int kBatch = 4;
  auto stage_part = [&](const OpDev& d) -> bool {
    const bool tagged = d.x_src >= 0;
    const int per_row = tagged ? d.K / 4 : d.K / 8;  // chunks per activation row
    const int total_chunks = MR * per_row;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        tagged ? reinterpret_cast<void*>(ws + d.xt_off) : reinterpret_cast<void*>(d.x_ext), (short)0, 0x7fffffff,
        0x00020000);
    const float scale = __builtin_ldexpf(1.0f, -d.x_shift);  // exact power of two
    for (int j0 = 0; (j0 * kWaves + wave) * 64 < total_chunks; j0 += kBatch) {
      int m[kBatch], cw[kBatch];
      u32x4 v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int c = min(((j0 + j) * kWaves + wave) * 64 + lane, total_chunks - 1);
        m[j] = MR == 1 ? 0 : c / per_row;
        cw[j] = c - m[j] * per_row;
        const int off = tagged ? (m[j] * d.x_stride + cw[j] * 4) * 4 : (m[j] * d.K + cw[j] * 8) * 2;
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      }
      if (tagged) {
        auto fresh = [&]() {
          bool ok = true;
#pragma unroll
          for (int j = 0; j < kBatch; ++j)
            ok &= (v[j].x >> 16) == tag && (v[j].y >> 16) == tag && (v[j].z >> 16) == tag && (v[j].w >> 16) == tag;
          return __builtin_amdgcn_read_exec() == __ballot(ok);
        };
        if (!fresh()) {
          const uint64_t t0 = wall_clock64();
          do {
            if (!wt.may_wait(t0, true)) return false;
            __builtin_amdgcn_s_sleep(2);
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
              v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, (m[j] * d.x_stride + cw[j] * 4) * 4, 0, 16 /* sc1 */);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the check below reads them all
          } while (!fresh());
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)(dev::half_bits_to_float(v[j].x & 0xFFFFu) * scale));
          const uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)(dev::half_bits_to_float(v[j].y & 0xFFFFu) * scale));
          const uint32_t h2 = __builtin_bit_cast(uint16_t, (_Float16)(dev::half_bits_to_float(v[j].z & 0xFFFFu) * scale));
          const uint32_t h3 = __builtin_bit_cast(uint16_t, (_Float16)(dev::half_bits_to_float(v[j].w & 0xFFFFu) * scale));
          uint2 packed;
          packed.x = h0 | (h1 << 16);
          packed.y = h2 | (h3 << 16);
          *reinterpret_cast<uint2*>(xs + m[j] * GG::kXRow + cw[j] * 4) = packed;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) *reinterpret_cast<u32x4*>(xs + m[j] * GG::kXRow + cw[j] * 8) = v[j];
      }
    }
    return true;
  };

  // A round's products: per tile, four MFMAs over the unpacked weights (x
  // from the LDS buffer as the A operand), the group sum scaled by its fp16
  // scale and added to the accumulators in tile order -- the fp32 operations
  // of the standalone kernels, in the same order, carried across rounds.
  // Tiles past the round (clamped duplicates) are computed and discarded by
  // a select. Every request of the buffer has arrived (the wait for it is
  // exact), so the tiles are left to the compiler's scheduling.
  auto compute = [&](const Buf& b, const Share& s, float (&acc)[GG::kRows]) {
    if (s.n <= 0) return;
    const _Float16* xbase = xs + s.beg * kGroup + 8 * piece;
#pragma unroll
    for (int u = 0; u < kShare; ++u) {
      const u32x4 wt = b.w[u];
      // this lane's scale and zero words of tile u, from the lanes that hold them
      const uint32_t st = uint32_t(__builtin_amdgcn_ds_bpermute((u * 8 + (rlane >> 1)) * 4, int(b.sw)));
      const uint32_t zt = uint32_t(__builtin_amdgcn_ds_bpermute((u * 2 + (rlane >> 3)) * 4, int(b.zw)));
      const dev::ZeroPairs zp = dev::zero_pairs((zt >> ((rlane & 7) * 4)) & 15u);
      const float sc = dev::half_bits_to_float((st >> ((rlane & 1) * 16)) & 0xFFFFu);
      const _Float16* xg = xbase + min(u, s.n - 1) * kGroup;  // clamped tiles read the last tile's x
      f32x4 dd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        dev::half2_t p[4];
        dev::unpack8(wt[kb], magic, zp, p);
        const dev::half8_t bw = {p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
        const dev::half8_t ax = *reinterpret_cast<const dev::half8_t*>(xg + mm * GG::kXRow + 32 * kb);
        dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(ax, bw, dd, 0, 0, 0);
      }
      const bool valid = u < s.n;
#pragma unroll
      for (int r2 = 0; r2 < GG::kRows; ++r2) acc[r2] = valid ? __builtin_fmaf(dd[r2], sc, acc[r2]) : acc[r2];
    }
  };

  // Hands the item's partial sums in through its slot, once the slot's
  // previous item has had its epilogue.
  auto hand_in = [&](int o, const float (&acc)[GG::kRows]) {
    const int slot = o % kSlots, gen = o / kSlots;
    const uint64_t t0 = wall_clock64();
    while (lds_ld(&lc->gen[slot]) != gen) {
      if (!wt.may_wait(t0, false)) return;
      __builtin_amdgcn_s_sleep(1);
    }
    lds_acquire();
    float* pw = part + (size_t(slot) * kWaves + wave) * GG::kRedWave;
#pragma unroll
    for (int r = 0; r < GG::kRows; ++r) pw[(piece * GG::kRows + r) * 16 + rlane] = acc[r];
    lds_release();
    if (lane == 0) __hip_atomic_fetch_add(&lc->cnt[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  // The epilogue of item ordinal o (GEMV op, tile group tg), once every wave
  // has handed the item in: adds the waves' partial sums in wave order and
  // stores the outputs (fp16, SwiGLU, or the split-K fixed-point atomics),
  // then frees the slot.
  auto epilogue = [&](int o, int op, int tg) {
    const int slot = o % kSlots;
    if (!wt.wait_lds(&lc->cnt[slot], kWaves)) return;
    const OpDev& d = ops[op];
    const float* pb = part + size_t(slot) * kWaves * GG::kRedWave;
    W4A16_GLOBAL uint32_t* yt = gptr<uint32_t>(wsa + d.yt_off);
    W4A16_GLOBAL uint16_t* yd = gptr<uint16_t>(d.y);
    // A GEMV tile has 16 outputs per activation row; a SwiGLU tile 8, the
    // gate sums of its rows 0-7 and the up sums of rows 8-15.
    const bool pair = d.kind == W4A16_CHAIN_SWIGLU;
    const int per_tile = pair ? MR * 8 : MR * 16;
    const int n_out = d.tp * per_tile;
    for (int idx = lane; idx < ((n_out + 63) & ~63); idx += 64) {
      const int id = idx < n_out ? idx : n_out - 1;
      const int lt = id / per_tile, rem = id - lt * per_tile;
      const int m = pair ? rem >> 3 : rem >> 4, r = pair ? rem & 7 : rem & 15;
      const int sl = ((m >> 2) * GG::kRows + (m & 3)) * 16 + r;
      const int w0 = lt * d.wpt;
      float sum = pb[w0 * GG::kRedWave + sl];
      for (int w2 = 1; w2 < d.wpt; ++w2) sum += pb[(w0 + w2) * GG::kRedWave + sl];
      if (pair) {
        float up = pb[w0 * GG::kRedWave + sl + 8];
        for (int w2 = 1; w2 < d.wpt; ++w2) up += pb[(w0 + w2) * GG::kRedWave + sl + 8];
        sum = sum / (1.f + expf(-sum)) * up;  // silu(gate) * up, rounded to fp32 (as in w4a16_gemv_swiglu)
        asm volatile("" : "+v"(sum));
      }
      const int64_t t = int64_t(tg) * d.tp + lt;
      const int64_t n = t * (pair ? 8 : kTileRows) + r;
      if (idx < n_out && t < d.row_tiles && n < d.N) {
        const int64_t oi = int64_t(m) * d.N + n;
        bool write = true;
        _Float16 v;
        if (d.splits > 1) {
          W4A16_GLOBAL unsigned long long* word = gptr<unsigned long long>(wsa + d.acc_off) + oi;
          const unsigned long long add = dev::splitk_addend(sum);
          const unsigned long long now =
              __hip_atomic_fetch_add(word, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
          write = dev::splitk_count(now) == unsigned(d.splits);
          v = dev::splitk_value(now, d.splits);
          if (write) __hip_atomic_store(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          v = (_Float16)sum;
        }
        if (write) {
          const uint16_t bits = __builtin_bit_cast(uint16_t, v);
          yd[oi] = bits;
          if (d.yt_off) st_dev(yt + oi, (tag << 16) | bits);
        }
      }
    }
    // the partial sums have been read: the slot is free for its next use
    lds_st(&lc->cnt[slot], 0);
    lds_release();
    lds_st(&lc->gen[slot], o / kSlots + 1);
  };

  // Wave 0 waits until the producer's sentinel word carries the launch's tag
  // and publishes that in LDS; the other waves wait for the LDS word.
  auto wait_ready = [&](const OpDev& d, int op) -> bool {
    if (wave != 0) return wt.wait_lds(&lc->ready, op);
    const W4A16_GLOBAL uint32_t* sent = gptr<uint32_t>(wsa + d.xt_off) + d.sentinel;
    const uint64_t t0 = wall_clock64();
    while ((ld_dev(sent) >> 16) != tag) {
      if (!wt.may_wait(t0, true)) return false;
      __builtin_amdgcn_s_sleep(1);
    }
    lds_st(&lc->ready, op);
    return true;
  };

  // The input of the GEMV at walk position wc: once every wave is done with
  // the previous GEMV's x buffer and the producer has been seen finishing,
  // the waves stage it into the x buffer. Meanwhile the weights of the
  // GEMV's first round are in flight (requested a round ago).
  int cur_op = -1, nchg = 0, o = 0;
  Walk wc, wp;
  wc.k = wg, wc.op = 0;
  if (wg < total) walk_enter(wc, ops);
  wp = wc;
  auto enter_gemv = [&]() -> bool {
    const OpDev& d = ops[wc.op];
    if (cur_op >= 0) {  // done with the previous GEMV's input
      lds_release();
      if (lane == 0) __hip_atomic_fetch_add(&lc->xfreed, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (!wt.wait_lds(&lc->xfreed, kWaves * nchg)) return false;  // every wave done with it
    if (d.x_src >= 0 && !wait_ready(d, wc.op)) return false;
    if (!stage_part(d)) return false;
    lds_release();
    if (lane == 0) __hip_atomic_fetch_add(&lc->xstaged, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (!wt.wait_lds(&lc->xstaged, kWaves * (nchg + 1))) return false;  // every part staged
    cur_op = wc.op;
    ++nchg;
    return true;
  };

  // One round: the round at walk position wc with weights in `cur`; the
  // weights of the round NBUF - 1 rounds on (walk wp) go into `nxt` first
  // (one request site, so their registers have a single definition and are
  // never copied), and stay in flight while this round computes and hands
  // in. The staging of a GEMV's input happens outside the round, so that
  // the wait for the round's weights is exact: it never waits for the next
  // round's.
  float acc[GG::kRows];
#pragma unroll
  for (int r = 0; r < GG::kRows; ++r) acc[r] = 0.f;
  bool pend = false;         // the previous item's epilogue is still owed
  int pend_op = 0, pend_tg = 0;
  auto step = [&](const Buf& cur, Buf& nxt) {
    const Share s = share_of(wc, wave);
    {
      const bool valid = wp.k < total;
      const Share sp = valid ? share_of(wp, wave) : s;
      load(nxt, ops[valid ? wp.op : wc.op], sp, valid && sp.n > 0);
      walk_advance(wp, ops, P, total);
    }
    compute(cur, s, acc);
    if (wc.rd == wc.rounds() - 1) {
      hand_in(o, acc);
      if (failed) return;
      // Epilogues rotate over the waves: wave o % 8 does item o's, one item
      // later (when every wave has most likely handed it in), or at once
      // for the workgroup's last item of a GEMV, whose consumers wait for it.
      if (pend && wave == ((o - 1) & (kWaves - 1))) epilogue(o - 1, pend_op, pend_tg);
      pend = wc.k + P < wc.end;
      if (!pend && wave == (o & (kWaves - 1))) epilogue(o, wc.op, wc.tg);
      pend_op = wc.op, pend_tg = wc.tg;
      ++o;
#pragma unroll
      for (int r = 0; r < GG::kRows; ++r) acc[r] = 0.f;
    }
    walk_advance(wc, ops, P, total);
  };

  Buf bufs[NBUF];
#pragma unroll
  for (int i = 0; i + 1 < NBUF; ++i) {
    if (wp.k < total) {
      const Share sp = share_of(wp, wave);
      load(bufs[i], ops[wp.op], sp, sp.n > 0);
    }
    walk_advance(wp, ops, P, total);
  }
  bool more = true;
  while (more) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (!more || failed || wc.k >= total || (wc.op != cur_op && !enter_gemv())) {
        more = false;
        break;
      }
      step(bufs[j], bufs[(j + NBUF - 1) % NBUF]);
    }
  }

  // Every wave is past its last item (or has left on an error): the last
  // workgroup to get here advances the launch number.
  __syncthreads();
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(ctl + kWsFinished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == uint32_t(P) - 1) {
      __hip_atomic_store(ctl + kWsFinished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(ctl + kWsEpoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------------ host side

constexpr size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

template <int MR, int NBUF>
hipError_t launch_typed(const void* plan, void* ws, size_t ws_bytes, hipStream_t stream, int grid) {
  constexpr size_t lds = Geo<MR>::kLds;
  static std::atomic<uint64_t> raised{0};
  if (lds > kDefaultLdsLimit) {
    const hipError_t e = dev::raise_lds_limit(reinterpret_cast<const void*>(&chain_kernel<MR, NBUF>), lds, raised);
    if (e != hipSuccess) return e;
  }
  return dev::launch_kernel(&chain_kernel<MR, NBUF>, dim3(unsigned(grid)), dim3(kThreads), lds, stream,
                            static_cast<const Header*>(plan), static_cast<uint8_t*>(ws), uint64_t(ws_bytes));
}

// Workgroups of one launch: as many per compute unit as can be resident at
// once (at most 2; 0 if none can).
template <int MR, int NBUF>
int resident_grid() {
  int device = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&device) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  constexpr size_t lds = Geo<MR>::kLds;
  static std::atomic<uint64_t> raised{0};
  if (lds > kDefaultLdsLimit &&
      dev::raise_lds_limit(reinterpret_cast<const void*>(&chain_kernel<MR, NBUF>), lds, raised) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&chain_kernel<MR, NBUF>),
                                                   kThreads, lds) != hipSuccess)
    return 0;
  return min(per_cu, 2) * cus;
}

}  // namespace chain
}  // namespace w4a16

using w4a16::chain::Header;
using w4a16::chain::OpDev;

namespace {

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Waves per tile, tiles per item and rounds per item for one GEMV: 4 waves
// per 16-row tile (two tiles per item) while each wave's share of the K
// range fits one round of 7 tiles (5 with split K, as the standalone split-K
// plan), else 8 waves per tile (one tile per item), each taking its share
// in rounds of at most 7 tiles. (8 waves per tile for the narrow GEMVs of a
// 7B step -- shorter shares, more items -- measured slower: 1329 against
// 1246 us per step.) A SwiGLU matrix (gate rows 0-7 and up rows 8-15 of
// each tile, 8 outputs per tile) takes the same geometry.
void chain_geometry(int G, int splits, int* wpt, int* tp, int* rounds) {
  constexpr int share = w4a16::chain::kShare;
  const int range = (G + splits - 1) / splits;
  const int cap4 = splits > 1 ? 5 : share;
  if ((range + 3) / 4 <= cap4) {
    *wpt = 4, *tp = 2, *rounds = 1;
  } else {
    *wpt = 8, *tp = 1;
    *rounds = ((range + 7) / 8 + share - 1) / share;
  }
}

}  // namespace

extern "C" int w4a16_chain_plan(int M, int n_ops, const w4a16_chain_op* ops, void* plan, size_t plan_bytes,
                                size_t* plan_bytes_needed, size_t* ws_bytes_needed) {
  using namespace w4a16::chain;
  if (M < 1 || n_ops < 1 || !ops) return W4A16_EINVAL;
  if (M > W4A16_MAX_M) return W4A16_EUNSUPPORTED;
  const size_t need_plan = sizeof(Header) + size_t(n_ops) * sizeof(OpDev);
  size_t ws = kWsHeader;
  int64_t total = 0;
  // First pass: check every GEMV and size the workspace.
  for (int j = 0; j < n_ops; ++j) {
    const w4a16_chain_op& o = ops[j];
    if (o.kind != W4A16_CHAIN_GEMV && o.kind != W4A16_CHAIN_SWIGLU) return W4A16_EINVAL;
    if (o.N < 1 || o.K < W4A16_GROUP || o.K % W4A16_GROUP != 0) return W4A16_EINVAL;
    const int G = o.K / W4A16_GROUP;
    if (o.splits < 1 || o.splits > G || o.splits > w4a16::kMaxSplits) return W4A16_EINVAL;
    if (o.kind == W4A16_CHAIN_SWIGLU && o.splits != 1) return W4A16_EINVAL;
    if (o.K > kMaxK) return W4A16_EUNSUPPORTED;  // a workgroup keeps the whole input in LDS
    if (!aligned16(o.wq) || !aligned16(o.scales) || !aligned16(o.zeros) || !aligned16(o.y)) return W4A16_EINVAL;
    if (o.x_src < -1 || o.x_src >= j) return W4A16_EINVAL;
    if (o.x_src < 0 && !aligned16(o.x)) return W4A16_EINVAL;
    if (o.x_src >= 0 && (ops[o.x_src].N < o.K || o.x_shift < 0 || o.x_shift > 24)) return W4A16_EINVAL;
    const int64_t row_tiles = o.kind == W4A16_CHAIN_SWIGLU ? (int64_t(o.N) + 7) / 8 : (int64_t(o.N) + 15) / 16;
    int wpt, tp, rounds;
    chain_geometry(G, o.splits, &wpt, &tp, &rounds);
    const int64_t items = (row_tiles + tp - 1) / tp * o.splits;
    total += items;
    if (total >= (int64_t(1) << 30) || row_tiles >= (int64_t(1) << 26)) return W4A16_EUNSUPPORTED;
    if (o.splits > 1) ws = align_up(ws, 256) + align_up(size_t(8) * M * o.N, 256);
  }
  std::vector<char> consumed(size_t(n_ops), 0);
  for (int j = 0; j < n_ops; ++j)
    if (ops[j].x_src >= 0) consumed[size_t(ops[j].x_src)] = 1;
  for (int j = 0; j < n_ops; ++j)
    if (consumed[size_t(j)]) ws = align_up(ws, 256) + align_up(size_t(4) * M * ops[j].N, 256);
  if (plan_bytes_needed) *plan_bytes_needed = need_plan;
  if (ws_bytes_needed) *ws_bytes_needed = ws;
  if (!plan) return W4A16_OK;
  if (plan_bytes < need_plan) return W4A16_EINVAL;
  // Second pass: the descriptors.
  Header h;
  std::memset(&h, 0, sizeof(h));
  h.magic = kMagic;
  h.M = M;
  h.n_ops = n_ops;
  h.total_items = int32_t(total);
  h.plan_bytes = need_plan;
  h.ws_bytes = ws;
  std::vector<OpDev> d(static_cast<size_t>(n_ops));
  std::memset(d.data(), 0, d.size() * sizeof(OpDev));
  size_t off = kWsHeader;
  std::vector<uint64_t> yt_off(size_t(n_ops), 0);
  int begin = 0;
  for (int j = 0; j < n_ops; ++j) {
    const w4a16_chain_op& o = ops[j];
    OpDev& e = d[size_t(j)];
    e.wq = reinterpret_cast<uintptr_t>(o.wq);
    e.sw = reinterpret_cast<uintptr_t>(o.scales);
    e.zw = reinterpret_cast<uintptr_t>(o.zeros);
    e.x_ext = o.x_src < 0 ? reinterpret_cast<uintptr_t>(o.x) : 0;
    e.y = reinterpret_cast<uintptr_t>(o.y);
    e.N = o.N;
    e.K = o.K;
    e.G = o.K / W4A16_GROUP;
    e.kind = o.kind;
    e.splits = o.splits;
    e.row_tiles = int32_t(o.kind == W4A16_CHAIN_SWIGLU ? (int64_t(o.N) + 7) / 8 : (int64_t(o.N) + 15) / 16);
    chain_geometry(e.G, o.splits, &e.wpt, &e.tp, &e.rounds);
    e.per_split = (e.row_tiles + e.tp - 1) / e.tp;
    e.items = e.per_split * o.splits;
    e.item_begin = begin;
    begin += e.items;
    e.x_src = o.x_src;
    e.x_shift = o.x_src >= 0 ? o.x_shift : 0;
    e.split_q = e.G / o.splits;
    if (o.splits > 1) {
      off = align_up(off, 256);
      e.acc_off = off;
      off += align_up(size_t(8) * M * o.N, 256);
    }
  }
  for (int j = 0; j < n_ops; ++j) {
    if (!consumed[size_t(j)]) continue;
    off = align_up(off, 256);
    yt_off[size_t(j)] = off;
    d[size_t(j)].yt_off = off;
    off += align_up(size_t(4) * M * ops[j].N, 256);
  }
  for (int j = 0; j < n_ops; ++j) {
    OpDev& e = d[size_t(j)];
    if (e.x_src < 0) continue;
    const int p = e.x_src;
    e.xt_off = yt_off[size_t(p)];
    e.x_stride = ops[p].N;
    e.sentinel = int32_t((M - 1) * ops[p].N + ops[p].N - 1);
  }
  std::memcpy(plan, &h, sizeof(h));
  std::memcpy(static_cast<char*>(plan) + sizeof(h), d.data(), d.size() * sizeof(OpDev));
  return W4A16_OK;
}

extern "C" int w4a16_chain_run(int M, const void* plan_dev, void* workspace, size_t ws_bytes, void* stream) {
  using namespace w4a16::chain;
  if (M < 1 || !aligned16(plan_dev) || !aligned16(workspace) || ws_bytes < kWsHeader) return W4A16_EINVAL;
  if (M > W4A16_MAX_M) return W4A16_EUNSUPPORTED;
  if (M != 1) return W4A16_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int grid = resident_grid<1, 2>();
  if (grid <= 0) return W4A16_EUNSUPPORTED;
  if (launch_typed<1, 2>(plan_dev, workspace, ws_bytes, s, grid) != hipSuccess) return W4A16_EHIP;
  return W4A16_OK;
}

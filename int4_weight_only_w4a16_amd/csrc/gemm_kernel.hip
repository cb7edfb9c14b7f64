// W4A16 GEMM for many activation rows (prefill-sized M), on the matrix
// cores: y[M][N] = x[M][K] W^T with W in layout ID 2, dequantized in
// registers. A 256-thread workgroup computes a 128 (m) x 128 (n) tile of y
// as four 128 x 32 wave tiles side by side in n, each 8 x 2 blocks of
// v_mfma_f32_16x16x32_f16 with fp32 accumulators, over K one 128-column
// group at a time. Every weight tile is dequantized once per workgroup, and
// each dequantized fragment feeds eight MFMAs: about two VALU instructions
// per MFMA, where a VALU:MFMA ratio of 4 alone caps gfx950 at about 60% of
// its MFMA rate (measured). Every wave reads all 128 rows of x from LDS,
// about 160 bytes per clock per CU at full MFMA rate, within the 256 the
// LDS delivers (also measured). For M <= 64 the tile has 16, 32 or 64 rows
// instead (MB = 1, 2 or 4 m blocks per wave): there the matrix cores are
// not the limit, and a 128-row tile would mostly multiply padding.
//  - x[m0 .. m0+16 MB-1][group] is staged in LDS by direct global-to-LDS loads
//    (double-buffered, 16-byte slots XOR-swizzled by row against bank
//    conflicts) and read as the A operand;
//  - each wave streams its two weight tiles (16 rows x 128 columns, 1 KiB
//    each; a lane's 16 bytes are exactly its B operand for the four 32-column
//    blocks) and dequantizes them to fp16 (q - z) * s, rounded once to
//    nearest even -- the values w4a16_dequant_f16 writes;
//  - the next group's requests go out before the current group is
//    multiplied: x into the other LDS buffer, the weights into the other of
//    two register buffers. (Weights two groups ahead, which needs x staged
//    through registers, measured 10% slower: the multiply is not waiting
//    on memory as much as on issue.)
#include <algorithm>

#include "w4a16_device.h"

namespace w4a16 {
namespace dev {

constexpr int kGemmBN = 128;                // weight rows per workgroup (8 row tiles)
constexpr int kGemmNB = 2;                  // 16-row weight tiles per wave (the 4 waves side by side in n)
constexpr int kOStride = kGemmBN + 8;       // halves per LDS row of the output tile (epilogue)
// A workgroup covers 16 MB activation rows (MB = 8, 4, 2 or 1 m blocks per
// wave): two staged x groups of 16 MB x 128 halves.
constexpr size_t gemm_lds_bytes(int mb) { return size_t(2) * 16 * mb * kGroup * 2; }
static_assert(size_t(16) * kOStride * 2 <= gemm_lds_bytes(1), "output tile must fit the x buffers");

// Split-K (splits > 1): workgroup (.., .., z) multiplies only the z-th of
// `splits` contiguous group ranges. With ws non-null it adds its fp32
// partial sums to ws, one uint64 word per output, in the fixed-point format
// of splitk_addend(); the add that completes an output's count writes y and
// zeroes the word (exact and order-free, as in the split-K GEMV). With part
// non-null instead it stores them, plain fp32, to part[z][M][N], and
// splitk_sum_kernel adds the splits afterwards in split order (the
// two-stage partial-then-final reduction): no atomics, whose cost grows with
// M * N * splits (a third of the launch for 4608 x 3584 at M = 64).
template <int MB>
__global__ __launch_bounds__(256, 2) void gemm_kernel(int M, int N, int K, int splits,
                                                   const uint8_t* __restrict__ wq,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros,
                                                   const _Float16* __restrict__ x, _Float16* __restrict__ y,
                                                   unsigned long long* __restrict__ ws, float* __restrict__ part) {
  constexpr int kBM = 16 * MB;           // activation rows per workgroup
  constexpr int kXTile = kBM * kGroup;   // halves of one staged x group
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  _Float16* xs = reinterpret_cast<_Float16*>(smem);  // [2][kBM][128], 16-byte slots swizzled
  const int G = K / kGroup;
  const int64_t NT = (int64_t(N) + kTileRows - 1) / kTileRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rlane = lane & 15, piece = lane >> 4;
  // Which output tile: consecutive workgroups go round-robin to the 8 XCDs,
  // each with its own L2. With blockIdx.x (m) fastest, every XCD's resident
  // workgroups hold 2 of 16 m blocks and so fetch every weight strip. Where
  // the tile count T of a split is a multiple of 8 and the m blocks one of 4,
  // XCD j (= linear id mod 8) takes instead the j-th eighth of a band order:
  // bands of 4 m blocks, n outside, m inside. Its resident workgroups then
  // cover 4 m blocks by 16 strips, and fewer L2s fetch each strip (4 of 8
  // at 16 m blocks; gate+up 37888x3584 2-7% faster at M = 512..2048).
  // Either order is a bijection of the grid, and each tile's arithmetic is
  // the same.
  int bm = int(blockIdx.x), bn = int(blockIdx.y);
  {
    const unsigned X = gridDim.x, Y = gridDim.y, T = X * Y;
    if ((T & 7) == 0 && (X & 3) == 0) {
      const unsigned b = blockIdx.x + X * blockIdx.y;
      const unsigned t = (b & 7) * (T >> 3) + (b >> 3);
      const unsigned band = t / (4 * Y), r = t - band * (4 * Y);
      bn = int(r >> 2);
      bm = int(band * 4 + (r & 3));
    }
  }
  const int64_t m0 = int64_t(bm) * kBM;
  // This workgroup's groups [g_beg, g_beg + ng) (all of K unsplit; a 32-bit
  // division otherwise, split * G < 31 * 2^24).
  const int g_beg = splits == 1 ? 0 : int(unsigned(blockIdx.z) * unsigned(G) / unsigned(splits));
  const int ng = (splits == 1 ? G : int(unsigned(blockIdx.z + 1) * unsigned(G) / unsigned(splits))) - g_beg;
  const int64_t tw = int64_t(bn) * (kGemmBN / kTileRows) + wave * kGemmNB;  // wave's first row tile

  // The wave's row tiles (clamped past the end: valid memory, never
  // stored). Their bases are wave-uniform, and a lane's part of each
  // request is one 32-bit offset for every tile and group, so requests take
  // a scalar base and a single offset register.
  const uint8_t* wbase[kGemmNB];
  const uint32_t* sbase[kGemmNB];
  const uint32_t* zbase[kGemmNB];
#pragma unroll
  for (int j = 0; j < kGemmNB; ++j) {
    const int64_t t = tw + j < NT ? tw + j : NT - 1;
    const int64_t q0 = t * G;
    wbase[j] = wq + q0 * kTileBytes;
    sbase[j] = reinterpret_cast<const uint32_t*>(scales) + q0 * (kTileRows / 2);
    zbase[j] = reinterpret_cast<const uint32_t*>(zeros) + q0 * (kTileRows / 8);
  }
  const uint32_t w_off = uint32_t(lane) * 16, s_off = uint32_t(rlane >> 1), z_off = uint32_t(rlane >> 3);
  // x[m0 .. m0+kBM-1][group g] -> LDS buffer buf, straight from global memory
  // (global_load_lds_dwordx4: lane l of a wave's request writes 16 bytes at
  // the request's LDS base + 16 l, so a request fills 1 KiB). Row r of the
  // tile keeps its 16 sixteen-byte chunks c in slots c ^ (r % 16): the A
  // operand reads of 16 consecutive rows then hit 16 distinct bank groups.
  // Rows past M read row M - 1 (valid memory, never stored). x_off[i] is
  // the element offset of request i's chunk from x[m0][0], below 128 K,
  // which the host keeps under 2^32. The 16 kBM slots take 4 MB requests,
  // MB per wave.
  uint32_t x_off[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int req = wave * MB + i;  // this wave's request i: slots 64 req .. 64 req + 63
    const int p = req * 64 + lane, row = p >> 4, c = (p & 15) ^ (row & 15);
    const int64_t mr = m0 + row < M ? row : M - 1 - m0;
    x_off[i] = uint32_t(mr * K + c * 8);
  }
  auto load_x = [&](int g, int buf) {
    const _Float16* xg = x + m0 * K + int64_t(g) * kGroup;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int req = wave * MB + i;
      load_lds16(xg + x_off[i], xs + buf * kXTile + req * 512);
    }
  };
  struct W {
    u32x4 w[kGemmNB];
    uint32_t s[kGemmNB], z[kGemmNB];
  };
  auto load_w = [&](int g, W& r) {
#pragma unroll
    for (int j = 0; j < kGemmNB; ++j) {
      r.w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wbase[j] + int64_t(g) * kTileBytes + w_off));
      r.s[j] = sbase[j][g * (kTileRows / 2) + s_off];
      r.z[j] = zbase[j][g * (kTileRows / 8) + z_off];
    }
  };

  f32x4 acc[MB][kGemmNB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < kGemmNB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t magic = kMagic1024;
  // Multiply group g: x from LDS buffer buf, the wave's weight tiles from
  // `cur`.
  auto compute = [&](int buf, const W& cur) {
    // Per tile: the fp16 scale pair and the zero-point pairs of row rlane.
    half2_t s2[kGemmNB];
    ZeroPairs zp[kGemmNB];
#pragma unroll
    for (int j = 0; j < kGemmNB; ++j) {
      const uint16_t sb = uint16_t((cur.s[j] >> ((rlane & 1) * 16)) & 0xFFFFu);
      s2[j] = as_h2(uint32_t(sb) * 0x00010001u);
      zp[j] = zero_pairs((cur.z[j] >> ((rlane & 7) * 4)) & 15u);
    }
    const _Float16* xa = xs + buf * kXTile + rlane * kGroup;  // row rlane of each 16-row block
    auto read_a = [&](int kb, int mb) {  // A fragment: rows mb*16.. of 32-column block kb
      return *reinterpret_cast<const half8_t*>(xa + mb * 16 * kGroup + ((kb * 4 + piece) ^ rlane) * 8);
    };
    auto dequant = [&](int kb, half8_t (&bw)[kGemmNB]) {  // B fragments of 32-column block kb
#pragma unroll
      for (int j = 0; j < kGemmNB; ++j) {
        half2_t p[4];
        unpack8(cur.w[j][kb], magic, zp[j], p);
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = p[i] * s2[j];  // (q - z) * s, rounded once
        bw[j] = half8_t{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
      }
    };
    if constexpr (MB == 8) {
      // 128-row tile: software-pipelined by one 32-column block. An A
      // fragment's next read (block kb + 1) is issued right after its two
      // MFMAs of block kb, into the same registers, and block kb + 1's
      // weights are dequantized while block kb multiplies; the group
      // barriers below fix the order MFMA, VALU, MFMA, LDS read, VALU. Each
      // read then has some 14 MFMAs (about 220 cycles) before its use, and
      // the loop waits on LDS once per block instead of ahead of almost
      // every MFMA (the compiler's own interleave). Every accumulator sees
      // the same MFMAs in the same order, so the sums are bit-identical;
      // 2-4% faster at M = 512 and 2048 on the 7B shapes. With 16-64 rows
      // the same schedule measured up to 27% slower, so those tiles keep
      // the compiler's interleave.
      half8_t af[MB], bw[2][kGemmNB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = read_a(0, mb);
      dequant(0, bw[0]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb + 1 < 4) dequant(kb + 1, bw[(kb + 1) & 1]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
          for (int nb = 0; nb < kGemmNB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bw[kb & 1][nb], acc[mb][nb], 0, 0, 0);
          if (kb + 1 < 4) af[mb] = read_a(kb + 1, mb);
        }
      }
      // Schedule of this block (mask 0x100 LDS read, 0x002 VALU, 0x008 MFMA).
      __builtin_amdgcn_sched_group_barrier(0x100, MB, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 30, 0);
#pragma unroll
      for (int i = 0; i < MB * kGemmNB * 4 / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    } else {
      // The compiler's single-wave MFMA interleave (LDS reads and VALU
      // slotted between the MFMAs): 2.5-9% faster than its default schedule
      // on the 7B shapes; raising wave priority around the MFMAs or
      // dequantizing the whole group before the first MFMA did nothing
      // measurable.
      __builtin_amdgcn_iglp_opt(1);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        half8_t bw[kGemmNB];
        dequant(kb, bw);
        half8_t af[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[mb] = read_a(kb, mb);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < kGemmNB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bw[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  };

  if constexpr (MB <= 4) {
    // Register pipeline (tiles of 16-64 rows): each workgroup streams a
    // whole strip of weights, so the requests in flight, not the products,
    // set the pace. x of a group is MB 16-byte loads per lane here, so both
    // x and the weights go through registers, kDepth groups ahead (two for
    // the 64-row tile, which then keeps three waves per SIMD; four for the
    // others; a sweep of 2-8 put these first): step i writes group i's x (requested kDepth steps earlier) into
    // LDS buffer i & 1 (last read by step i - 2, which every wave finished
    // before the previous step's barrier), requests group i + kDepth's x
    // into the registers just written out, meets the others at an LDS-only
    // barrier, multiplies, and requests group i + kDepth's weights into the
    // registers it multiplied. Ordinary loads retire in order, so each wait
    // is an exact count that leaves the later groups' requests in flight.
    // The LDS slots and their swizzle are those of load_x. Past the last
    // group the requests repeat it (in bounds, unused).
    constexpr int kDepth = MB == 4 ? 2 : 4;
    struct XR {
      u32x4 v[MB];
    };
    auto load_xr = [&](int g, XR& r) {
      const _Float16* xg = x + m0 * K + int64_t(g) * kGroup;
#pragma unroll
      for (int j = 0; j < MB; ++j) r.v[j] = *reinterpret_cast<const u32x4*>(xg + x_off[j]);
    };
    auto group = [&](int i) { return g_beg + (i < ng ? i : ng - 1); };
    XR xr[kDepth];
    W wr[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      load_xr(group(d), xr[d]);
      load_w(group(d), wr[d]);
    }
    auto step = [&](int i, XR& xc, W& wc) {  // step i multiplies group g_beg + i
#pragma unroll
      for (int j = 0; j < MB; ++j)
        *reinterpret_cast<u32x4*>(xs + (i & 1) * kXTile + (wave * MB + j) * 512 + lane * 8) = xc.v[j];
      __builtin_amdgcn_sched_barrier(0);
      load_xr(group(i + kDepth), xc);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      compute(i & 1, wc);
      __builtin_amdgcn_sched_barrier(0);
      load_w(group(i + kDepth), wc);
      __builtin_amdgcn_sched_barrier(0);
    };
    int i = 0;
    for (; i + kDepth <= ng; i += kDepth) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) step(i + d, xr[d], wr[d]);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (i + d < ng) step(i + d, xr[d], wr[d]);  // ng is the same for the whole workgroup
    lds_barrier();  // the LDS epilogue below reuses the x buffers
  } else {
    // One step per group: request the next group's x (into the other LDS
    // buffer, last read before the previous barrier) and weights (the last
    // step re-requests the last group: in bounds, unused), multiply this
    // group, wait for the x requests only, and meet at an LDS-only barrier.
    // The requests are unconditional and the two weight buffers alternate
    // statically (the loop is unrolled by two), so the only wait before the
    // multiply is for the weights requested one step earlier; a branch around
    // the requests or a register copy between the buffers let the compiler
    // wait for all of them, and __syncthreads() would wait for every
    // outstanding load too.
    W wa, wb;
    auto step = [&](int i, const W& cur, W& nxt) {  // step i multiplies group g_beg + i
      const int gn = g_beg + (i + 1 < ng ? i + 1 : ng - 1);
      load_x(gn, (i & 1) ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      load_w(gn, nxt);
      __builtin_amdgcn_sched_barrier(0);
      compute(i & 1, cur);
      // The x requests are global-to-LDS requests, which need not complete in
      // order with the weight loads issued after them (see load_lds16), so the
      // only wait that guarantees the next x buffer is complete before the
      // barrier is a full one. It also waits for the weights requested this
      // step, which the next step needs first anyway.
      __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
      lds_barrier();
    };
    load_x(g_beg, 0);
    load_w(g_beg, wa);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    lds_barrier();
    int i = 0;
    for (; i + 1 < ng; i += 2) {
      step(i, wa, wb);
      step(i + 1, wb, wa);
    }
    if (i < ng) step(i, wa, wb);
  }

  if (part) {
    // This split's partial sums, plain fp32 stores: a wave instruction
    // writes 64-byte runs of four rows.
    float* pz = part + int64_t(blockIdx.z) * M * N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < kGemmNB; ++nb) {
        const int64_t n = (tw + nb) * kTileRows + rlane;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + mb * 16 + piece * 4 + r;
          if (m < M && n < N && tw + nb < NT) pz[m * N + n] = acc[mb][nb][r];
        }
      }
    return;
  }

  if (ws) {
    // Split-K: one relaxed device-scope atomic add per output. A lane's adds
    // go out 16 at a time (two row blocks) before their results are
    // examined: checking each result before the next add made the epilogue
    // 64 round trips long, and holding all 64 results spills. The adds are
    // unconditional within a batch (a branch around each made the compiler
    // serialize them again). Row blocks holding no row below M are skipped
    // (a workgroup-uniform test); a position past M or N adds 0 to a valid
    // word, which changes neither its value nor its count and is never
    // examined. Past M the target is row m0 + ((m - m0) mod p), p the
    // largest power of two not above the tile's valid rows, which spreads
    // those adds over the valid rows (zero adds all aimed at one word
    // serialized the whole epilogue; all aimed at row M - 1 cost 40% at
    // M = 16). Adds whose results are not read, with one count per tile and
    // the tile's last workgroup finishing it, measured 5-10% slower from
    // M = 64 on: that workgroup's pass over the tile is serial.
    constexpr int kChunk = MB < 2 ? MB : 2;  // row blocks per batch of adds
    const int m_left = int(M - m0 < kBM ? M - m0 : kBM);  // rows of this tile below M (>= 1)
    const int m_pow2 = 1 << (31 - __builtin_clz(unsigned(m_left)));
#pragma unroll
    for (int mb0 = 0; mb0 < MB; mb0 += kChunk) {
      if (mb0 * 16 >= m_left) break;
      unsigned long long now[kChunk][kGemmNB][4];
      bool valid[kChunk][kGemmNB][4];
#pragma unroll
      for (int dm = 0; dm < kChunk; ++dm)
#pragma unroll
        for (int nb = 0; nb < kGemmNB; ++nb) {
          const int64_t t = tw + nb;
          const int64_t n = t * kTileRows + rlane;
          const int64_t nc = n < N ? n : N - 1;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + (mb0 + dm) * 16 + piece * 4 + r;
            const int64_t mc = m < M ? m : m0 + ((m - m0) & (m_pow2 - 1));
            const bool ok = t < NT && n < N && m < M;
            const unsigned long long add = ok ? splitk_addend(acc[mb0 + dm][nb][r]) : 0ull;
            valid[dm][nb][r] = ok;
            now[dm][nb][r] =
                __hip_atomic_fetch_add(ws + mc * N + nc, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + add;
          }
        }
#pragma unroll
      for (int dm = 0; dm < kChunk; ++dm)
#pragma unroll
        for (int nb = 0; nb < kGemmNB; ++nb) {
          const int64_t n = (tw + nb) * kTileRows + rlane;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (valid[dm][nb][r] && splitk_count(now[dm][nb][r]) == unsigned(splits)) {
              const int64_t m = m0 + (mb0 + dm) * 16 + piece * 4 + r;
              y[m * N + n] = splitk_value(now[dm][nb][r], splits);
              // Every split has added: nothing else touches the word in this call.
              __hip_atomic_store(ws + m * N + n, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
    }
    return;
  }

  // Epilogue through LDS (free after the last barrier): the tile's fp16
  // values go to a [128][136] array (rows padded so the four 16-lane
  // pieces of a write hit distinct banks), then every thread stores whole
  // 16-byte runs along n. Stored straight from the MFMA layout, each
  // instruction would write 32-byte pieces of four rows: a quarter of each
  // cache line, which cost up to 15% of the kernel when y is not already
  // in cache.
  _Float16* ot = xs;
  // D layout: lane l holds D[4 * (l / 16) + r][l % 16] of each 16 x 16 block.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < kGemmNB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ot[(mb * 16 + piece * 4 + r) * kOStride + wave * (kGemmNB * 16) + nb * 16 + rlane] = (_Float16)acc[mb][nb][r];
  lds_barrier();
  const int64_t n_wg = int64_t(bn) * kGemmBN;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int c = tid + 256 * i, row = c >> 4, col = (c & 15) * 8;
    const int64_t m = m0 + row, n0 = n_wg + col;
    if (m >= M || n0 >= N) continue;
    const _Float16* src = ot + row * kOStride + col;
    _Float16* dst = y + m * N + n0;
    if ((N & 7) == 0 && n0 + 8 <= N) {
      *reinterpret_cast<half8_t*>(dst) = *reinterpret_cast<const half8_t*>(src);
    } else {
      for (int e = 0; e < 8 && n0 + e < N; ++e) dst[e] = src[e];
    }
  }
}

// Final stage of the partials combine: y[i] = fp16(part[0][i] + part[1][i] +
// ... + part[S-1][i]), added in split order in fp32, for i < count = M * N.
// VEC: four consecutive outputs per thread (count a multiple of 4).
template <bool VEC>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* __restrict__ part, int64_t count, int splits,
                                                         _Float16* __restrict__ y) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  if constexpr (VEC) {
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; 4 * i < count; i += stride) {
      f32x4v s = *reinterpret_cast<const f32x4v*>(part + 4 * i);
      for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4v*>(part + int64_t(z) * count + 4 * i);
      *reinterpret_cast<half4_t*>(y + 4 * i) = half4_t{(_Float16)s[0], (_Float16)s[1], (_Float16)s[2], (_Float16)s[3]};
    }
  } else {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count; i += stride) {
      float s = part[i];
      for (int z = 1; z < splits; ++z) s += part[int64_t(z) * count + i];
      y[i] = (_Float16)s;
    }
  }
}

}  // namespace dev

namespace {

template <int MB>
int launch_gemm_mb(int M, int N, int K, int splits, const void* wq, const void* scales, const void* zeros,
                   const void* x, void* y, unsigned long long* ws, float* part, hipStream_t stream) {
  static std::atomic<uint64_t> raised{0};  // devices on which the kernel's LDS limit is raised
  const size_t lds = dev::gemm_lds_bytes(MB);
  const hipError_t e = dev::raise_lds_limit(reinterpret_cast<const void*>(&dev::gemm_kernel<MB>), lds, raised);
  if (e != hipSuccess) return int(e);
  const int64_t NT = (int64_t(N) + kTileRows - 1) / kTileRows;
  const dim3 grid(unsigned((M + 16 * MB - 1) / (16 * MB)),
                  unsigned((NT + dev::kGemmBN / kTileRows - 1) / (dev::kGemmBN / kTileRows)), unsigned(splits));
  return int(dev::launch_kernel(&dev::gemm_kernel<MB>, grid, dim3(256), lds, stream, M, N, K, splits,
                                static_cast<const uint8_t*>(wq), static_cast<const uint16_t*>(scales),
                                static_cast<const uint8_t*>(zeros), static_cast<const _Float16*>(x),
                                static_cast<_Float16*>(y), splits > 1 && !part ? ws : nullptr,
                                splits > 1 ? part : nullptr));
}

}  // namespace

int launch_gemm(int M, int N, int K, int splits, const void* wq, const void* scales, const void* zeros,
                const void* x, void* y, unsigned long long* ws, void* stream, float* part) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc;
  switch (splits > 1 ? gemm_m_blocks(M) : gemm_m_blocks_unsplit(M, N)) {
    case 1: rc = launch_gemm_mb<1>(M, N, K, splits, wq, scales, zeros, x, y, ws, part, s); break;
    case 2: rc = launch_gemm_mb<2>(M, N, K, splits, wq, scales, zeros, x, y, ws, part, s); break;
    case 4: rc = launch_gemm_mb<4>(M, N, K, splits, wq, scales, zeros, x, y, ws, part, s); break;
    default: rc = launch_gemm_mb<8>(M, N, K, splits, wq, scales, zeros, x, y, ws, part, s); break;
  }
  if (rc != 0 || !part || splits < 2) return rc;
  // The final stage, on the same stream: about four outputs per thread
  // at once, 1024 workgroups at most (a grid-stride loop takes the rest).
  const int64_t count = int64_t(M) * N;
  const bool vec = (count & 3) == 0;
  const int64_t items = vec ? count / 4 : count;
  const unsigned grid = unsigned(std::min<int64_t>((items + 255) / 256, 1024));
  hipError_t e = vec ? dev::launch_kernel(&dev::splitk_sum_kernel<true>, dim3(grid), dim3(256), 0, s,
                                          static_cast<const float*>(part), count, splits, static_cast<_Float16*>(y))
                     : dev::launch_kernel(&dev::splitk_sum_kernel<false>, dim3(grid), dim3(256), 0, s,
                                          static_cast<const float*>(part), count, splits, static_cast<_Float16*>(y));
  return int(e);
}

}  // namespace w4a16

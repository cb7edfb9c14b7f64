// Host packer and unpacker for layout ID 2 (declared in include/w4a16.h).
//
// A tile is 16 rows x one group of 128 columns, 1024 bytes: 64 lanes of
// 16 bytes, lane l carrying row l%16 and four 8-column pieces
// (k = 32*kb + 8*(l/16) .. +7, kb = 0..3), one 32-bit word each. That is the
// A-operand footprint of a 16x16x32 fp16 MFMA and, for the VALU kernel, a
// lane-private run of 32 weights of one row, so one 16-byte load per lane
// fetches a wave's whole kilobyte contiguously.
//
// Inside a word the 8 weights follow the ValueShuffle interleave of
// "Building an LLM Inference Runtime ... H100", Bug #3 (weight j at nibble
// slot {0,4,1,5,2,6,3,7}[j]; AWQ's order in "Custom AWQ Dequantization
// Kernel", Part 2). With it, masking a word with 0x000F000F (and 0x00F000F0,
// then both again after a shift by 8) yields the fp16 pairs (w0,w1),
// (w2,w3), (w4,w5), (w6,w7) in column order, which is what the kernels use.
//
// The 16 scales and 16 zero points of a tile sit next to each other in tile
// order (32 and 8 bytes), so the scale and zero requests of a wave touch one
// cache line each instead of one line per row.
#include <cstdint>
#include <cstring>

#include "w4a16.h"
#include "w4a16_internal.h"

namespace {

// Bit position of weight j within its 32-bit word.
constexpr int kShift[8] = {0, 16, 4, 20, 8, 24, 12, 28};

bool shape_ok(int N, int K) { return N >= 0 && K >= W4A16_GROUP && K % W4A16_GROUP == 0; }

inline void store_le32(uint8_t* p, uint32_t v) {
  p[0] = uint8_t(v);
  p[1] = uint8_t(v >> 8);
  p[2] = uint8_t(v >> 16);
  p[3] = uint8_t(v >> 24);
}

inline uint32_t load_le32(const uint8_t* p) {
  return uint32_t(p[0]) | (uint32_t(p[1]) << 8) | (uint32_t(p[2]) << 16) | (uint32_t(p[3]) << 24);
}

}  // namespace

extern "C" int w4a16_layout_id(void) { return w4a16::kLayoutId; }

extern "C" int w4a16_check_layout(int layout_id) {
  return layout_id == w4a16::kLayoutId ? W4A16_OK : W4A16_ELAYOUT;
}

extern "C" int w4a16_packed_sizes(int N, int K, size_t* wq_bytes, size_t* s_bytes, size_t* z_bytes) {
  if (!shape_ok(N, K)) return W4A16_EINVAL;
  const w4a16::Geometry geo(N, K);
  if (wq_bytes) *wq_bytes = geo.wq_bytes();
  if (s_bytes) *s_bytes = geo.s_bytes();
  if (z_bytes) *z_bytes = geo.z_bytes();
  return W4A16_OK;
}

namespace {

// Logical data of one row of the matrix being packed; all null for a row
// that is zero (padding of the gate/up interleave).
struct RowData {
  const uint8_t* q;   // [K]
  const uint16_t* s;  // [K/128]
  const uint8_t* z;   // [K/128]
};

// Packs `rows` rows (rows past the last one up to the 16-row boundary are
// padding) whose data row_src(r) returns. Returns W4A16_EINVAL if a q or z
// value exceeds 15 (the outputs are then unspecified). Allocates nothing.
template <typename RowSrc>
int pack_rows(int64_t rows, int K, RowSrc row_src, void* wq_out, void* s_out, void* z_out) {
  const w4a16::Geometry geo(rows, K);
  uint8_t* wq = static_cast<uint8_t*>(wq_out);
  uint8_t* sp = static_cast<uint8_t*>(s_out);
  uint8_t* zp = static_cast<uint8_t*>(z_out);

  unsigned bad = 0;  // any bit above the low nibble of a q or z value
  for (int64_t t = 0; t < geo.row_tiles; ++t) {
    for (int lane16 = 0; lane16 < 16; ++lane16) {
      const int64_t row = 16 * t + lane16;
      const RowData d = row < rows ? row_src(row) : RowData{nullptr, nullptr, nullptr};
      for (int64_t g = 0; g < geo.groups; ++g) {
        uint8_t* tile = wq + (t * geo.groups + g) * w4a16::kTileBytes;
        for (int lane = lane16; lane < 64; lane += 16) {
          for (int kb = 0; kb < 4; ++kb) {
            uint32_t word = 0;
            if (d.q) {
              const uint8_t* src = d.q + g * W4A16_GROUP + 32 * kb + 8 * (lane >> 4);
              for (int j = 0; j < 8; ++j) {
                bad |= src[j];
                word |= uint32_t(src[j] & 15u) << kShift[j];
              }
            }
            store_le32(tile + lane * 16 + kb * 4, word);
          }
        }
      }
    }
  }
  bad &= ~15u;

  std::memset(sp, 0, geo.s_bytes());
  std::memset(zp, 0, geo.z_bytes());
  for (int64_t n = 0; n < rows; ++n) {
    const RowData d = row_src(n);
    if (!d.q) continue;
    for (int64_t g = 0; g < geo.groups; ++g) {
      const int64_t e = geo.meta_index(n, g);
      const uint16_t sv = d.s[g];
      sp[2 * e] = uint8_t(sv);
      sp[2 * e + 1] = uint8_t(sv >> 8);
      const uint8_t zv = d.z[g];
      bad |= zv & ~15u;
      zp[e >> 1] |= uint8_t((zv & 15u) << ((n & 1) * 4));
    }
  }
  return bad ? W4A16_EINVAL : W4A16_OK;
}

}  // namespace

extern "C" int w4a16_pack(int N, int K, const uint8_t* q, const uint16_t* s, const uint8_t* z,
                          void* wq_out, void* s_out, void* z_out) {
  if (!shape_ok(N, K)) return W4A16_EINVAL;
  if (N == 0) return W4A16_OK;
  if (!q || !s || !z || !wq_out || !s_out || !z_out) return W4A16_EINVAL;
  const int64_t G = K / W4A16_GROUP;
  return pack_rows(
      N, K, [&](int64_t r) { return RowData{q + r * int64_t(K), s + r * G, z + r * G}; }, wq_out, s_out, z_out);
}

extern "C" int w4a16_pack_gate_up(int F, int K, const uint8_t* qg, const uint16_t* sg, const uint8_t* zg,
                                  const uint8_t* qu, const uint16_t* su, const uint8_t* zu, void* wq_out,
                                  void* s_out, void* z_out) {
  if (!shape_ok(F, K)) return W4A16_EINVAL;
  if (F == 0) return W4A16_OK;
  if (!qg || !sg || !zg || !qu || !su || !zu || !wq_out || !s_out || !z_out) return W4A16_EINVAL;
  // 8-row blocks interleaved inside each 16-row tile: packed rows
  // 16j .. 16j+7 are gate rows 8j .. 8j+7, packed rows 16j+8 .. 16j+15 the
  // up rows of the same outputs; rows past F within a tile are zero. The
  // result has 16 * ceil(F/8) rows, which w4a16_packed_sizes must be able
  // to describe.
  const int64_t G = K / W4A16_GROUP, rows = 16 * ((int64_t(F) + 7) / 8);
  if (rows > INT32_MAX) return W4A16_EINVAL;
  return pack_rows(
      rows, K,
      [&](int64_t r) {
        const int64_t f = 8 * (r / 16) + r % 8;
        if (f >= F) return RowData{nullptr, nullptr, nullptr};
        return (r % 16) < 8 ? RowData{qg + f * K, sg + f * G, zg + f * G}
                            : RowData{qu + f * K, su + f * G, zu + f * G};
      },
      wq_out, s_out, z_out);
}

extern "C" int w4a16_unpack(int N, int K, const void* wq_in, const void* s_packed, const void* z_packed,
                            uint8_t* q, uint16_t* s, uint8_t* z) {
  if (!shape_ok(N, K)) return W4A16_EINVAL;
  if (N == 0) return W4A16_OK;
  if (!wq_in || !s_packed || !z_packed || !q || !s || !z) return W4A16_EINVAL;
  const w4a16::Geometry geo(N, K);
  const uint8_t* wq = static_cast<const uint8_t*>(wq_in);
  const uint8_t* sp = static_cast<const uint8_t*>(s_packed);
  const uint8_t* zp = static_cast<const uint8_t*>(z_packed);
  for (int64_t t = 0; t < geo.row_tiles; ++t) {
    for (int64_t g = 0; g < geo.groups; ++g) {
      const uint8_t* tile = wq + (t * geo.groups + g) * w4a16::kTileBytes;
      for (int lane = 0; lane < 64; ++lane) {
        const int64_t row = 16 * t + (lane & 15);
        if (row >= N) continue;
        for (int kb = 0; kb < 4; ++kb) {
          const uint32_t word = load_le32(tile + lane * 16 + kb * 4);
          uint8_t* dst = q + row * int64_t(K) + g * W4A16_GROUP + 32 * kb + 8 * (lane >> 4);
          for (int j = 0; j < 8; ++j) dst[j] = uint8_t((word >> kShift[j]) & 15u);
        }
      }
    }
  }
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < geo.groups; ++g) {
      const int64_t e = geo.meta_index(n, g);
      s[n * geo.groups + g] = uint16_t(sp[2 * e] | (sp[2 * e + 1] << 8));
      z[n * geo.groups + g] = uint8_t((zp[e >> 1] >> ((n & 1) * 4)) & 15u);
    }
  }
  return W4A16_OK;
}

extern "C" const char* w4a16_strerror(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_EINVAL: return "invalid argument (shape, pointer, alignment or value)";
    case W4A16_EUNSUPPORTED: return "unsupported: more than 8 activation rows, or a shape beyond an entry point's stated limits";
    case W4A16_ELAYOUT: return "packed layout ID mismatch";
    case W4A16_EHIP: return "HIP runtime refused the launch";
    default: return "unknown status";
  }
}

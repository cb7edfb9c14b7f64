// Host round-to-nearest quantizer (declared in include/w4a16.h): fp16 weights
// -> the logical (q, s, z) that w4a16_pack takes. One group of 128
// consecutive weights of a row at a time, in double precision, rows spread
// over the host's hardware threads.
//  - Symmetric, the scheme of "Building an LLM Inference Runtime ... H100",
//    "The Stack Architecture", and of "CodeAlign-Runtime", Level 3: the scale
//    is absmax / 7 and the signed code t in [-8, 7] is stored as q = t + 8
//    with z = 8.
//  - Asymmetric, for the uint4 zero points: the group's range widened to
//    contain 0, [lo, hi], gives s = (hi - lo) / 15 and z = round(-lo / s).
// Codes divide by the stored fp16 scale and round half to even.
#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "w4a16.h"
#include "w4a16_internal.h"

namespace {

uint16_t to_f16_bits(double v) {  // round to nearest even (the compiler's conversion)
  const _Float16 h = static_cast<_Float16>(v);
  uint16_t b;
  std::memcpy(&b, &h, 2);
  return b;
}

double from_f16_bits(uint16_t b) {
  _Float16 h;
  std::memcpy(&h, &b, 2);
  return static_cast<double>(h);
}

// Quantizes rows [r0, r1); returns false on a non-finite weight.
bool quantize_rows(int64_t r0, int64_t r1, int K, const uint16_t* w, int mode, uint8_t* q, uint16_t* s,
                   uint8_t* z) {
  std::fesetround(FE_TONEAREST);  // std::nearbyint rounds half to even under it
  const int G = K / W4A16_GROUP;
  double v[W4A16_GROUP];
  for (int64_t n = r0; n < r1; ++n) {
    for (int g = 0; g < G; ++g) {
      const uint16_t* wg = w + n * K + int64_t(g) * W4A16_GROUP;
      double lo = 0.0, hi = 0.0;
      for (int j = 0; j < W4A16_GROUP; ++j) {
        v[j] = from_f16_bits(wg[j]);
        if (!std::isfinite(v[j])) return false;
        lo = std::min(lo, v[j]);
        hi = std::max(hi, v[j]);
      }
      const double amax = std::max(std::fabs(lo), hi);  // +0 for an all-zero group
      const uint16_t sb = to_f16_bits(mode == 0 ? amax / 7.0 : (hi - lo) / 15.0);
      const double sv = from_f16_bits(sb);
      int zz = mode == 0 ? 8 : 0;
      if (mode == 1 && sv > 0.0) zz = int(std::clamp(std::nearbyint(-lo / sv), 0.0, 15.0));
      s[n * G + g] = sb;
      z[n * G + g] = uint8_t(zz);
      uint8_t* qg = q + n * K + int64_t(g) * W4A16_GROUP;
      for (int j = 0; j < W4A16_GROUP; ++j) {
        int code = zz;
        if (sv > 0.0) {
          const double r = std::nearbyint(v[j] / sv);
          code = mode == 0 ? int(std::clamp(r, -8.0, 7.0)) + 8 : int(std::clamp(r + zz, 0.0, 15.0));
        }
        qg[j] = uint8_t(code);
      }
    }
  }
  return true;
}

}  // namespace

extern "C" int w4a16_quantize(int N, int K, const uint16_t* w, int mode, uint8_t* q, uint16_t* s, uint8_t* z) {
  if (N < 0 || K < W4A16_GROUP || K % W4A16_GROUP != 0 || (mode != 0 && mode != 1)) return W4A16_EINVAL;
  if (N == 0) return W4A16_OK;
  if (!w || !q || !s || !z) return W4A16_EINVAL;
  const unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  const int64_t chunks = std::min<int64_t>(hw, std::max<int64_t>(1, int64_t(N) * K / (1 << 20)));
  auto rows_of = [&](int64_t c, int64_t& r0, int64_t& r1) {
    r0 = int64_t(N) * c / chunks;
    r1 = int64_t(N) * (c + 1) / chunks;
  };
  // Chunks go to host threads. A chunk no thread could be started for (or
  // every chunk, if the bookkeeping cannot be allocated) runs on the calling
  // thread, whose rounding mode is restored afterwards; every started
  // thread is joined. No exception leaves this C entry point.
  std::vector<std::thread> pool;
  std::vector<char> ok;
  int64_t started = 0;
  try {
    ok.assign(size_t(chunks), 1);
    pool.reserve(size_t(chunks));
    for (; started < chunks; ++started) {
      int64_t r0, r1;
      rows_of(started, r0, r1);
      char* flag = &ok[size_t(started)];
      pool.emplace_back([=] { *flag = quantize_rows(r0, r1, K, w, mode, q, s, z) ? 1 : 0; });
    }
  } catch (...) {
  }
  bool good = true;
  if (started < chunks) {
    const int saved = std::fegetround();
    for (int64_t c = started; c < chunks; ++c) {
      int64_t r0, r1;
      rows_of(c, r0, r1);
      good = quantize_rows(r0, r1, K, w, mode, q, s, z) && good;
    }
    std::fesetround(saved);
  }
  for (auto& th : pool) th.join();
  for (int64_t c = 0; c < started; ++c) good = good && ok[size_t(c)] != 0;
  return good ? W4A16_OK : W4A16_EINVAL;
}

/*
 * oracle_w4a16.c -- plain, slow, obviously correct fp64 CPU oracle for the
 * batch-1 W4A16 GEMV (4-bit weights, one fp16 scale and one 4-bit zero point
 * per group of 128 consecutive weights along K, fp16 activations).
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library. It shares no source, header, table
 * or helper with the HIP library; the two meet only through the seeded input
 * generators (synthetic.py), which hold none of the method's arithmetic.
 *
 * What is computed, and from which passage:
 *  - w[n][k] = (q[n][k] - z[n][g]) * s[n][g], g = floor(k/128): one fp16
 *    scale per group of 128 weights of one output row ("Building an LLM
 *    Inference Runtime ... Qwen2.5-Coder-7B on NVIDIA H100", section "The
 *    Stack Architecture"; "CodeAlign-Runtime", Level 3, "Quantization
 *    Scheme"), with the unsigned-q / 4-bit-zero-point form of the workload
 *    definition. The signed symmetric form of those pages is the special
 *    case q = t xor 8, z = 8.
 *  - y[m][n] = sum_k w[n][k] * x[m][k]: the row-major matrix-vector product
 *    of "CodeAlign-Runtime", Level 1 (one output per row of an N x K matrix),
 *    done in one pass without materialising W (Level 3).
 *  - The sum runs over k in ascending order in fp64; absref = sum_k |w*x|.
 *  - fp16 values are decoded and encoded (round to nearest, ties to even)
 *    from the IEEE-754 binary16 definition, written out below.
 *  - The INT8-activation alternative of "Building an LLM Inference Runtime",
 *    Bug #3 (Path A): per-group int8 activation codes and the integer-sum
 *    product (or_act_quant_i8, or_gemv_a8, at the end of this file).
 *
 * The packed layout (ID 2) is this project's own device layout; pack/unpack
 * here follow its written definition element by element. The nibble order
 * inside a 32-bit word is the interleave of "Building an LLM Inference
 * Runtime", Bug #3 (the ValueShuffle shift table), which is also the
 * interleaved order of "Custom AWQ Dequantization Kernel", Part 2.
 *
 * Layout ID 2, for an N x K matrix (K a multiple of 128, G = K/128):
 *   NP = N rounded up to 16, rows n >= N are zero. Tile (t, g) covers rows
 *   16t .. 16t+15 and group g; all three buffers list tiles in the order
 *   q = t*G + g.
 *   weights: NP/16 * G tiles of 1024 bytes; tile (t, g) starts at byte
 *     (t*G + g)*1024. Its 32-bit little-endian word (lane, kb), lane in
 *     [0,64), kb in [0,4), sits at byte lane*16 + kb*4 of the tile and holds
 *     row 16t + lane%16, columns k = 128g + 32kb + 8*(lane/16) + j, j in
 *     [0,8); weight j occupies bits 4*SLOT[j] .. 4*SLOT[j]+3,
 *     SLOT = {0,4,1,5,2,6,3,7}.
 *   scales: 16 fp16 values per tile; row n group g is element
 *     (t*G + g)*16 + n%16, t = n/16.
 *   zeros: 8 bytes per tile; row n group g is in byte (t*G + g)*8 + (n%16)/2,
 *     low nibble for even n, high nibble for odd n.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_GROUP 128

/* Deliberate mistakes, compiled in only by the planted-mistake test to show
 * that the pins catch them. The default build plants nothing. */
#ifndef OR_PLANT
#define OR_PLANT 0
#endif

int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int or_plant(void) { return OR_PLANT; }

/* ---------------------------------------------------------------- fp16 --- */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits. Exponent field 0: subnormal, value = f * 2^-24. Field 31: inf/NaN.
 * Otherwise value = (1024 + f) * 2^(e - 25). */
double or_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
#if OR_PLANT == 7
    v = ldexp((double)(1024 + f), -25); /* planted: hidden bit on subnormals */
#else
    v = ldexp((double)f, -24);
#endif
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even. */
uint16_t or_f64_to_f16(double v) {
  if (isnan(v)) return 0x7E00;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);           /* a = f * 2^e, f in [0.5, 1) : a in [2^(e-1), 2^e) */
  int ulp = e - 11;       /* spacing of binary16 numbers in that binade */
  if (ulp < -24) ulp = -24; /* subnormal spacing */
#if OR_PLANT == 6
  double r = floor(ldexp(a, -ulp)); /* planted: truncation instead of rounding */
#else
  double r = rint(ldexp(a, -ulp)); /* exact scaling, then ties-to-even */
#endif
  if (r >= 2048.0) {      /* rounded up into the next binade */
    r /= 2.0;
    ulp += 1;
  }
  if (ulp == -24 && r <= 1024.0) /* subnormal, or exactly the smallest normal */
    return sign | (uint16_t)r;
  int field = ulp + 25;   /* value = (1024 + frac) * 2^(field - 25) */
  if (field >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(field << 10) | (uint16_t)((int)r - 1024);
}

void or_f16_to_f64_array(const uint16_t* h, double* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = or_f16_to_f64(h[i]);
}

void or_f64_to_f16_array(const double* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = or_f64_to_f16(v[i]);
}

/* ------------------------------------------------------ layout ID 2 --- */

static const int SLOT[8] = {0, 4, 1, 5, 2, 6, 3, 7};

static int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

static int shape_ok(int64_t N, int64_t K) {
  return N >= 0 && K >= OR_GROUP && K % OR_GROUP == 0;
}

int or_layout_id(void) { return 2; }

/* out[0] = weight bytes, out[1] = scale bytes, out[2] = zero bytes */
int or_layout_sizes(int64_t N, int64_t K, int64_t* out) {
  if (!shape_ok(N, K)) return -1;
  int64_t NP = round_up(N, 16), G = K / OR_GROUP;
  out[0] = NP * K / 2;
  out[1] = NP * G * 2;
  out[2] = NP * G / 2;
  return 0;
}

/* Where weight (n, k) lives: byte offset of its 32-bit word, and bit shift. */
static void locate_weight(int64_t n, int64_t k, int64_t G, int64_t* word_byte, int* shift) {
  int64_t t = n / 16, i = n % 16, g = k / OR_GROUP, r = k % OR_GROUP;
  int64_t kb = r / 32, lane_group = (r % 32) / 8, j = r % 8;
  int64_t lane = i + 16 * lane_group;
#if OR_PLANT == 5
  j = 7 - j; /* planted: nibble order reversed */
#endif
  *word_byte = (t * G + g) * 1024 + lane * 16 + kb * 4;
  *shift = 4 * SLOT[j];
}

static uint32_t read_u32le(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static void write_u32le(uint8_t* p, uint32_t v) {
  p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); p[2] = (uint8_t)(v >> 16); p[3] = (uint8_t)(v >> 24);
}

static int weight_at(const uint8_t* wq, int64_t n, int64_t k, int64_t G) {
  int64_t wb; int sh;
  locate_weight(n, k, G, &wb, &sh);
  return (int)((read_u32le(wq + wb) >> sh) & 15u);
}

/* Element index of (n, g) in the scale buffer; the zero buffer holds half
 * as many bytes per tile (two nibbles per byte). */
static int64_t scale_index(int64_t n, int64_t g, int64_t G) {
#if OR_PLANT == 13
  /* planted: rows of a block reversed past the first row tile (a permutation:
     round trips and first-tile checks cannot see it) */
  if (n >= 16) return ((n / 16) * G + g) * 16 + 15 - n % 16;
#endif
  return ((n / 16) * G + g) * 16 + n % 16;
}

static uint16_t scale_at(const uint8_t* sp, int64_t n, int64_t g, int64_t G) {
  const uint8_t* p = sp + 2 * scale_index(n, g, G);
  return (uint16_t)(p[0] | (p[1] << 8));
}

static int zero_at(const uint8_t* zp, int64_t n, int64_t g, int64_t G) {
  uint8_t b = zp[scale_index(n, g, G) / 2];
  return (n & 1) ? (b >> 4) : (b & 15);
}

/* q: [N][K] values 0..15; s: [N][G] fp16 bits; z: [N][G] values 0..15.
 * Outputs are overwritten entirely (padding included). */
int or_pack(int64_t N, int64_t K, const uint8_t* q, const uint16_t* s, const uint8_t* z,
            uint8_t* wq, uint8_t* sp, uint8_t* zp) {
  int64_t sz[3];
  if (or_layout_sizes(N, K, sz)) return -1;
  int64_t G = K / OR_GROUP;
  memset(wq, 0, (size_t)sz[0]);
  memset(sp, 0, (size_t)sz[1]);
  memset(zp, 0, (size_t)sz[2]);
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k = 0; k < K; k++) {
      uint8_t v = q[n * K + k];
      if (v > 15) return -1;
      int64_t wb; int sh;
      locate_weight(n, k, G, &wb, &sh);
      write_u32le(wq + wb, read_u32le(wq + wb) | ((uint32_t)v << sh));
    }
    for (int64_t g = 0; g < G; g++) {
      uint16_t sv = s[n * G + g];
      int64_t e = scale_index(n, g, G);
      sp[2 * e] = (uint8_t)(sv & 0xFF);
      sp[2 * e + 1] = (uint8_t)(sv >> 8);
      uint8_t zv = z[n * G + g];
      if (zv > 15) return -1;
      zp[e / 2] |= (uint8_t)((n & 1) ? (zv << 4) : zv);
    }
  }
  return 0;
}

int or_unpack(int64_t N, int64_t K, const uint8_t* wq, const uint8_t* sp, const uint8_t* zp,
              uint8_t* q, uint16_t* s, uint8_t* z) {
  if (!shape_ok(N, K)) return -1;
  int64_t G = K / OR_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k = 0; k < K; k++) q[n * K + k] = (uint8_t)weight_at(wq, n, k, G);
    for (int64_t g = 0; g < G; g++) {
      s[n * G + g] = scale_at(sp, n, g, G);
      z[n * G + g] = (uint8_t)zero_at(zp, n, g, G);
    }
  }
  return 0;
}

/* ------------------------------------------------------ arithmetic --- */

/* The dequantized weight, exact in fp64 (|q - z| <= 15 has 4 bits, s has an
 * 11-bit significand). */
static double dequant_one(int q, int z, uint16_t s_bits) {
#if OR_PLANT == 1
  (void)z;
  return (double)q * or_f16_to_f64(s_bits); /* planted: zero point dropped */
#elif OR_PLANT == 2
  return (double)(z - q) * or_f16_to_f64(s_bits); /* planted: sign flipped */
#else
  return (double)(q - z) * or_f16_to_f64(s_bits);
#endif
}

static int64_t group_of(int64_t k) {
#if OR_PLANT == 3
  return k / OR_GROUP / 2; /* planted: neighbouring groups share a scale */
#else
  return k / OR_GROUP;
#endif
}

/* w: [N][K] doubles */
int or_dequant(int64_t N, int64_t K, const uint8_t* q, const uint16_t* s, const uint8_t* z, double* w) {
  if (!shape_ok(N, K)) return -1;
  int64_t G = K / OR_GROUP;
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      int64_t g = group_of(k);
      w[n * K + k] = dequant_one(q[n * K + k], z[n * G + g], s[n * G + g]);
    }
  return 0;
}

/* ref, absref: [M][N] doubles; x: [M][K] fp16 bits. */
/* ------------------------------------------------------- quantizer --- */

/* Round-to-nearest quantization of fp16 weights w[N][K] to (q, s, z), one
 * group of 128 consecutive weights of a row at a time, in fp64.
 *  mode 0, symmetric ("Building an LLM Inference Runtime", "The Stack
 *    Architecture"; "CodeAlign-Runtime", Level 3, "Quantization Scheme"):
 *    s = fp16(absmax / 7), t = clamp(round(w / s), -8, 7), stored unsigned
 *    as q = t + 8 with z = 8 (so (q - z) * s = t * s).
 *  mode 1, asymmetric (the uint4 zero points of the workload; the range is
 *    widened to contain 0 so that 0 and constant groups stay exact):
 *    lo = min(min(w), 0), hi = max(max(w), 0), s = fp16((hi - lo) / 15),
 *    z = clamp(round(-lo / s), 0, 15), q = clamp(round(w / s) + z, 0, 15).
 * round() is round-half-to-even; the division uses the stored fp16 scale.
 * A group whose scale rounds to 0 gets q = z (mode 0: 8, mode 1: 0), which
 * dequantizes to 0. */
static double round_half_even(double v) {
  double f = floor(v);
  double d = v - f;
  if (d > 0.5) return f + 1.0;
  if (d < 0.5) return f;
  return fmod(f, 2.0) == 0.0 ? f : f + 1.0;
}

static double clamp_d(double v, double lo, double hi) { return v < lo ? lo : (v > hi ? hi : v); }

int or_quantize(int64_t N, int64_t K, const uint16_t* w, int mode, uint8_t* q, uint16_t* s, uint8_t* z) {
  if (!shape_ok(N, K) || (mode != 0 && mode != 1)) return -1;
  int64_t G = K / OR_GROUP;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const uint16_t* wg = w + n * K + g * OR_GROUP;
      double lo = 0.0, hi = 0.0, amax = 0.0;
      for (int j = 0; j < OR_GROUP; j++) {
        double v = or_f16_to_f64(wg[j]);
        if (v != v || v - v != 0.0) return -1; /* NaN or infinite weight */
        if (v < lo) lo = v;
        if (v > hi) hi = v;
        if (fabs(v) > amax) amax = fabs(v);
      }
#if OR_PLANT == 8
      uint16_t sb = mode == 0 ? or_f64_to_f16(amax / 8.0) : or_f64_to_f16((hi - lo) / 15.0); /* planted */
#else
      uint16_t sb = mode == 0 ? or_f64_to_f16(amax / 7.0) : or_f64_to_f16((hi - lo) / 15.0);
#endif
      double sd = or_f16_to_f64(sb);
      int zz = mode == 0 ? 8 : 0;
      if (sd > 0.0 && mode == 1) zz = (int)clamp_d(round_half_even(-lo / sd), 0.0, 15.0);
      s[n * G + g] = sb;
      z[n * G + g] = (uint8_t)zz;
      for (int j = 0; j < OR_GROUP; j++) {
        int qq = zz;
        if (sd > 0.0) {
          double r = round_half_even(or_f16_to_f64(wg[j]) / sd);
#if OR_PLANT == 9
          qq = mode == 0 ? (int)clamp_d(r, -8.0, 7.0) + 8 : (int)clamp_d(r, 0.0, 15.0); /* planted: z dropped */
#else
          qq = mode == 0 ? (int)clamp_d(r, -8.0, 7.0) + 8 : (int)clamp_d(r + zz, 0.0, 15.0);
#endif
        }
        q[n * K + g * OR_GROUP + j] = (uint8_t)qq;
      }
    }
  }
  return 0;
}

int or_gemv(int64_t M, int64_t N, int64_t K, const uint8_t* q, const uint16_t* s, const uint8_t* z,
            const uint16_t* x, double* ref, double* absref) {
  if (M < 0 || !shape_ok(N, K)) return -1;
  if (M == 0 || N == 0) return 0;
  int64_t G = K / OR_GROUP;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd) return -2;
  for (int64_t i = 0; i < M * K; i++) xd[i] = or_f16_to_f64(x[i]);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t m = 0; m < M; m++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        int64_t g = group_of(k);
        double w = dequant_one(q[n * K + k], z[n * G + g], s[n * G + g]);
#if OR_PLANT == 4
        double xv = xd[k * M + m]; /* planted: activations read as [K][M] */
#else
        double xv = xd[m * K + k];
#endif
        acc += w * xv;
        aacc += fabs(w * xv);
      }
      ref[m * N + n] = acc;
      absref[m * N + n] = aacc;
    }
  }
  free(xd);
  return 0;
}

/* Same product with the weights given in layout ID 2: every element is
 * located through the layout definition, then the same formula applies. */
int or_gemv_packed(int64_t M, int64_t N, int64_t K, const uint8_t* wq, const uint8_t* sp,
                   const uint8_t* zp, const uint16_t* x, double* ref, double* absref) {
  if (M < 0 || !shape_ok(N, K)) return -1;
  if (M == 0 || N == 0) return 0;
  int64_t G = K / OR_GROUP;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K));
  if (!xd) return -2;
  for (int64_t i = 0; i < M * K; i++) xd[i] = or_f16_to_f64(x[i]);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t n = 0; n < N; n++) {
    for (int64_t m = 0; m < M; m++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        int64_t g = group_of(k);
        double w = dequant_one(weight_at(wq, n, k, G), zero_at(zp, n, g, G), scale_at(sp, n, g, G));
        double xv = xd[m * K + k];
        acc += w * xv;
        aacc += fabs(w * xv);
      }
      ref[m * N + n] = acc;
      absref[m * N + n] = aacc;
    }
  }
  free(xd);
  return 0;
}

/* Rows listed in `rows` only (for sampled checks at full size):
 * ref/absref are [M][nrows]. */
int or_gemv_packed_rows(int64_t M, int64_t N, int64_t K, const uint8_t* wq, const uint8_t* sp,
                        const uint8_t* zp, const uint16_t* x, const int64_t* rows, int64_t nrows,
                        double* ref, double* absref) {
  if (M < 0 || !shape_ok(N, K)) return -1;
  int64_t G = K / OR_GROUP;
  for (int64_t r = 0; r < nrows; r++)
    if (rows[r] < 0 || rows[r] >= N) return -1;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
  if (!xd) return -2;
  for (int64_t i = 0; i < M * K; i++) xd[i] = or_f16_to_f64(x[i]);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; r++) {
    int64_t n = rows[r];
    for (int64_t m = 0; m < M; m++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        int64_t g = group_of(k);
        double w = dequant_one(weight_at(wq, n, k, G), zero_at(zp, n, g, G), scale_at(sp, n, g, G));
        double xv = xd[m * K + k];
        acc += w * xv;
        aacc += fabs(w * xv);
      }
      ref[m * nrows + r] = acc;
      absref[m * nrows + r] = aacc;
    }
  }
  free(xd);
  return 0;
}

/* ---------------------------------------------------------------------------
 * INT8 activations: the alternative path of "Building an LLM Inference
 * Runtime ... on NVIDIA H100", Bug #3 (Path A). A separate step turns the fp16
 * activations into signed 8-bit codes with one scale per group; the weight
 * codes and activation codes are multiplied and summed as integers; each
 * group's integer sum is then brought back to a real value with the
 * activation scale and the weight scale.
 *
 * The pages name the per-group activation scale but fix neither the group,
 * the code range, the rounding nor the precision. Readings taken here:
 *  - an activation group is 128 consecutive k of one activation row m, the
 *    same k range as a weight group, so exactly one activation scale meets
 *    one weight scale in each group sum;
 *  - symmetric codes in [-127, 127]: sx = absmax / 127 and
 *    xq = clamp(round_half_even(x / sx), -127, 127), a group of zeros giving
 *    sx = 0 and xq = 0;
 *  - the rounding decision is taken in IEEE single precision: absmax is
 *    exact, sx is one correctly rounded division and x / sx another;
 *  - xsum[m][g], the sum of the group's codes, is an output of the same step.
 */
int or_act_quant_i8(int64_t M, int64_t K, const uint16_t* x, int8_t* xq, float* sx, int32_t* xsum) {
  if (M < 0 || K < OR_GROUP || K % OR_GROUP != 0) return -1;
  int64_t G = K / OR_GROUP;
  for (int64_t m = 0; m < M; m++) {
    for (int64_t g = 0; g < G; g++) {
      const uint16_t* xg = x + m * K + g * OR_GROUP;
      float amax = 0.0f;
      for (int j = 0; j < OR_GROUP; j++) {
        double v = or_f16_to_f64(xg[j]);
        if (v != v || v - v != 0.0) return -1; /* NaN or infinite activation */
        float a = (float)fabs(v);              /* exact: fp16 values are floats */
        if (a > amax) amax = a;
      }
#if OR_PLANT == 10
      float scale = amax / 128.0f; /* planted: code range 128 */
#else
      float scale = amax / 127.0f;
#endif
      int32_t sum = 0;
      for (int j = 0; j < OR_GROUP; j++) {
        int code = 0;
        if (scale > 0.0f) {
          float r = (float)or_f16_to_f64(xg[j]) / scale;
          code = (int)clamp_d(round_half_even((double)r), -127.0, 127.0);
        }
        xq[m * K + g * OR_GROUP + j] = (int8_t)code;
        sum += code;
      }
      sx[m * G + g] = scale;
      xsum[m * G + g] = sum;
    }
  }
  return 0;
}

/* y[m][n] = sum_g s[n][g] * sx[m][g] * sum_{k in g} (q[n][k] - z[n][g]) * xq[m][k]
 * from the logical q, s, z. The integer sum is exact (|.| <= 128*15*127 <
 * 2^18) and so is the product of the three factors in fp64 (11 + 24 + 18
 * significant bits); only the fp64 sum over groups, in ascending g, rounds.
 * absref = sum_g |s * sx * integer sum|. With `rows` (nrows entries), only
 * those rows, ref/absref [M][nrows]; with rows == NULL all N rows, [M][N]. */
int or_gemv_a8(int64_t M, int64_t N, int64_t K, const uint8_t* q, const uint16_t* s, const uint8_t* z,
               const int8_t* xq, const float* sx, const int64_t* rows, int64_t nrows, double* ref,
               double* absref) {
  if (M < 0 || !shape_ok(N, K)) return -1;
  int64_t G = K / OR_GROUP;
  int64_t R = rows ? nrows : N;
  for (int64_t r = 0; rows && r < nrows; r++)
    if (rows[r] < 0 || rows[r] >= N) return -1;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < R; r++) {
    int64_t n = rows ? rows[r] : r;
    for (int64_t m = 0; m < M; m++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t g = 0; g < G; g++) {
        int64_t isum = 0;
        for (int64_t k = g * OR_GROUP; k < (g + 1) * OR_GROUP; k++) {
#if OR_PLANT == 12
          isum += (int64_t)q[n * K + k] * xq[m * K + k]; /* planted: zero point dropped */
#else
          isum += ((int64_t)q[n * K + k] - z[n * G + g]) * xq[m * K + k];
#endif
        }
#if OR_PLANT == 11
        double term = or_f16_to_f64(s[n * G + g]) * (double)sx[g] * (double)isum; /* planted: row 0's scale */
#else
        double term = or_f16_to_f64(s[n * G + g]) * (double)sx[m * G + g] * (double)isum;
#endif
        acc += term;
        aacc += fabs(term);
      }
      ref[m * R + r] = acc;
      absref[m * R + r] = aacc;
    }
  }
  return 0;
}

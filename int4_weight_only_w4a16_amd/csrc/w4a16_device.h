// Device helpers shared by the HIP kernels of libw4a16.so (gfx950): packed
// fp16 types, the in-register unpack of one packed word, and an LDS-only
// workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "w4a16_internal.h"

namespace w4a16 {
namespace dev {

template <typename T>
struct same_type {
  using type = T;
};

// Launches `kernel` and returns the status of this launch alone (a launch
// followed by hipGetLastError() would also report an error an earlier,
// unrelated runtime call left behind in the thread). The arguments convert
// to the kernel's parameter types; their copies are what the launch reads.
template <typename... KArgs>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         typename same_type<KArgs>::type... args) {
  void* ptrs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, stream);
}

// Raises `kernel`'s dynamic-LDS limit to `bytes` on the current device, once
// per device: `done` is the caller's per-kernel record, one bit per device
// (64 devices; beyond that the call is simply repeated). Concurrent first
// calls may both set the attribute, which is harmless.
inline hipError_t raise_lds_limit(const void* kernel, size_t bytes, std::atomic<uint64_t>& done) {
  int device = 0;
  const hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  const uint64_t bit = device >= 0 && device < 64 ? uint64_t(1) << device : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t r = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (r == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return r;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagic1024 = 0x64006400u;  // fp16 pair (1024, 1024)

// Split-K accumulation word (uint64 per output). Bits 0..58 hold the sum of
// the splits' biased fixed-point partials, bits 59..63 the number of splits
// that have added. A partial p becomes f = round(p * 2^24) (RNE), clamped to
// |f| < 2^53, i.e. |p| < 2^29; the addend is 2^59 + (f + 2^53), which lies in
// [2^59, 2^59 + 2^54). With at most kMaxSplits = 31 splits the biased sum
// stays below 31 * 2^54 < 2^59 and never carries into the count. A NaN
// partial counts as 0. (2^29 is far past anything an fp16 output can hold:
// where a partial reaches it, the GEMV bound 2e-3 * sum|w x| already exceeds
// the whole fp16 range.)
constexpr double kSplitkScale = 16777216.0;  // 2^24
constexpr double kSplitkLimit = 9007199254740991.0;  // 2^53 - 1

__device__ __forceinline__ unsigned long long splitk_addend(float p) {
  double d = double(p) * kSplitkScale;  // exact: an fp32 times a power of two
  d = d != d ? 0.0 : fmin(fmax(d, -kSplitkLimit), kSplitkLimit);
  const long long f = (long long)rint(d);
  return (1ull << 59) + (unsigned long long)(f + (1ll << 53));
}

__device__ __forceinline__ unsigned splitk_count(unsigned long long word) { return unsigned(word >> 59); }

// fp16 of the exact fixed-point total of a complete word (via fp64 and fp32).
__device__ __forceinline__ _Float16 splitk_value(unsigned long long word, int splits) {
  const long long total = (long long)(word & ((1ull << 59) - 1)) - (long long)splits * (1ll << 53);
  return (_Float16)(float)(double(total) / kSplitkScale);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// s_waitcnt operand (gfx9 encoding) that waits until at most n (< 64)
// vector-memory requests are outstanding, not waiting on expcnt or lgkmcnt.
constexpr int vmcnt_at_most(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// One 16-byte global-to-LDS request per active lane: lane l writes its 16
// bytes at l + 16 l (l = the wave-uniform LDS address). Before a later LDS
// read the compiler waits for every outstanding vector-memory request
// (vmcnt 0): these requests need not complete in order with ordinary loads
// (counting them exactly, from inline asm, gave run-to-run differences), so
// that is the only safe wait. (A plain device function: the host-side
// instantiation of a kernel template that names the builtin fails, and the
// kernel's launch stub silently goes missing.)
__device__ __forceinline__ void load_lds16(const _Float16* g, _Float16* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Activation row of staged chunk c, chunks_per_row chunks per row (c below
// MR * chunks_per_row): 0 without a division for one row, else an unsigned
// 32-bit division (cheaper than the signed one).
template <int MR>
__device__ __forceinline__ int row_of_chunk(int c, int chunks_per_row) {
  if constexpr (MR == 1) {
    return 0;
  } else {
    return int(unsigned(c) / unsigned(chunks_per_row));
  }
}

// fp16 pairs (1024 + z, 1024 + z) and (64 + z, 64 + z) for a zero point z.
// 1024 + z has bits 0x6400 | z (spacing 1 in [1024, 2048)); 64 + z has bits
// 0x5400 | (z << 4) (spacing 1/16 in [64, 128)).
struct ZeroPairs {
  half2_t z1024, z64;
};

__device__ __forceinline__ ZeroPairs zero_pairs(uint32_t z) {
  return {as_h2((0x6400u | z) * 0x00010001u), as_h2((0x5400u | (z << 4)) * 0x00010001u)};
}

// (w & mask) | magic in one VALU op. gfx9 VOP3 has no literal operand, so
// with literal operands the compiler splits this into v_and_b32 + v_or_b32;
// with the mask in an SGPR and the magic in a VGPR (each made opaque by an
// empty asm, which emits no instruction) it selects a single v_and_or_b32
// itself. The instruction is the compiler's own, not inline asm: the
// compiler then knows which VGPR it writes and keeps that write clear of the
// destination of an MFMA still in flight (a VGPR written by an inline asm
// instruction is invisible to its hazard checks).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  asm("" : "+s"(mask));
  asm("" : "+v"(magic));
  return (w & mask) | magic;
}

// Eight weights of one ValueShuffle word -> (q - z) as four fp16 pairs in
// column order (w0,w1), (w2,w3), (w4,w5), (w6,w7). OR-ing a nibble into the
// mantissa of 1024.0 gives 1024 + q exactly; a nibble four bits higher gives
// 1024 + 16q, and (1024 + 16q)/16 - (64 + z) = q - z. Every step is exact in
// fp16 (all values are integers or sixteenths below 2048).
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t magic, const ZeroPairs& zp, half2_t p[4]) {
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  p[0] = as_h2(and_or(w, 0x000F000Fu, magic)) - zp.z1024;
  p[1] = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, magic)), sixteenth, -zp.z64);
  p[2] = as_h2(and_or(w8, 0x000F000Fu, magic)) - zp.z1024;
  p[3] = __builtin_elementwise_fma(as_h2(and_or(w8, 0x00F000F0u, magic)), sixteenth, -zp.z64);
}

// Workgroup barrier that orders LDS only. __syncthreads() also fences global
// memory, which makes every wave wait for all of its outstanding loads
// (vmcnt(0)) -- including weight tiles requested ahead -- before the barrier.
// No thread here communicates through global memory, so an LDS-scope fence
// (lgkmcnt only) is all the barriers need.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Inner-product engines. kEngineMfma*: v_mfma_f32_16x16x32_f16
// with the activations as the A operand (row m of A = x[m]; rows >= M repeat
// the last x row and are ignored) and the unpacked weights as the B operand
// (column j of B = weight row j of the tile), so D[m][j] = sum_k x[m][k]
// w[j][k]; the multiply-adds leave the VALU, which then only unpacks. The
// A operand comes from LDS (kEngineMfma) or, when x of the K range does not
// fit in LDS, straight from global memory with the weights of the batch
// (kEngineMfmaGlobalX).
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

}  // namespace dev
}  // namespace w4a16

// Split-K GEMV without a caller workspace (w4a16_gemv_splitk_noalloc), for
// callers that cannot allocate device memory: code under graph capture,
// serving loops and harnesses that forbid hipMalloc. The split-K
// accumulation words (one uint64 per output, zero between calls) live in a
// file-scope device array instead of a workspace argument. Each GPU the
// library runs on holds its own copy of the array until the process ends.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "w4a16.h"
#include "w4a16_device.h"
#include "w4a16_internal.h"

namespace {

constexpr size_t kScratchWords = W4A16_NOALLOC_SCRATCH_BYTES / sizeof(unsigned long long);

// The accumulation words. In host code `scratch` names a host-side stand-in,
// not the device array: every host use goes through the address that
// hipGetSymbolAddress returned for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned long long scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_setup;                                     // serializes first calls
std::atomic<unsigned long long*> g_scratch[kMaxDevices];  // device address of `scratch`, per device

__global__ __launch_bounds__(256) void zero_words(unsigned long long* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// Device address of this device's `scratch`, looked up once per device with
// that device current. The first call on a device also clears the array
// with a fill kernel on `stream` (the array starts zero when the code object
// loads; the fill makes that explicit, and it is a kernel, not a memset, so
// that a captured first call stays correct on every replay). Returns null on
// a runtime error.
unsigned long long* scratch_ptr(hipStream_t stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices) return nullptr;
  unsigned long long* p = g_scratch[device].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_setup);
  p = g_scratch[device].load(std::memory_order_acquire);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
  p = static_cast<unsigned long long*>(addr);
  const int n = int(kScratchWords);
  if (w4a16::dev::launch_kernel(&zero_words, dim3((n + 255) / 256), dim3(256), 0, stream, p, n) != hipSuccess)
    return nullptr;
  g_scratch[device].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" int w4a16_gemv_splitk_noalloc(int M, int N, int K, int splits, const void* Wq, const void* scales,
                                         const void* zeros, const void* x, void* y, void* stream) {
  if (K < W4A16_GROUP || K % W4A16_GROUP != 0 || M < 0 || N < 0) return W4A16_EINVAL;
  if (M > W4A16_MAX_M) return W4A16_EUNSUPPORTED;
  if (splits < 1 || splits > K / W4A16_GROUP || splits > w4a16::kMaxSplits) return W4A16_EINVAL;
  if (M == 0 || N == 0) return W4A16_OK;
  if (splits == 1) return w4a16_gemv(M, N, K, Wq, scales, zeros, x, y, stream);
  if (size_t(M) * size_t(N) > kScratchWords) return W4A16_EUNSUPPORTED;
  for (const void* ptr : {Wq, scales, zeros, x, static_cast<const void*>(y)})
    if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 15u) != 0) return W4A16_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* acc = scratch_ptr(s);
  if (!acc) return W4A16_EHIP;
  // The same plan and kernel as w4a16_gemv_splitk, so the result is that
  // entry point's, bit for bit.
  return w4a16::gemv_splitk_status(M, N, K, splits, Wq, scales, zeros, x, y, acc, stream);
}

// GEMV instantiations for M = 5 activation rows.
#include "gemv_kernel.h"

namespace w4a16 {

int launch_gemv_m5(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                    const void* zeros, const void* x, void* y, unsigned long long* acc, void* stream) {
  return int(dev::launch_engine<5>(N, K, plan, wq, scales, zeros, x, y, acc,
                                     static_cast<hipStream_t>(stream)));
}

}  // namespace w4a16

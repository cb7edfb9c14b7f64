// GEMV instantiations for M = 1 activation rows.
#include "gemv_kernel.h"

namespace w4a16 {

int launch_gemv_m1(int N, int K, const LaunchPlan& plan, const void* wq, const void* scales,
                    const void* zeros, const void* x, void* y, unsigned long long* acc, void* stream) {
  return int(dev::launch_engine<1>(N, K, plan, wq, scales, zeros, x, y, acc,
                                     static_cast<hipStream_t>(stream)));
}

}  // namespace w4a16

// finite.hip -- the debug finiteness check behind SSMVJP_CHECK_FINITE: a scan
// of an output tensor that raises a flag if any element is NaN or infinite.
// Every writer stores the same value, so the flag does not depend on the order
// in which the threads run.
#include "common.cuh"
#include "kernels.h"

namespace ssmvjp {
namespace {

__global__ void __launch_bounds__(256) flag_clear_kernel(unsigned* flag) {
  if (threadIdx.x == 0) *flag = 0u;
}

template <typename T>
__global__ void __launch_bounds__(256) nonfinite_scan_kernel(const T* p, i64 n, unsigned* flag) {
  bool bad = false;
  for (i64 i = (i64)blockIdx.x * 256 + threadIdx.x; i < n; i += (i64)gridDim.x * 256) {
    const float v = (float)p[i];
    bad |= !(fabsf(v) <= 3.402823466e38f);  // false for NaN and +-inf
  }
  if (bad) *flag = 1u;
}

}  // namespace

void launch_flag_clear(unsigned* flag, hipStream_t stream) {
  hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(64), 0, stream, flag);
}

void launch_nonfinite_check(const void* p, int64_t n, bool is_bf16, unsigned* flag, hipStream_t stream) {
  if (!p || n <= 0) return;
  const i64 blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  if (is_bf16)
    hipLaunchKernelGGL(nonfinite_scan_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, stream, (const bf16*)p, n,
                       flag);
  else
    hipLaunchKernelGGL(nonfinite_scan_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream, (const float*)p, n,
                       flag);
}

}  // namespace ssmvjp

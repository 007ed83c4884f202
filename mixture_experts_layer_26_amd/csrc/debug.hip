// Index validation for MOE_DEBUG=1: the calls that take index arrays from earlier calls
// (topk_idx, expert_offset, sorted_token, pair_row) check them on the device before
// launching anything that uses them as addresses. The result is one int in a file-scope
// device variable, so nothing is allocated; reading it back synchronises the stream,
// which only debug mode pays.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

__device__ int g_bad;  // nonzero once a check found an index out of range

__global__ void clear_flag_kernel(int* flag) {
  if (threadIdx.x == 0) flag[0] = 0;
}

// every p[i] in [lo, hi)
__global__ void check_range_kernel(const int32_t* __restrict__ p, int64_t n, int32_t lo, int32_t hi, int* flag) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int32_t v = p[i];
    if (v < lo || v >= hi) flag[0] = 1;
  }
}

// offset[0] == 0, offset[n] == total, non-decreasing
__global__ void check_offsets_kernel(const int32_t* __restrict__ offset, int n, int32_t total, int* flag) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i <= n; i += gridDim.x * blockDim.x) {
    const int32_t v = offset[i];
    bool bad = (i == 0 && v != 0) || (i == n && v != total);
    if (i < n && offset[i + 1] < v) bad = true;
    if (bad) flag[0] = 1;
  }
}

}  // namespace

hipError_t debug_check_indices(const IndexCheck* checks, int count, hipStream_t stream, bool* bad) {
  int* flag = nullptr;
  hipError_t err = hipGetSymbolAddress(reinterpret_cast<void**>(&flag), HIP_SYMBOL(g_bad));
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(64), 0, stream, flag);
  for (int i = 0; i < count; ++i) {
    const IndexCheck& c = checks[i];
    if (c.offsets) {
      hipLaunchKernelGGL(check_offsets_kernel, dim3(1), dim3(256), 0, stream, c.p, static_cast<int>(c.n),
                         c.hi, flag);
    } else {
      const int64_t want = (c.n + 255) / 256;
      const unsigned blocks = static_cast<unsigned>(want < 1024 ? (want > 0 ? want : 1) : 1024);
      hipLaunchKernelGGL(check_range_kernel, dim3(blocks), dim3(256), 0, stream, c.p, c.n, c.lo, c.hi, flag);
    }
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  int host = 0;
  if ((err = hipMemcpyAsync(&host, flag, sizeof(int), hipMemcpyDeviceToHost, stream)) != hipSuccess) return err;
  if ((err = hipStreamSynchronize(stream)) != hipSuccess) return err;
  *bad = host != 0;
  return hipSuccess;
}

}  // namespace moe

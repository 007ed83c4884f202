// Grouped SwiGLU expert FFN for fp32 operands (the small fp32 workload): one thread per
// output element, plain fp32 FMA dot products. Same row layout as the bf16 path:
// H routed [P, d_ff] in sorted-row order, then H shared [T, n_s * d_ff].
// FFN_i of the DeepSeek-V3 explainer's equation for h'_t (method section 2), gated
// SiLU form.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int expert_of_row(const int32_t* offset, int n_r, int64_t r) {
  int lo = 0, hi = n_r - 1;  // last expert with offset[e] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (offset[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void gate_up_f32(
    const float* __restrict__ u, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ sorted_token, const float* __restrict__ w1r,
    const float* __restrict__ w3r, const float* __restrict__ w1s, const float* __restrict__ w3s,
    int64_t T, int d, int d_ff, int n_r, int K, int n_s, float* __restrict__ h) {
  const int64_t P = T * K;
  const int64_t rows = P + T * n_s;
  const int64_t total = rows * d_ff;
  for (int64_t o = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; o < total;
       o += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t r = o / d_ff;
    const int n = static_cast<int>(o % d_ff);
    const float *x, *a, *b;
    float* dst;
    if (r < P) {
      const int e = expert_of_row(offset, n_r, r);
      x = u + static_cast<int64_t>(sorted_token[r]) * d;
      a = w1r + (static_cast<int64_t>(e) * d_ff + n) * d;
      b = w3r + (static_cast<int64_t>(e) * d_ff + n) * d;
      dst = h + r * d_ff + n;
    } else {
      const int64_t q = r - P;
      const int j = static_cast<int>(q / T);
      const int64_t t = q % T;
      x = u + t * d;
      a = w1s + (static_cast<int64_t>(j) * d_ff + n) * d;
      b = w3s + (static_cast<int64_t>(j) * d_ff + n) * d;
      dst = h + P * d_ff + t * (static_cast<int64_t>(n_s) * d_ff) + static_cast<int64_t>(j) * d_ff + n;
    }
    float za = 0.0f, zb = 0.0f;
    for (int c = 0; c < d; ++c) {
      za = fmaf(x[c], a[c], za);
      zb = fmaf(x[c], b[c], zb);
    }
    *dst = za / (1.0f + expf(-za)) * zb;
  }
}

__global__ __launch_bounds__(kThreads) void down_f32(
    const float* __restrict__ h, const int32_t* __restrict__ offset, const float* __restrict__ w2r,
    const float* __restrict__ w2s, int64_t T, int d, int d_ff, int n_r, int K, int n_s,
    float* __restrict__ y_routed, float* __restrict__ y_shared) {
  const int64_t P = T * K;
  const int64_t total = (P + (n_s > 0 ? T : 0)) * d;  // no shared rows (and no y_shared) when n_s = 0
  for (int64_t o = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; o < total;
       o += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t r = o / d;
    const int n = static_cast<int>(o % d);
    if (r < P) {
      const int e = expert_of_row(offset, n_r, r);
      const float* hr = h + r * d_ff;
      const float* w = w2r + (static_cast<int64_t>(e) * d + n) * d_ff;
      float z = 0.0f;
      for (int j = 0; j < d_ff; ++j) z = fmaf(hr[j], w[j], z);
      y_routed[r * d + n] = z;
    } else {
      const int64_t t = r - P;
      const float* hr = h + P * d_ff + t * (static_cast<int64_t>(n_s) * d_ff);
      float z = 0.0f;
      for (int s = 0; s < n_s; ++s) {
        const float* w = w2s + (static_cast<int64_t>(s) * d + n) * d_ff;
        for (int j = 0; j < d_ff; ++j) z = fmaf(hr[s * d_ff + j], w[j], z);
      }
      y_shared[t * d + n] = z;
    }
  }
}

int grid_for(int64_t total) {
  int64_t g = (total + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  return static_cast<int>(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_ffn_f32(const float* u, const int32_t* offset, const int32_t* sorted_token,
                          const float* w1r, const float* w3r, const float* w2r, const float* w1s,
                          const float* w3s, const float* w2s, int64_t T, int d, int d_ff, int n_r,
                          int K, int n_s, float* h, float* y_routed, float* y_shared,
                          hipStream_t stream) {
  const int64_t P = T * K;
  hipLaunchKernelGGL(gate_up_f32, dim3(grid_for((P + T * n_s) * d_ff)), dim3(kThreads), 0, stream, u,
                     offset, sorted_token, w1r, w3r, w1s, w3s, T, d, d_ff, n_r, K, n_s, h);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(down_f32, dim3(grid_for((P + (n_s > 0 ? T : 0)) * d)), dim3(kThreads), 0, stream, h, offset,
                     w2r, w2s, T, d, d_ff, n_r, K, n_s, y_routed, y_shared);
  return hipGetLastError();
}

}  // namespace moe

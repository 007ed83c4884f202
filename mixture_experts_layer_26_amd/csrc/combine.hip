// Combine and bias update.
//
// combine: h'_t = u_t + (shared sum)_t + sum_k g_{k,t} * y_routed[pair_row[t,k]], the
// DeepSeek-V3 explainer's equation for h'_t (method section 2), as a gather over the
// token's K sorted rows (no atomics), added in fp32 in the order residual, shared,
// routed experts ascending, and rounded once to the output dtype. One workgroup per
// token with one thread per 16-byte vector of the row (up to 1024). A thread issues the
// loads of all K routed rows before it adds the first (K <= 16, unrolled), so they are in
// flight together instead of one latency per row.
//
// bias update: the same section's end-of-step rule, b_i -= gamma when expert i's load
// is above the mean T*K/N_r, += gamma when below, compared exactly in integers.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {


template <int ACT>  // 0: fp32 in/out (4 per vector), 1: bf16 (8 per vector)
__global__ __launch_bounds__(1024) void combine_kernel(
    const void* __restrict__ u, const void* __restrict__ y_routed, const float* __restrict__ y_shared,
    const int32_t* __restrict__ pair_row, const float* __restrict__ gate, void* __restrict__ out,
    int64_t T, int d, int K) {
  constexpr int V = ACT == 1 ? 8 : 4;
  __shared__ int32_t rows[16];
  __shared__ float gs[16];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) {
    rows[threadIdx.x] = pair_row[t * K + threadIdx.x];
    gs[threadIdx.x] = gate[t * K + threadIdx.x];
  }
  __syncthreads();
  for (int c0 = threadIdx.x * V; c0 < d; c0 += blockDim.x * V) {
    // every load of this vector first: the residual, the shared sum, the K routed rows
    const uint4 uv = ACT == 1 ? ld16(static_cast<const uint16_t*>(u) + t * d + c0)
                              : ld16(static_cast<const float*>(u) + t * d + c0);
    float4 sv[V / 4];
    if (y_shared) {
#pragma unroll
      for (int q = 0; q < V / 4; ++q) sv[q] = *reinterpret_cast<const float4*>(y_shared + t * d + c0 + 4 * q);
    }
    uint4 yv[16];  // the K routed rows' vectors (bf16: 8 values; fp32: 4)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K) {
        const int64_t r = rows[k];
        yv[k] = ACT == 1 ? ld16(static_cast<const uint16_t*>(y_routed) + r * d + c0)
                         : ld16(static_cast<const float*>(y_routed) + r * d + c0);
      }
    }
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q)
      acc[q] = ACT == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(&uv)[q]) : reinterpret_cast<const float*>(&uv)[q];
    if (y_shared) {
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        acc[4 * q] += sv[q].x; acc[4 * q + 1] += sv[q].y; acc[4 * q + 2] += sv[q].z; acc[4 * q + 3] += sv[q].w;
      }
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k < K) {
        const float g = gs[k];
        if (ACT == 1) {
          const uint16_t* yp = reinterpret_cast<const uint16_t*>(&yv[k]);
#pragma unroll
          for (int q = 0; q < V; ++q) acc[q] = fmaf(g, bf16_to_f32(yp[q]), acc[q]);
        } else {
          const float* yp = reinterpret_cast<const float*>(&yv[k]);
#pragma unroll
          for (int q = 0; q < V; ++q) acc[q] = fmaf(g, yp[q], acc[q]);
        }
      }
    }
    if (ACT == 1) {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      st16(static_cast<uint16_t*>(out) + t * d + c0, o);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(out) + t * d + c0) =
          make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

__global__ void zero_i32_kernel(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ void bias_update_kernel(const int32_t* __restrict__ count, int64_t total, int n_r,
                                   float gamma, float* __restrict__ bias) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_r) return;
  const int64_t load = static_cast<int64_t>(count[i]) * n_r;
  if (load > total)
    bias[i] = bias[i] - gamma;
  else if (load < total)
    bias[i] = bias[i] + gamma;
}

}  // namespace

hipError_t launch_combine(int act, const void* u, const void* y_routed, const float* y_shared,
                          const int32_t* pair_row, const float* gate, void* out, int64_t T, int d,
                          int K, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(T));
  const int V = act == 1 ? 8 : 4;
  int thr = (d / V + 63) / 64 * 64;
  thr = thr > 1024 ? 1024 : (thr < 64 ? 64 : thr);
  if (act == 1)
    hipLaunchKernelGGL(combine_kernel<1>, grid, dim3(thr), 0, stream, u, y_routed, y_shared,
                       pair_row, gate, out, T, d, K);
  else
    hipLaunchKernelGGL(combine_kernel<0>, grid, dim3(thr), 0, stream, u, y_routed, y_shared,
                       pair_row, gate, out, T, d, K);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int* p, int n, hipStream_t stream) {
  const int blocks = n <= 0 ? 1 : (n + 255) / 256 < 256 ? (n + 255) / 256 : 256;
  hipLaunchKernelGGL(zero_i32_kernel, dim3(blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* count, int64_t T, int n_r, int K, float gamma,
                              float* bias, hipStream_t stream) {
  hipLaunchKernelGGL(bias_update_kernel, dim3((n_r + 255) / 256), dim3(256), 0, stream, count,
                     T * K, n_r, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe

// Backward of the combine and of the router (bf16 activations).
//
// The layer (DeepSeek-V3 explainer, method section 2) is h'_t = u_t + sum_j FFN^(s)_j(u_t)
// + sum_k g_{k,t} FFN^(r)_{i_k}(u_t), and its gradient with the selection held fixed:
//   combine: dy_{k,t} = g_{k,t} dout_t (the routed rows' output gradient, bf16 in sorted
//            row order) and dg_{k,t} = dout_t . y_{k,t};
//   router:  sigmoid gates g_k = s_k / S (the bias only selects, so it has no gradient):
//            dz_k = (dg_k - sum_j g_j dg_j) / S * s_k (1 - s_k); softmax gates (the
//            deepseekmodel.com forward listing): dz_k = g_k (dg_k - sum_j g_j dg_j);
//   input:   du_t = dout_t + shared dx_t + sum_k dx_{k,t} + sum_k dz_k e_{i_k}, added in
//            that order in fp32 and rounded once; de_i = sum over i's rows (tokens
//            ascending) of dz u_t.
// The logits of the selected experts are recomputed in fp32 (dot products over d).
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 16;

// Sum of one value per thread over the workgroup, in a fixed order (waves ascending).
__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = x;
  __syncthreads();
  float s = 0.0f;
  for (int i = 0; i < kThreads / kWave; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ void unpack8(uint4 v, float (&f)[8]) {
  const uint16_t* p = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
  for (int q = 0; q < 8; ++q) f[q] = bf16_to_f32(p[q]);
}

// One workgroup per token.
__global__ __launch_bounds__(kThreads) void combine_backward_kernel(
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ y_routed, const int32_t* __restrict__ pair_row,
    const float* __restrict__ gate, uint16_t* __restrict__ dy_routed, float* __restrict__ dgate, int d, int K) {
  __shared__ int32_t rows[kMaxK];
  __shared__ float gs[kMaxK];
  __shared__ float red[kThreads / kWave];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) {
    rows[threadIdx.x] = pair_row[t * K + threadIdx.x];
    gs[threadIdx.x] = gate[t * K + threadIdx.x];
  }
  __syncthreads();
  float part[kMaxK];
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) part[k] = 0.0f;
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += kThreads * 8) {
    float o[8];
    unpack8(ld16(dout + t * d + c0), o);
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      if (k >= K) break;
      const int64_t r = rows[k];
      float y[8];
      unpack8(ld16(y_routed + r * d + c0), y);
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) s = fmaf(o[q], y[q], s);
      part[k] += s;
      uint4 dy;
      dy.x = pack_bf16x2(gs[k] * o[0], gs[k] * o[1]);
      dy.y = pack_bf16x2(gs[k] * o[2], gs[k] * o[3]);
      dy.z = pack_bf16x2(gs[k] * o[4], gs[k] * o[5]);
      dy.w = pack_bf16x2(gs[k] * o[6], gs[k] * o[7]);
      st16(dy_routed + r * d + c0, dy);
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxK; ++k) {  // K is uniform: every thread takes the same barriers
    if (k >= K) break;
    const float s = block_sum(part[k], red);
    if (threadIdx.x == 0) dgate[t * K + k] = s;
  }
}

// One workgroup per token: dz of the K picks, then du.
template <int SCORE>
__global__ __launch_bounds__(kThreads) void route_backward_kernel(
    const uint16_t* __restrict__ u, const uint16_t* __restrict__ e, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dgate, const int32_t* __restrict__ pair_row,
    const uint16_t* __restrict__ dout, const uint16_t* __restrict__ dx_routed, const float* __restrict__ dx_shared,
    uint16_t* __restrict__ du, float* __restrict__ dz_out, float* __restrict__ dz_sorted, int d, int K) {
  __shared__ int32_t ids[kMaxK], rows[kMaxK];
  __shared__ float dzs[kMaxK];
  __shared__ float zs[kMaxK];
  __shared__ float red[kThreads / kWave];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) {
    ids[threadIdx.x] = idx[t * K + threadIdx.x];
    rows[threadIdx.x] = pair_row[t * K + threadIdx.x];
  }
  __syncthreads();
  if (SCORE == 0) {  // logits of the picks
    float part[kMaxK];
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) part[k] = 0.0f;
    for (int c0 = threadIdx.x * 8; c0 < d; c0 += kThreads * 8) {
      float x[8];
      unpack8(ld16(u + t * d + c0), x);
#pragma unroll
      for (int k = 0; k < kMaxK; ++k) {
        if (k >= K) break;
        float ev[8];
        unpack8(ld16(e + static_cast<int64_t>(ids[k]) * d + c0), ev);
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) s = fmaf(x[q], ev[q], s);
        part[k] += s;
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {  // K is uniform: every thread takes the same barriers
      if (k >= K) break;
      const float s = block_sum(part[k], red);
      if (threadIdx.x == 0) zs[k] = s;
    }
  }
  if (threadIdx.x == 0) {
    // sigmoid: s_k from the recomputed logits, S = sum s_k, g_k = s_k / S; softmax: the gates
    float S = 0.0f;
    if (SCORE == 0)
      for (int k = 0; k < K; ++k) {
        zs[k] = 1.0f / (1.0f + expf(-zs[k]));  // zs now holds s_k
        S += zs[k];
      }
    float gbar = 0.0f;
    for (int k = 0; k < K; ++k) gbar += (SCORE == 0 ? zs[k] / S : gate[t * K + k]) * dgate[t * K + k];
    for (int k = 0; k < K; ++k) {
      const float dg = dgate[t * K + k] - gbar;
      const float dz = SCORE == 0 ? dg / S * zs[k] * (1.0f - zs[k]) : gate[t * K + k] * dg;
      dzs[k] = dz;
      dz_out[t * K + k] = dz;
      dz_sorted[rows[k]] = dz;
    }
  }
  __syncthreads();
  for (int c0 = threadIdx.x * 8; c0 < d; c0 += kThreads * 8) {
    float acc[8];
    unpack8(ld16(dout + t * d + c0), acc);
    if (dx_shared) {
#pragma unroll
      for (int q = 0; q < 8; q += 4) {
        const float4 s = *reinterpret_cast<const float4*>(dx_shared + t * d + c0 + q);
        acc[q] += s.x; acc[q + 1] += s.y; acc[q + 2] += s.z; acc[q + 3] += s.w;
      }
    }
    for (int k = 0; k < K; ++k) {
      float x[8];
      unpack8(ld16(dx_routed + static_cast<int64_t>(rows[k]) * d + c0), x);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += x[q];
    }
    for (int k = 0; k < K; ++k) {
      float ev[8];
      unpack8(ld16(e + static_cast<int64_t>(ids[k]) * d + c0), ev);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(dzs[k], ev[q], acc[q]);
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    st16(du + t * d + c0, o);
  }
}

// de_i = sum over expert i's sorted rows of dz u_t; grid (n_r, ceil(d / 2048)).
__global__ __launch_bounds__(kThreads) void centroid_grad_kernel(
    const uint16_t* __restrict__ u, const int32_t* __restrict__ offset, const int32_t* __restrict__ sorted_token,
    const float* __restrict__ dz_sorted, uint16_t* __restrict__ de, int d) {
  const int i = blockIdx.x;
  const int c0 = (blockIdx.y * kThreads + threadIdx.x) * 8;
  if (c0 >= d) return;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  const int r1 = offset[i + 1];
  for (int r = offset[i]; r < r1; ++r) {
    const float z = dz_sorted[r];
    float x[8];
    unpack8(ld16(u + static_cast<int64_t>(sorted_token[r]) * d + c0), x);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(z, x[q], acc[q]);
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  st16(de + static_cast<int64_t>(i) * d + c0, o);
}

}  // namespace

hipError_t launch_combine_backward(const void* dout, const void* y_routed, const int32_t* pair_row,
                                   const float* gate, void* dy_routed, float* dgate, int64_t T, int d, int K,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(combine_backward_kernel, dim3(static_cast<unsigned>(T)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(y_routed), pair_row, gate,
                     static_cast<uint16_t*>(dy_routed), dgate, d, K);
  return hipGetLastError();
}

hipError_t launch_route_backward(int score, const void* u, const void* e, const int32_t* idx, const float* gate,
                                 const float* dgate, const int32_t* offset, const int32_t* sorted_token,
                                 const int32_t* pair_row, const void* dout, const void* dx_routed,
                                 const float* dx_shared, void* du, void* de, float* dz, float* dz_sorted,
                                 int64_t T, int d, int n_r, int K, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(T));
  const uint16_t* u16 = static_cast<const uint16_t*>(u);
  const uint16_t* e16 = static_cast<const uint16_t*>(e);
  if (score == 1)
    hipLaunchKernelGGL(route_backward_kernel<1>, grid, dim3(kThreads), 0, stream, u16, e16, idx, gate, dgate,
                       pair_row, static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(dx_routed),
                       dx_shared, static_cast<uint16_t*>(du), dz, dz_sorted, d, K);
  else
    hipLaunchKernelGGL(route_backward_kernel<0>, grid, dim3(kThreads), 0, stream, u16, e16, idx, gate, dgate,
                       pair_row, static_cast<const uint16_t*>(dout), static_cast<const uint16_t*>(dx_routed),
                       dx_shared, static_cast<uint16_t*>(du), dz, dz_sorted, d, K);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 g2(static_cast<unsigned>(n_r), static_cast<unsigned>((d + kThreads * 8 - 1) / (kThreads * 8)));
  hipLaunchKernelGGL(centroid_grad_kernel, g2, dim3(kThreads), 0, stream, u16, offset, sorted_token, dz_sorted,
                     static_cast<uint16_t*>(de), d);
  return hipGetLastError();
}

}  // namespace moe

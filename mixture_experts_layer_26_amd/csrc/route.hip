// Router: s = Sigmoid(u . e_i), top-K of s + b with the lower index first on ties,
// gates = selected s normalised over the selection.
// DeepSeek-V3 explainer (xyznot.com), method section 2: the sigmoid affinity and the
// equation for g'_{i,t}; gates normalise g'.
//
// One workgroup of 4 waves owns 32 tokens and every expert. Logits come from bf16
// MFMA 32x32x16 (fp32 accumulate) straight from global memory: each wave takes two
// 32-expert blocks in one K loop; the 32 x N_r sigmoid scores are parked in LDS, then each wave
// selects the top-K of 8 tokens with 64-bit (score, ~index) keys reduced across the
// wave. For fp32 activations the logits are plain fp32 FMA dot products.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kTok = 32;
constexpr int kThreads = 256;
constexpr int kMaxExperts = 256;

__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), off, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), off, kWave);
    uint64_t y = (static_cast<uint64_t>(hi) << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}

__device__ __forceinline__ float sigmoid_precise(float z) { return 1.0f / (1.0f + expf(-z)); }

// logits of 32 tokens x n_r experts, bf16 inputs, into sc[32][n_r] as sigmoid scores.
// Wave w owns expert blocks w and w + 4 (32 experts each) and runs both in one K loop,
// so each u fragment is loaded once per wave. K advances in chunks of KC*16 with the
// next chunk's loads in flight while the current chunk's MFMAs run.
template <int KC>
__device__ void logits_bf16_kc(const uint16_t* __restrict__ u, const uint16_t* __restrict__ e,
                               int64_t T, int d, int n_r, int64_t t0, float* sc) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int r = lane % 32, kh = (lane / 32) * 8;
  int64_t trow = t0 + r;
  if (trow >= T) trow = T - 1;
  const uint16_t* ap = u + trow * d + kh;
  const int nblk = (n_r + 31) / 32;
  const bool two = wave + 4 < nblk;
  if (wave >= nblk) return;
  int e0 = wave * 32 + r, e1 = (wave + 4) * 32 + r;
  if (e0 >= n_r) e0 = n_r - 1;
  if (e1 >= n_r) e1 = n_r - 1;
  const uint16_t* bp0 = e + static_cast<int64_t>(e0) * d + kh;
  const uint16_t* bp1 = e + static_cast<int64_t>(two ? e1 : e0) * d + kh;
  f32x16 acc0 = {}, acc1 = {};
  uint4 a[KC], b0[KC], b1[KC];
  auto load = [&](int k0) {
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      a[s] = ld16(ap + k0 + s * 16);
      b0[s] = ld16(bp0 + k0 + s * 16);
      b1[s] = ld16(bp1 + k0 + s * 16);
    }
  };
  load(0);
  for (int k0 = 0; k0 < d; k0 += KC * 16) {
    uint4 ca[KC], cb0[KC], cb1[KC];
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      ca[s] = a[s];
      cb0[s] = b0[s];
      cb1[s] = b1[s];
    }
    if (k0 + KC * 16 < d) load(k0 + KC * 16);
#pragma unroll
    for (int s = 0; s < KC; ++s) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ca[s]),
                                                     __builtin_bit_cast(bf16x8, cb0[s]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ca[s]),
                                                     __builtin_bit_cast(bf16x8, cb1[s]), acc1, 0, 0, 0);
    }
  }
  // C layout of 32x32 MFMA: lane holds column (expert) lane%32, rows 8*(v/4)+4*(lane/32)+v%4
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk == 1 && !two) break;
    const int j = (wave + 4 * blk) * 32 + (lane % 32);
    if (j < n_r) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
        sc[i * n_r + j] = sigmoid_precise(blk == 0 ? acc0[v] : acc1[v]);
      }
    }
  }
}

__device__ void logits_bf16(const uint16_t* __restrict__ u, const uint16_t* __restrict__ e,
                            int64_t T, int d, int n_r, int64_t t0, float* sc) {
  if (d % 128 == 0)
    logits_bf16_kc<8>(u, e, T, d, n_r, t0, sc);
  else
    logits_bf16_kc<4>(u, e, T, d, n_r, t0, sc);
}

__device__ void logits_f32(const float* __restrict__ u, const float* __restrict__ e, int64_t T,
                           int d, int n_r, int64_t t0, float* sc) {
  for (int p = threadIdx.x; p < kTok * n_r; p += kThreads) {
    const int i = p / n_r, j = p % n_r;
    int64_t t = t0 + i;
    if (t >= T) t = T - 1;
    const float* a = u + t * d;
    const float* b = e + static_cast<int64_t>(j) * d;
    float z = 0.0f;
    for (int c = 0; c < d; ++c) z = fmaf(a[c], b[c], z);
    sc[i * n_r + j] = sigmoid_precise(z);
  }
}

template <int ACT>
__global__ __launch_bounds__(kThreads) void route_kernel(const void* __restrict__ u,
                                                         const void* __restrict__ e,
                                                         const float* __restrict__ bias, int64_t T,
                                                         int d, int n_r, int K,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_gate) {
  __shared__ float sc[kTok * kMaxExperts];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  if (ACT == 1)
    logits_bf16(static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(e), T, d, n_r, t0, sc);
  else
    logits_f32(static_cast<const float*>(u), static_cast<const float*>(e), T, d, n_r, t0, sc);
  __syncthreads();

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // this lane's candidates: experts lane, lane+64, lane+128, lane+192
  float bl[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = lane + 64 * c;
    bl[c] = j < n_r ? bias[j] : 0.0f;
  }
  for (int i = wave; i < kTok; i += 4) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    uint64_t key[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = lane + 64 * c;
      key[c] = 0;  // below every real key
      if (j < n_r) {
        const float v = sc[i * n_r + j] + bl[c];
        key[c] = (static_cast<uint64_t>(orderable(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(j));
      }
    }
    int sel[16];
    for (int k = 0; k < K; ++k) {
      uint64_t best = key[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
      const int j = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
      sel[k] = j;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (lane + 64 * c == j) key[c] = 0;
    }
    // ascending expert ids (insertion sort; identical in every lane)
    for (int a = 1; a < K; ++a) {
      const int x = sel[a];
      int b = a - 1;
      while (b >= 0 && sel[b] > x) {
        sel[b + 1] = sel[b];
        --b;
      }
      sel[b + 1] = x;
    }
    float denom = 0.0f;
    for (int k = 0; k < K; ++k) denom += sc[i * n_r + sel[k]];
    if (lane < K) {
      int myj = sel[0];
      for (int k = 1; k < K; ++k)
        if (k == lane) myj = sel[k];
      topk_idx[t * K + lane] = myj;
      topk_gate[t * K + lane] = sc[i * n_r + myj] / denom;
    }
  }
}

}  // namespace

hipError_t launch_route(int act, const void* u, const void* e, const float* bias, int64_t T, int d,
                        int n_r, int K, int32_t* idx, float* gate, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((T + kTok - 1) / kTok));
  if (act == 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, dim3(kThreads), 0, stream, u, e, bias, T, d, n_r, K,
                       idx, gate);
  else
    hipLaunchKernelGGL(route_kernel<0>, grid, dim3(kThreads), 0, stream, u, e, bias, T, d, n_r, K,
                       idx, gate);
  return hipGetLastError();
}

}  // namespace moe

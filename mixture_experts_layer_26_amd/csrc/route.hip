// Router: s = Sigmoid(u . e_i), top-K of s + b with the lower index first on ties,
// gates = selected s normalised over the selection.
// DeepSeek-V3 explainer (xyznot.com), method section 2: the sigmoid affinity and the
// equation for g'_{i,t}; gates normalise g'.
//
// One workgroup of 8 waves owns 32 tokens and every expert. Logits come from bf16
// MFMA 32x32x16 (fp32 accumulate) straight from global memory: each wave takes two
// 32-expert blocks over half of K; the 32 x N_r sigmoid scores are parked in LDS, then
// each wave selects the top-K of 4 tokens with 64-bit (score, ~index) keys reduced
// across the wave. For fp32 activations the logits are plain fp32 FMA dot products.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kTok = 32;
constexpr int kThreads = 512;
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
// 8 waves: wave w owns expert blocks (w%4) and (w%4)+4 (32 experts each) over half of
// the K range (w/4), running both blocks in one loop so each u fragment is loaded once.
// K advances in chunks of KC*16 with the next chunk's loads in flight. The two K
// halves meet in LDS and are added in a fixed order (first half + second half).
template <int KC>
__device__ void logits_bf16_kc(const uint16_t* __restrict__ u, const uint16_t* __restrict__ e,
                               int64_t T, int d, int n_r, int64_t t0, float* sc, float* part) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int bp = wave % 4, kh = wave / 4;
  const int r = lane % 32, koff = (lane / 32) * 8;
  int64_t trow = t0 + r;
  if (trow >= T) trow = T - 1;
  const int nblk = (n_r + 31) / 32;
  const bool active = bp < nblk;
  const bool two = bp + 4 < nblk;
  const int khalf = d / 2;  // d % (2 * KC * 16) == 0 (host check)
  const uint16_t* ap = u + trow * d + koff + kh * khalf;
  int e0 = bp * 32 + r, e1 = (bp + 4) * 32 + r;
  if (e0 >= n_r) e0 = n_r - 1;
  if (e1 >= n_r) e1 = n_r - 1;
  if (!two) e1 = e0;
  const uint16_t* bp0 = e + static_cast<int64_t>(e0) * d + koff + kh * khalf;
  const uint16_t* bp1 = e + static_cast<int64_t>(e1) * d + koff + kh * khalf;
  f32x16 acc0 = {}, acc1 = {};
  if (active) {
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
    for (int k0 = 0; k0 < khalf; k0 += KC * 16) {
      uint4 ca[KC], cb0[KC], cb1[KC];
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        ca[s] = a[s];
        cb0[s] = b0[s];
        cb1[s] = b1[s];
      }
      if (k0 + KC * 16 < khalf) load(k0 + KC * 16);
#pragma unroll
      for (int s = 0; s < KC; ++s) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ca[s]),
                                                       __builtin_bit_cast(bf16x8, cb0[s]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ca[s]),
                                                       __builtin_bit_cast(bf16x8, cb1[s]), acc1, 0, 0, 0);
      }
    }
  }
  // C layout of 32x32 MFMA: lane holds column (expert) lane%32, rows 8*(v/4)+4*(lane/32)+v%4
  auto store = [&](float* dst, bool sig) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      if (!active || (blk == 1 && !two)) continue;
      const int j = (bp + 4 * blk) * 32 + (lane % 32);
      if (j >= n_r) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
        const float z = blk == 0 ? acc0[v] : acc1[v];
        if (sig)
          dst[i * n_r + j] = sigmoid_precise(dst[i * n_r + j] + z);  // first half + second half
        else
          dst[i * n_r + j] = z;
      }
    }
  };
  if (kh == 0) store(part, false);
  __syncthreads();
  if (kh == 1) store(part, true);
  __syncthreads();
  for (int p = threadIdx.x; p < kTok * n_r; p += kThreads) sc[p] = part[p];
}

__device__ void logits_bf16(const uint16_t* __restrict__ u, const uint16_t* __restrict__ e,
                            int64_t T, int d, int n_r, int64_t t0, float* sc, float* part) {
  if (d % 256 == 0)
    logits_bf16_kc<8>(u, e, T, d, n_r, t0, sc, part);
  else
    logits_bf16_kc<2>(u, e, T, d, n_r, t0, sc, part);
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
  __shared__ float part[kTok * kMaxExperts];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTok;
  if (ACT == 1)
    logits_bf16(static_cast<const uint16_t*>(u), static_cast<const uint16_t*>(e), T, d, n_r, t0, sc, part);
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
  for (int i = wave; i < kTok; i += kThreads / kWave) {
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
    // lane k < K keeps the k-th pick; no per-lane arrays indexed at run time
    int mysel = 0x7FFFFFFF;
    for (int k = 0; k < K; ++k) {
      uint64_t best = key[0];
#pragma unroll
      for (int c = 1; c < 4; ++c) best = key[c] > best ? key[c] : best;
      best = wave_max_u64(best);
      const int j = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
      if (lane == k) mysel = j;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (lane + 64 * c == j) key[c] = 0;
    }
    // position of each pick in ascending expert order
    int rank = 0;
    for (int k = 0; k < K; ++k) rank += __shfl(mysel, k, kWave) < mysel ? 1 : 0;
    // gate denominator: the picked scores summed in ascending expert order
    const float myv = lane < K ? sc[i * n_r + mysel] : 0.0f;
    float denom = 0.0f;
    for (int p = 0; p < K; ++p) {
      const uint64_t m = __ballot(lane < K && rank == p);
      denom += __shfl(myv, __ffsll(static_cast<unsigned long long>(m)) - 1, kWave);
    }
    if (lane < K) {
      topk_idx[t * K + rank] = mysel;
      topk_gate[t * K + rank] = myv / denom;
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

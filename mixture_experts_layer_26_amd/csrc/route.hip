// Router: s = Sigmoid(u . e_i), top-K of s + b with the lower index first on ties,
// gates = selected s normalised over the selection.
// DeepSeek-V3 explainer (xyznot.com), method section 2: the sigmoid affinity and the
// equation for g'_{i,t}; gates normalise g'.
// Softmax scoring (the DeepSeekMoE forward listing of deepseekmodel.com): top-K of the
// logits z themselves, no bias, gates = softmax of the selected logits.
//
// bf16 activations take two kernels. route_logits: a workgroup owns 128 tokens x 256
// experts over one chunk of K (the grid splits K so that it fills the chip even for a
// small batch), stages u and e through swizzled LDS in steps of 64 and accumulates with
// bf16 MFMA 32x32x16 in fp32; it writes the chunk's partial logits. route_topk: one
// wave per token adds the chunks' partials in chunk order, takes the sigmoid and
// selects the top-K with 64-bit (score, ~index) keys reduced across the wave. fp32
// activations take one kernel (route_kernel): fp32 dot products from LDS-staged chunks of u
// and e, then the same selection.
#include "gemm_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kTokF32 = 8;  // tokens per workgroup of the fp32 router: one per wave
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

// Top-K of one token held by one wave: lane l holds the keys and scores of experts
// l + 64 c (c = 0..3; key 0 = no expert). Lane k < K keeps the k-th pick (no per-lane
// array is indexed at run time); picks are written in ascending expert order with
// gates = score / (sum of the picked scores, added in ascending expert order). With
// SOFTMAX the scores are the logits and each picked one becomes expf(z - z_max) first;
// the first pick has the largest key, so its logit is z_max.
template <bool SOFTMAX>
__device__ __forceinline__ void topk_select(uint64_t (&key)[4], const float (&sv)[4], int lane, int K,
                                            int32_t* __restrict__ idx, float* __restrict__ gate) {
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
  // the pick's score lives in lane mysel % 64, slot mysel / 64
  const int src = (lane < K ? mysel : 0) & 63, slot = (lane < K ? mysel : 0) >> 6;
  float v0 = __shfl(sv[0], src, kWave), v1 = __shfl(sv[1], src, kWave);
  float v2 = __shfl(sv[2], src, kWave), v3 = __shfl(sv[3], src, kWave);
  float myv = lane < K ? (slot == 0 ? v0 : slot == 1 ? v1 : slot == 2 ? v2 : v3) : 0.0f;
  if (SOFTMAX) {
    const float zmax = __shfl(myv, 0, kWave);
    myv = lane < K ? expf(myv - zmax) : 0.0f;
  }
  float denom = 0.0f;
  for (int p = 0; p < K; ++p) {
    const uint64_t m = __ballot(lane < K && rank == p);
    denom += __shfl(myv, __ffsll(static_cast<unsigned long long>(m)) - 1, kWave);
  }
  if (lane < K) {
    idx[rank] = mysel;
    gate[rank] = myv / denom;
  }
}

// ---------------------------------------------------------------------------- bf16
constexpr int kTB = 128;   // tokens per logits workgroup
constexpr int kEB = 256;   // experts per logits workgroup (all of them, n_r <= 256)
constexpr int kLK = 64;    // K per LDS stage (128-byte rows)

// Partial logits of tokens t0.. (128) x experts 0..255 over K-steps [k0, k1) of 64:
// part[chunk][t][j]. Waves: token block w % 4 (32 tokens), expert half w / 4 (4 blocks
// of 32 experts). Rows past T or n_r repeat a valid row and are not stored.
__global__ __launch_bounds__(kThreads) void route_logits(const uint16_t* __restrict__ u,
                                                         const uint16_t* __restrict__ e, int64_t T, int d,
                                                         int n_r, int steps_per_chunk,
                                                         float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) unsigned char su[2][kTB * 128];
  __shared__ __attribute__((aligned(16))) unsigned char se[2][kEB * 128];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTB;
  const int chunk = blockIdx.y;
  const int nsteps = d / kLK;
  const int k0 = chunk * steps_per_chunk;
  const int k1 = k0 + steps_per_chunk < nsteps ? k0 + steps_per_chunk : nsteps;
  // loads: u tile 128 rows x 8 chunks (2 per thread), e tile 256 rows x 8 (4 per thread)
  const int cc = tid % 8, cr = tid / 8;  // 16-byte chunk, row 0..63
  const uint16_t* ua[2];
  const uint16_t* ea[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int64_t t = t0 + cr + 64 * i;
    if (t >= T) t = T - 1;
    ua[i] = u + t * d + cc * 8;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int j = cr + 64 * i;
    if (j >= n_r) j = n_r - 1;
    ea[i] = e + static_cast<int64_t>(j) * d + cc * 8;
  }
  uint4 ru[2], re[4];
  auto gload = [&](int kt) {
    const int64_t off = static_cast<int64_t>(kt) * kLK;
#pragma unroll
    for (int i = 0; i < 2; ++i) ru[i] = ld16(ua[i] + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) re[i] = ld16(ea[i] + off);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(su[st] + gemm::swz(cr + 64 * i, cc)) = ru[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(se[st] + gemm::swz(cr + 64 * i, cc)) = re[i];
  };
  const int tb = wave % 4, eh = wave / 4;
  const int arow = 32 * tb + lane % 32;
  f32x16 acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x16{};
  if (k0 < k1) {
    gload(k0);
    lstore(0);
    __syncthreads();
    for (int kt = k0; kt < k1; ++kt) {
      const int cur = (kt - k0) & 1;
      if (kt + 1 < k1) gload(kt + 1);
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) {
        const int ch = 2 * sub + lane / 32;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(su[cur] + gemm::swz(arow, ch));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bf16x8 w = *reinterpret_cast<const bf16x8*>(se[cur] + gemm::swz(128 * eh + 32 * b + lane % 32, ch));
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w, acc[b], 0, 0, 0);
        }
      }
      if (kt + 1 < k1) lstore(cur ^ 1);
      __syncthreads();
    }
  }
  // C layout of 32x32 MFMA: lane holds column (expert) lane%32, rows 8*(v/4)+4*(lane/32)+v%4
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int j = 128 * eh + 32 * b + lane % 32;
    if (j >= n_r) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t t = t0 + 32 * tb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
      if (t < T) part[(static_cast<int64_t>(chunk) * T + t) * n_r + j] = acc[b][v];
    }
  }
}

// Selection key and score of one expert from its logit z.
template <int SCORE>
__device__ __forceinline__ void score_key(float z, const float* __restrict__ bias, int j, float& sv, uint64_t& key) {
  float v;
  if (SCORE == 1) {
    sv = z;
    v = z;
  } else {
    sv = sigmoid_precise(z);
    v = sv + bias[j];
  }
  key = (static_cast<uint64_t>(orderable(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(j));
}

constexpr int kSumBatch = 8;  // partial logits a lane loads before adding them

// Top-K of one token per wave from the partial logits of n_chunks chunks.
template <int SCORE>
__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ part, int n_chunks,
                                                  const float* __restrict__ bias, int64_t T, int n_r, int K,
                                                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  const int lane = threadIdx.x % kWave;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  // this lane's candidates: experts lane, lane+64, lane+128, lane+192. Their logits are the
  // chunks' partials added in chunk order; each batch of kSumBatch chunks is loaded for all
  // four candidates before the first of its additions, so those loads are in flight together.
  float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int q0 = 0; q0 < n_chunks; q0 += kSumBatch) {
    float pv[4][kSumBatch];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < kSumBatch; ++i)
        if (lane + 64 * c < n_r && q0 + i < n_chunks)
          pv[c][i] = part[(static_cast<int64_t>(q0 + i) * T + t) * n_r + lane + 64 * c];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < kSumBatch; ++i)
        if (lane + 64 * c < n_r && q0 + i < n_chunks) z[c] += pv[c][i];
  }
  float sv[4];
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int j = lane + 64 * c;
    sv[c] = 0.0f;
    key[c] = 0;  // below every real key
    if (j < n_r) score_key<SCORE>(z[c], bias, j, sv[c], key[c]);
  }
  topk_select<SCORE == 1>(key, sv, lane, K, topk_idx + t * K, topk_gate + t * K);
}

// fp32 logits of the workgroup's kTokF32 tokens against every expert, accumulated in zs
// ([kTokF32][n_r]). u and e go to LDS in K chunks (256 wide when N_r <= 64, else 64, so
// that both fit beside zs) with 16-byte coalesced loads, at a pitch of one float more
// than the chunk so that the experts (and tokens) a wave reads at one k fall in
// different banks; each (token, expert) logit is one fp32 FMA chain in ascending k,
// carried in zs from chunk to chunk. Tokens past T repeat the last token (their logits
// are not used).
constexpr int kStageFloats = (kTokF32 + 64) * 257;  // the larger of the two chunk layouts
static_assert(kStageFloats >= (kTokF32 + kMaxExperts) * 65, "the 64-wide chunks fit");
constexpr int kPerF32 = 8;  // float4 loads a thread keeps in flight while staging

__device__ void logits_f32(const float* __restrict__ u, const float* __restrict__ e, int64_t T,
                           int d, int n_r, int64_t t0, float* zs, float* stage) {
  const int kcmax = n_r <= 64 ? 256 : 64;
  const int pitch = kcmax + 1;
  float* us = stage;
  float* es = stage + kTokF32 * pitch;
  for (int k0 = 0; k0 < d; k0 += kcmax) {
    const int kc = d - k0 < kcmax ? d - k0 : kcmax;  // d is a multiple of 64
    const int q4 = kc / 4;
    if (k0 > 0) __syncthreads();  // the previous chunk has been read
    // rows 0..kTokF32-1 of the chunk are u's, the rest e's; each thread issues all its loads
    // of a pass before its LDS stores, so they are in flight together
    const int n = (kTokF32 + n_r) * q4;
    for (int q0 = 0; q0 < n; q0 += kThreads * kPerF32) {
      float4 v[kPerF32];
#pragma unroll
      for (int i = 0; i < kPerF32; ++i) {
        const int q = q0 + threadIdx.x + i * kThreads;
        if (q < n) {
          const int row = q / q4, k = 4 * (q % q4);
          int64_t t = t0 + row;
          if (t >= T) t = T - 1;
          const float* src = row < kTokF32 ? u + t * d + k0 + k : e + static_cast<int64_t>(row - kTokF32) * d + k0 + k;
          v[i] = *reinterpret_cast<const float4*>(src);
        }
      }
#pragma unroll
      for (int i = 0; i < kPerF32; ++i) {
        const int q = q0 + threadIdx.x + i * kThreads;
        if (q < n) {
          const int row = q / q4, k = 4 * (q % q4);
          float* dst = row < kTokF32 ? us + row * pitch + k : es + (row - kTokF32) * pitch + k;
          dst[0] = v[i].x;
          dst[1] = v[i].y;
          dst[2] = v[i].z;
          dst[3] = v[i].w;
        }
      }
    }
    __syncthreads();
    for (int p = threadIdx.x; p < kTokF32 * n_r; p += kThreads) {
      const int i = p / n_r, j = p % n_r;
      const float* a = us + i * pitch;
      const float* b = es + j * pitch;
      float z = k0 == 0 ? 0.0f : zs[p];
      for (int c = 0; c < kc; c += 16) {  // 16 values read ahead of their FMAs (kc % 64 == 0)
        float av[16], bv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          av[q] = a[c + q];
          bv[q] = b[c + q];
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) z = fmaf(av[q], bv[q], z);
      }
      zs[p] = z;
    }
  }
}

// fp32 activations: one workgroup of 8 waves owns 8 tokens; their logits are formed in
// LDS (logits_f32), then one wave per token scores and selects.
template <int SCORE>
__global__ __launch_bounds__(kThreads) void route_kernel(const float* __restrict__ u, const float* __restrict__ e,
                                                         const float* __restrict__ bias, int64_t T, int d, int n_r,
                                                         int K, int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_gate) {
  __shared__ float zs[kTokF32 * kMaxExperts];
  __shared__ float stage[kStageFloats];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTokF32;
  logits_f32(u, e, T, d, n_r, t0, zs, stage);
  __syncthreads();
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  for (int i = wave; i < kTokF32; i += kThreads / kWave) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    uint64_t key[4];
    float sv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = lane + 64 * c;
      key[c] = 0;  // below every real key
      sv[c] = 0.0f;
      if (j < n_r) score_key<SCORE>(zs[i * n_r + j], bias, j, sv[c], key[c]);
    }
    topk_select<SCORE == 1>(key, sv, lane, K, topk_idx + t * K, topk_gate + t * K);
  }
}

}  // namespace

RouteChunks route_chunks(int64_t T, int d) {
  // enough (token block, K chunk) workgroups to fill the chip: about 512, at most 32
  // chunks, each a whole number of 64-wide K-steps
  const int64_t blocks = T > 0 ? (T + kTB - 1) / kTB : 1;
  const int nsteps = d / kLK;
  int64_t want = (512 + blocks - 1) / blocks;
  const int cap = nsteps < 32 ? nsteps : 32;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  RouteChunks r;
  r.steps_per_chunk = static_cast<int>((nsteps + want - 1) / want);
  r.chunks = (nsteps + r.steps_per_chunk - 1) / r.steps_per_chunk;
  return r;
}

size_t route_workspace_bytes(int64_t T, int d, int n_r) {
  return static_cast<size_t>(route_chunks(T, d).chunks) * static_cast<size_t>(T) * n_r * sizeof(float);
}

hipError_t launch_route(int act, int score, const void* u, const void* e, const float* bias, int64_t T, int d,
                        int n_r, int K, int32_t* idx, float* gate, float* part, hipStream_t stream) {
  if (act == 1) {
    const RouteChunks rc = route_chunks(T, d);
    const dim3 grid(static_cast<unsigned>((T + kTB - 1) / kTB), static_cast<unsigned>(rc.chunks));
    hipLaunchKernelGGL(route_logits, grid, dim3(kThreads), 0, stream, static_cast<const uint16_t*>(u),
                       static_cast<const uint16_t*>(e), T, d, n_r, rc.steps_per_chunk, part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const unsigned waves_per_block = 256 / kWave;
    const dim3 tgrid(static_cast<unsigned>((T + waves_per_block - 1) / waves_per_block));
    if (score == 1)
      hipLaunchKernelGGL(route_topk<1>, tgrid, dim3(256), 0, stream, part, rc.chunks, bias, T, n_r, K, idx, gate);
    else
      hipLaunchKernelGGL(route_topk<0>, tgrid, dim3(256), 0, stream, part, rc.chunks, bias, T, n_r, K, idx, gate);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((T + kTokF32 - 1) / kTokF32));
  if (score == 1)
    hipLaunchKernelGGL(route_kernel<1>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(u),
                       static_cast<const float*>(e), bias, T, d, n_r, K, idx, gate);
  else
    hipLaunchKernelGGL(route_kernel<0>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(u),
                       static_cast<const float*>(e), bias, T, d, n_r, K, idx, gate);
  return hipGetLastError();
}

}  // namespace moe

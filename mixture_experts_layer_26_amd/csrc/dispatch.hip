// Dispatch: stable counting sort of the (token, slot) pairs by expert, giving each
// expert's load, the exclusive offsets, the source token of every sorted row and the
// row of every pair. This is the per-expert grouping of the sums in the DeepSeek-V3
// explainer's equation for h'_t (method section 2); the deepseekmodel.com forward
// listing forms the same groups with one token mask per expert. The loads feed the
// end-of-step bias rule of the same section.
//
// Two kernels, and no atomic operation anywhere (global or LDS): the counts and the
// permutation come from wave ballots, so the result is deterministic by construction.
//   count:   block b counts the pairs of its token range per expert -> hist[b][e]
//   scatter: every block scans hist over blocks and experts (for its own bases), then
//            re-reads its pairs in passes of 256 and gives each pair its row: the rows of
//            earlier passes, of earlier waves in this pass and of lower lanes of its own
//            wave that hold the same expert. Pairs are read in index order t * K + k, so
//            rows inside an expert keep ascending token order.
// Inside a wave, the lanes that hold the same expert id are found by one ballot per bit
// of the id (a match over 8 bits); the lowest such lane writes the group's size to the
// wave's own LDS slot of that expert, which no other lane writes in that pass.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 256;          // tokens per block are a multiple of this
constexpr int kMaxExperts = 256;
constexpr int kIdBits = 8;           // expert ids are below 256

// Active lanes of this wave that hold expert id e (bit j for lane j). Every lane of the
// wave must call it (the ballots are wave-wide).
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool active) {
  uint64_t m = __ballot(active);
#pragma unroll
  for (int bit = 0; bit < kIdBits; ++bit) {
    const uint64_t ones = __ballot((e >> bit) & 1);
    m &= ((e >> bit) & 1) ? ones : ~ones;
  }
  return m;
}

__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x % kWave); }

// the lowest lane of a non-empty lane set
__device__ __forceinline__ int first_lane(uint64_t m) { return __ffsll(static_cast<unsigned long long>(m)) - 1; }

__global__ __launch_bounds__(kThreads) void count_kernel(const int32_t* __restrict__ idx, int64_t T,
                                                         int K, int n_r, int64_t tok_per_block,
                                                         int32_t* __restrict__ hist) {
  __shared__ int32_t wh[kWaves][kMaxExperts];  // pairs per wave and expert
  for (int i = threadIdx.x; i < kWaves * kMaxExperts; i += kThreads) (&wh[0][0])[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tok_per_block;
  int64_t t1 = t0 + tok_per_block;
  if (t1 > T) t1 = T;
  const int64_t p1 = t1 * K;
  for (int64_t q0 = t0 * K; q0 < p1; q0 += kThreads) {  // uniform over the block
    const int64_t p = q0 + threadIdx.x;
    const bool act = p < p1;
    const int e = act ? idx[p] : 0;
    const uint64_t peers = same_expert_lanes(e, act);
    if (act && first_lane(peers) == lane) wh[wave][e] += __popcll(peers);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_r; e += kThreads) {
    int32_t n = 0;
    for (int w = 0; w < kWaves; ++w) n += wh[w][e];
    hist[static_cast<int64_t>(blockIdx.x) * n_r + e] = n;
  }
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int K, int n_r, int64_t tok_per_block, int nblocks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ count, int32_t* __restrict__ offset,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pair_row) {
  __shared__ int32_t base[kMaxExperts];  // first row of this block's pairs, per expert
  __shared__ int32_t run[kMaxExperts];   // pairs of earlier passes of this block, per expert
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t wc[2][kWaves][kMaxExperts];  // pairs per wave and expert of a pass (two buffers)
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < n_r; e += kThreads) {
    int32_t before = 0, all = 0;
    for (int q = 0; q < nblocks; ++q) {
      const int32_t c = hist[static_cast<int64_t>(q) * n_r + e];
      if (q < b) before += c;
      all += c;
    }
    base[e] = before;
    tot[e] = all;
    run[e] = 0;
  }
  for (int i = threadIdx.x; i < 2 * kWaves * kMaxExperts; i += kThreads) (&wc[0][0][0])[i] = 0;
  __syncthreads();
  // exclusive scan of tot over experts (n_r <= 256, serial in thread 0)
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int e = 0; e < n_r; ++e) {
      const int32_t c = tot[e];
      tot[e] = acc;  // now the expert's offset
      acc += c;
    }
    if (b == 0) offset[n_r] = acc;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_r; e += kThreads) {
    if (b == 0) {
      offset[e] = tot[e];
      int32_t all = 0;
      for (int q = 0; q < nblocks; ++q) all += hist[static_cast<int64_t>(q) * n_r + e];
      count[e] = all;
    }
    base[e] += tot[e];
  }
  __syncthreads();
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const uint64_t below = (uint64_t(1) << lane) - 1;  // lanes under this one
  const int64_t t0 = static_cast<int64_t>(b) * tok_per_block;
  int64_t t1 = t0 + tok_per_block;
  if (t1 > T) t1 = T;
  const int64_t p1 = t1 * K;
  int cur = 0;
  for (int64_t q0 = t0 * K; q0 < p1; q0 += kThreads, cur ^= 1) {  // uniform over the block
    // phase 1: each wave's group sizes of this pass (buffer cur was cleared two passes ago)
    const int64_t p = q0 + threadIdx.x;
    const bool act = p < p1;
    const int e = act ? idx[p] : 0;
    const uint64_t peers = same_expert_lanes(e, act);
    if (act && first_lane(peers) == lane) wc[cur][wave][e] = __popcll(peers);
    __syncthreads();
    // phase 2: rows of this pass's pairs
    if (act) {
      int32_t row = base[e] + run[e] + __popcll(peers & below);
      for (int w = 0; w < wave; ++w) row += wc[cur][w][e];
      sorted_token[row] = static_cast<int32_t>(p / K);
      pair_row[p] = row;
    }
    __syncthreads();
    // phase 3: carry the pass's counts into run and clear buffer cur for the pass after
    // next (the next pass writes the other buffer, and its phase 2 reads run only after
    // its own barrier)
    for (int e2 = threadIdx.x; e2 < n_r; e2 += kThreads) {
      int32_t n = 0;
      for (int w = 0; w < kWaves; ++w) {
        n += wc[cur][w][e2];
        wc[cur][w][e2] = 0;
      }
      run[e2] += n;
    }
  }
}

}  // namespace

int dispatch_blocks(int64_t T) {
  int64_t nb = (T + kChunk - 1) / kChunk;
  if (nb > 128) nb = 128;
  return static_cast<int>(nb);
}

hipError_t launch_dispatch(const int32_t* idx, int64_t T, int K, int n_r, int32_t* hist,
                           int32_t* count, int32_t* offset, int32_t* sorted_token,
                           int32_t* pair_row, hipStream_t stream) {
  const int nb = dispatch_blocks(T);
  // tokens per block: a multiple of the chunk, so chunks never straddle blocks
  int64_t per = (T + nb - 1) / nb;
  per = (per + kChunk - 1) / kChunk * kChunk;
  hipLaunchKernelGGL(count_kernel, dim3(nb), dim3(kThreads), 0, stream, idx, T, K, n_r, per, hist);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scatter_kernel, dim3(nb), dim3(kThreads), 0, stream, idx, T, K, n_r, per, nb,
                     hist, count, offset, sorted_token, pair_row);
  return hipGetLastError();
}

}  // namespace moe

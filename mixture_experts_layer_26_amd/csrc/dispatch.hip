// Dispatch: stable counting sort of the (token, slot) pairs by expert, giving each
// expert's load, the exclusive offsets, the source token of every sorted row and the
// row of every pair. This is the per-expert grouping of the sums in the DeepSeek-V3
// explainer's equation for h'_t (method section 2); the deepseekmodel.com forward
// listing forms the same groups with one token mask per expert.
//
// Two kernels, no global atomics (the result is deterministic):
//   count:   block b histograms the pairs of its token range in LDS -> hist[b][e]
//   scatter: every block scans hist over blocks and experts (for its own bases),
//            re-reads its tokens in chunks of 256 and ranks each pair within the
//            chunk by a popcount over a per-expert LDS bitmap of the chunk's tokens,
//            so rows inside an expert keep ascending token order.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;          // tokens per bitmap chunk
constexpr int kWords = kChunk / 32;  // bitmap words per expert
constexpr int kMaxExperts = 256;

__global__ __launch_bounds__(kThreads) void count_kernel(const int32_t* __restrict__ idx, int64_t T,
                                                         int K, int n_r, int64_t tok_per_block,
                                                         int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < n_r; e += kThreads) h[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tok_per_block;
  int64_t t1 = t0 + tok_per_block;
  if (t1 > T) t1 = T;
  for (int64_t p = t0 * K + threadIdx.x; p < t1 * K; p += kThreads) atomicAdd(&h[idx[p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < n_r; e += kThreads) hist[static_cast<int64_t>(blockIdx.x) * n_r + e] = h[e];
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(
    const int32_t* __restrict__ idx, int64_t T, int K, int n_r, int64_t tok_per_block, int nblocks,
    const int32_t* __restrict__ hist, int32_t* __restrict__ count, int32_t* __restrict__ offset,
    int32_t* __restrict__ sorted_token, int32_t* __restrict__ pair_row) {
  __shared__ int32_t base[kMaxExperts];  // first row of this block's pairs, per expert
  __shared__ int32_t run[kMaxExperts];   // pairs of earlier chunks of this block, per expert
  __shared__ int32_t tot[kMaxExperts];
  __shared__ uint32_t bits[kMaxExperts * kWords];
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
  const int64_t t0 = static_cast<int64_t>(b) * tok_per_block;
  int64_t t1 = t0 + tok_per_block;
  if (t1 > T) t1 = T;
  for (int64_t c0 = t0; c0 < t1; c0 += kChunk) {
    const int64_t c1 = (c0 + kChunk < t1) ? c0 + kChunk : t1;
    for (int w = threadIdx.x; w < n_r * kWords; w += kThreads) bits[w] = 0;
    __syncthreads();
    for (int64_t p = c0 * K + threadIdx.x; p < c1 * K; p += kThreads) {
      const int tl = static_cast<int>(p / K - c0);
      atomicOr(&bits[idx[p] * kWords + tl / 32], 1u << (tl % 32));
    }
    __syncthreads();
    for (int64_t p = c0 * K + threadIdx.x; p < c1 * K; p += kThreads) {
      const int64_t t = p / K;
      const int tl = static_cast<int>(t - c0);
      const int e = idx[p];
      const uint32_t* bw = bits + e * kWords;
      int rank = __popc(bw[tl / 32] & ((1u << (tl % 32)) - 1u));
      for (int q = 0; q < tl / 32; ++q) rank += __popc(bw[q]);
      const int32_t row = base[e] + run[e] + rank;
      sorted_token[row] = static_cast<int32_t>(t);
      pair_row[p] = row;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n_r; e += kThreads) {
      int32_t n = 0;
      for (int q = 0; q < kWords; ++q) n += __popc(bits[e * kWords + q]);
      run[e] += n;
    }
    __syncthreads();
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

// Grouped SwiGLU expert FFN for fp32 operands (the small fp32 workload), with the same
// row layout as the bf16 path: H routed [P, d_ff] in sorted-row order, then H shared
// [T, n_s * d_ff]. FFN_i of the DeepSeek-V3 explainer's equation for h'_t (method
// section 2), gated SiLU form.
//
// Both launches cut each group into tiles of 16 rows x 16 output columns, one workgroup
// of 256 threads per tile and one output per thread. Groups: the routed experts (their
// sorted rows), then the shared experts (phase 1: one group per expert, over all tokens;
// phase 2: one group over all tokens whose K runs through every shared expert's d_ff
// columns in turn). The tile's operand rows go to LDS in K chunks of 256 with 16-byte
// coalesced loads, at a pitch of 257 floats so that the 16 columns (and 4 rows) a wave
// reads at one k fall in different banks; each thread then runs its dot products from
// LDS, 16 K values read ahead of their FMAs. Every output is one fp32 FMA chain in
// ascending K (phase 2, shared: ascending expert, then ascending K), so a chunk boundary
// changes nothing in the result.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kR = 16;              // rows per tile
constexpr int kC = 16;              // output columns per tile
constexpr int kKC = 256;            // K per staged chunk
constexpr int kPitch = kKC + 1;     // LDS row pitch in floats
static_assert(kR * kC == kThreads, "one output per thread");
// K values a thread reads from LDS before it runs their FMAs, so that one LDS round trip
// serves 16 FMAs instead of one (the chain itself stays in ascending K)
constexpr int kUnroll = 16;
constexpr int kMaxRouted = 256;  // the ABI's bound on N_r

// Group and tile-local index of tile `id`: the offsets are copied to LDS by all threads
// at once, then thread 0 walks the groups (rows of group q: routed expert q < n_r from the
// offsets, else T) in LDS, and the result is shared through LDS. Returns false past the
// last tile.
__device__ bool find_tile(const int32_t* __restrict__ offset, int n_r, int n_groups, int64_t T, int ncb,
                          int64_t id, int* sh, int* soff) {
  for (int i = threadIdx.x; i <= n_r; i += kThreads) soff[i] = offset[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t base = 0;
    int g = -1, local = 0;
    for (int q = 0; q < n_groups; ++q) {
      const int64_t rows = q < n_r ? static_cast<int64_t>(soff[q + 1] - soff[q]) : T;
      const int64_t n = (rows + kR - 1) / kR * ncb;
      if (id < base + n) {
        g = q;
        local = static_cast<int>(id - base);
        break;
      }
      base += n;
    }
    sh[0] = g;
    sh[1] = local;
  }
  __syncthreads();
  return sh[0] >= 0;
}

// A 16-row tile operand's K chunk [k0, k0 + kc) goes to LDS at pitch kPitch in two
// halves: load_rows fetches a thread's pieces of rows [0, nrows) into registers (at most
// kPer float4: 16 rows x 256 floats / 256 threads / 4), store_rows writes them. A tile
// loads all its operands before it stores any, so every load of the chunk is in flight
// at once. src(row, k) gives the address of the 4 floats at (row, k..k+3).
constexpr int kPer = kR * kKC / 4 / kThreads;
template <class Src>
__device__ __forceinline__ void load_rows(float4 (&v)[kPer], int nrows, int kc, Src&& src) {
  const int q4 = kc / 4, n = nrows * q4;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = threadIdx.x + i * kThreads;
    if (q < n) v[i] = *reinterpret_cast<const float4*>(src(q / q4, 4 * (q % q4)));
  }
}
__device__ __forceinline__ void store_rows(float* lds, const float4 (&v)[kPer], int nrows, int kc) {
  const int q4 = kc / 4, n = nrows * q4;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int q = threadIdx.x + i * kThreads;
    if (q < n) {
      float* d = lds + (q / q4) * kPitch + 4 * (q % q4);
      d[0] = v[i].x;
      d[1] = v[i].y;
      d[2] = v[i].z;
      d[3] = v[i].w;
    }
  }
}

__global__ __launch_bounds__(kThreads) void gate_up_f32(
    const float* __restrict__ u, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ sorted_token, const float* __restrict__ w1r,
    const float* __restrict__ w3r, const float* __restrict__ w1s, const float* __restrict__ w3s,
    int64_t T, int d, int d_ff, int n_r, int K, int n_s, float* __restrict__ h) {
  __shared__ float xs[kR * kPitch], as[kC * kPitch], bs[kC * kPitch];
  __shared__ int sh[2], soff[kMaxRouted + 1];
  const int ncb = d_ff / kC;
  if (!find_tile(offset, n_r, n_r + n_s, T, ncb, blockIdx.x, sh, soff)) return;
  const int g = sh[0], local = sh[1];
  const bool routed = g < n_r;
  const int64_t P = T * K;
  const int64_t rows = routed ? static_cast<int64_t>(soff[g + 1] - soff[g]) : T;
  const int64_t m0 = static_cast<int64_t>(local / ncb) * kR;  // first row of the tile in the group
  const int n0 = (local % ncb) * kC;
  const int nrows = rows - m0 < kR ? static_cast<int>(rows - m0) : kR;
  const int64_t rbase = routed ? soff[g] : 0;
  const float* wa = routed ? w1r + static_cast<int64_t>(g) * d_ff * d : w1s + static_cast<int64_t>(g - n_r) * d_ff * d;
  const float* wb = routed ? w3r + static_cast<int64_t>(g) * d_ff * d : w3s + static_cast<int64_t>(g - n_r) * d_ff * d;
  auto xrow = [&](int row) -> const float* {
    const int64_t m = m0 + row;
    return u + (routed ? static_cast<int64_t>(sorted_token[rbase + m]) : m) * d;
  };
  const int lr = threadIdx.x / kC, lc = threadIdx.x % kC;
  float za = 0.0f, zb = 0.0f;
  for (int k0 = 0; k0 < d; k0 += kKC) {
    const int kc = d - k0 < kKC ? d - k0 : kKC;
    if (k0 > 0) __syncthreads();  // the previous chunk has been read
    float4 vx[kPer], va[kPer], vb[kPer];
    load_rows(vx, nrows, kc, [&](int row, int k) { return xrow(row) + k0 + k; });
    load_rows(va, kC, kc, [&](int row, int k) { return wa + static_cast<int64_t>(n0 + row) * d + k0 + k; });
    load_rows(vb, kC, kc, [&](int row, int k) { return wb + static_cast<int64_t>(n0 + row) * d + k0 + k; });
    store_rows(xs, vx, nrows, kc);
    store_rows(as, va, kC, kc);
    store_rows(bs, vb, kC, kc);
    __syncthreads();
    if (lr < nrows) {
      const float* x = xs + lr * kPitch;
      const float* a = as + lc * kPitch;
      const float* b = bs + lc * kPitch;
      for (int c = 0; c < kc; c += kUnroll) {  // kc is a multiple of 64
        float xv[kUnroll], av[kUnroll], bv[kUnroll];
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
          xv[q] = x[c + q];
          av[q] = a[c + q];
          bv[q] = b[c + q];
        }
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
          za = fmaf(xv[q], av[q], za);
          zb = fmaf(xv[q], bv[q], zb);
        }
      }
    }
  }
  if (lr < nrows) {
    const int64_t m = m0 + lr;
    const int n = n0 + lc;
    float* dst = routed ? h + (rbase + m) * d_ff + n
                        : h + P * d_ff + m * (static_cast<int64_t>(n_s) * d_ff) + static_cast<int64_t>(g - n_r) * d_ff + n;
    *dst = za / (1.0f + expf(-za)) * zb;
  }
}

__global__ __launch_bounds__(kThreads) void down_f32(
    const float* __restrict__ h, const int32_t* __restrict__ offset, const float* __restrict__ w2r,
    const float* __restrict__ w2s, int64_t T, int d, int d_ff, int n_r, int K, int n_s,
    float* __restrict__ y_routed, float* __restrict__ y_shared) {
  __shared__ float hs[kR * kPitch], ws[kC * kPitch];
  __shared__ int sh[2], soff[kMaxRouted + 1];
  const int ncb = d / kC;
  if (!find_tile(offset, n_r, n_r + (n_s > 0 ? 1 : 0), T, ncb, blockIdx.x, sh, soff)) return;
  const int g = sh[0], local = sh[1];
  const bool routed = g < n_r;
  const int64_t P = T * K;
  const int64_t rows = routed ? static_cast<int64_t>(soff[g + 1] - soff[g]) : T;
  const int64_t m0 = static_cast<int64_t>(local / ncb) * kR;
  const int n0 = (local % ncb) * kC;
  const int nrows = rows - m0 < kR ? static_cast<int>(rows - m0) : kR;
  const int64_t rbase = routed ? soff[g] : 0;
  // K: d_ff (routed), or n_s * d_ff through the shared experts in turn
  const int kt = routed ? d_ff : n_s * d_ff;
  const int64_t hpitch = routed ? d_ff : static_cast<int64_t>(n_s) * d_ff;
  const float* hbase = routed ? h + rbase * d_ff : h + P * d_ff;
  const int lr = threadIdx.x / kC, lc = threadIdx.x % kC;
  float z = 0.0f;
  for (int k0 = 0; k0 < kt; k0 += kKC) {
    const int kc = kt - k0 < kKC ? kt - k0 : kKC;
    if (k0 > 0) __syncthreads();
    float4 vh[kPer], vw[kPer];
    load_rows(vh, nrows, kc, [&](int row, int k) { return hbase + (m0 + row) * hpitch + k0 + k; });
    load_rows(vw, kC, kc, [&](int row, int k) {
      const int kk = k0 + k;  // 4 consecutive k never straddle two experts (d_ff % 4 == 0)
      if (routed) return w2r + (static_cast<int64_t>(g) * d + n0 + row) * d_ff + kk;
      const int s = kk / d_ff;
      return w2s + (static_cast<int64_t>(s) * d + n0 + row) * d_ff + (kk - s * d_ff);
    });
    store_rows(hs, vh, nrows, kc);
    store_rows(ws, vw, kC, kc);
    __syncthreads();
    if (lr < nrows) {
      const float* x = hs + lr * kPitch;
      const float* w = ws + lc * kPitch;
      for (int c = 0; c < kc; c += kUnroll) {
        float xv[kUnroll], wv[kUnroll];
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
          xv[q] = x[c + q];
          wv[q] = w[c + q];
        }
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) z = fmaf(xv[q], wv[q], z);
      }
    }
  }
  if (lr < nrows) {
    const int64_t m = m0 + lr;
    const int n = n0 + lc;
    if (routed)
      y_routed[(rbase + m) * d + n] = z;
    else
      y_shared[m * d + n] = z;
  }
}

// Tiles of a launch, bounded from above without reading the offsets: each group adds at
// most one partial row block.
int64_t tile_bound(int64_t rows, int groups, int ncb) { return ((rows + kR - 1) / kR + groups) * ncb; }

}  // namespace

hipError_t launch_ffn_f32(const float* u, const int32_t* offset, const int32_t* sorted_token,
                          const float* w1r, const float* w3r, const float* w2r, const float* w1s,
                          const float* w3s, const float* w2s, int64_t T, int d, int d_ff, int n_r,
                          int K, int n_s, float* h, float* y_routed, float* y_shared,
                          hipStream_t stream) {
  if (d % kC != 0 || d_ff % kC != 0 || d % 4 != 0 || d_ff % 4 != 0) return hipErrorInvalidValue;
  const int64_t P = T * K;
  const int64_t g1 = tile_bound(P + T * n_s, n_r + n_s, d_ff / kC);
  const int64_t g2 = tile_bound(P + (n_s > 0 ? T : 0), n_r + (n_s > 0 ? 1 : 0), d / kC);
  if (g1 > INT32_MAX || g2 > INT32_MAX) return hipErrorInvalidValue;
  if (g1 > 0) {
    hipLaunchKernelGGL(gate_up_f32, dim3(static_cast<unsigned>(g1)), dim3(kThreads), 0, stream, u, offset,
                       sorted_token, w1r, w3r, w1s, w3s, T, d, d_ff, n_r, K, n_s, h);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (g2 > 0)
    hipLaunchKernelGGL(down_f32, dim3(static_cast<unsigned>(g2)), dim3(kThreads), 0, stream, h, offset, w2r,
                       w2s, T, d, d_ff, n_r, K, n_s, y_routed, y_shared);
  return hipGetLastError();
}

}  // namespace moe

// FP8 E4M3 tile quantisation: per tile, amax = max|x|, s = fl32(amax / 448),
// q = E4M3_RNE(fl32(x / s)) with magnitudes clamped at 448; s == 0 gives q = 0.
// The quantisation pseudo-code of "DeepSeek モデルアーキテクチャ徹底解説"
// (deepseekmodel.com; 448 is the E4M3 maximum), with the tile shapes of the
// DeepSeek-V3 explainer's key ideas (1x128 activation tiles, 128x128 weight blocks).
// Conversion: v_cvt_pk_fp8_f32 (OCP E4M3FN on gfx950, round to nearest even).
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// 16 bytes of x at element index i as floats: 8 bf16 or 4 fp32 values
template <int XT>
__device__ __forceinline__ void load_chunk(const void* x, int64_t i, float* v) {
  const uint4 raw = XT == 1 ? ld16(static_cast<const uint16_t*>(x) + i) : ld16(static_cast<const float*>(x) + i);
  if (XT == 1) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
    v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
  }
}

// E4M3 codes of n = 8 (bf16) or 4 (fp32) values, packed little-endian
template <int N>
__device__ __forceinline__ uint64_t codes(const float* v, float s) {
  uint64_t out = 0;
#pragma unroll
  for (int k = 0; k < N; k += 2) {
    const uint32_t pair = s == 0.0f ? 0u : e4m3_pair(v[k] / s, v[k + 1] / s);
    out |= static_cast<uint64_t>(pair) << (8 * k);
  }
  return out;
}

// 1 x 128 tiles: a group of G lanes (16 for bf16, 32 for fp32) covers one tile with one
// 16-byte load each; the tile's amax is reduced across the group.
template <int XT>
__global__ __launch_bounds__(256) void quant_row_tiles(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int E = XT == 1 ? 8 : 4;  // elements per lane
  constexpr int G = 128 / E;          // lanes per tile
  const int64_t tiles = rows * (cols / 128);
  const int64_t tile = (blockIdx.x * 256LL + threadIdx.x) / G;
  const int gl = threadIdx.x % G;
  const bool live = tile < tiles;
  const int64_t r = live ? tile / (cols / 128) : 0, cb = live ? tile % (cols / 128) : 0;
  const int64_t base = r * cols + cb * 128 + gl * E;
  float v[E];
  if (live) load_chunk<XT>(x, base, v);
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < E; ++k) m = fmaxf(m, live ? fabsf(v[k]) : 0.0f);
#pragma unroll
  for (int off = 1; off < G; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  if (!live) return;
  const float s = m / 448.0f;
  const uint64_t c = codes<E>(v, s);
  if (E == 8)
    *reinterpret_cast<uint64_t*>(q + base) = c;
  else
    *reinterpret_cast<uint32_t*>(q + base) = static_cast<uint32_t>(c);
  if (gl == 0) scale[tile] = s;
}

// 128 x 128 tiles: one workgroup of 256 threads per tile; each thread holds 64 values
// (16-byte chunks of 8 rows), the amax is reduced across the workgroup.
template <int XT>
__global__ __launch_bounds__(256) void quant_block_tiles(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  constexpr int E = XT == 1 ? 8 : 4;  // elements per chunk
  constexpr int CPR = 128 / E;        // chunks per tile row
  constexpr int RPP = 256 / CPR;      // rows covered per pass
  constexpr int NP = 128 / RPP;       // passes
  __shared__ float wmax[4];
  const int64_t nbc = cols / 128;
  const int64_t br = blockIdx.x / nbc, bc = blockIdx.x % nbc;
  const int tid = threadIdx.x;
  const int cc = tid % CPR, rr = tid / CPR;
  float v[NP][E];
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t row = br * 128 + rr + RPP * p;
    load_chunk<XT>(x, row * cols + bc * 128 + cc * E, v[p]);
#pragma unroll
    for (int k = 0; k < E; ++k) m = fmaxf(m, fabsf(v[p][k]));
  }
  m = wave_max(m);
  if (tid % kWave == 0) wmax[tid / kWave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax / 448.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int64_t row = br * 128 + rr + RPP * p;
    const uint64_t c = codes<E>(v[p], s);
    uint8_t* dst = q + row * cols + bc * 128 + cc * E;
    if (E == 8)
      *reinterpret_cast<uint64_t*>(dst) = c;
    else
      *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(c);
  }
  if (tid == 0) scale[blockIdx.x] = s;
}

// grid (ceil((P + T) / 256), nkb): one thread per output, coalesced writes
__global__ __launch_bounds__(256) void scale_columns_kernel(const float* __restrict__ s, int nkb,
                                                            const int32_t* __restrict__ sorted_token, int64_t P,
                                                            int64_t T, float* __restrict__ out) {
  const int64_t j = blockIdx.x * 256LL + threadIdx.x;
  const int kb = blockIdx.y;
  if (j >= P + T) return;
  const int64_t tok = j < P ? sorted_token[j] : j - P;
  out[kb * (P + T) + j] = s[tok * nkb + kb];
}

}  // namespace

hipError_t launch_scale_columns(const float* s, int nkb, const int32_t* sorted_token, int64_t P, int64_t T,
                                float* out, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((P + T + 255) / 256), static_cast<unsigned>(nkb));
  hipLaunchKernelGGL(scale_columns_kernel, grid, dim3(256), 0, stream, s, nkb, sorted_token, P, T, out);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, int xt, int64_t rows, int64_t cols, int tile_r,
                               int tile_c, uint8_t* q, float* scale, hipStream_t stream) {
  (void)tile_c;
  if (tile_r == 1) {
    const int64_t lanes = rows * (cols / 128) * (xt == 1 ? 16 : 32);
    const dim3 grid(static_cast<unsigned>((lanes + 255) / 256));
    if (xt == 1)
      hipLaunchKernelGGL(quant_row_tiles<1>, grid, dim3(256), 0, stream, x, rows, cols, q, scale);
    else
      hipLaunchKernelGGL(quant_row_tiles<0>, grid, dim3(256), 0, stream, x, rows, cols, q, scale);
  } else {
    const dim3 grid(static_cast<unsigned>((rows / 128) * (cols / 128)));
    if (xt == 1)
      hipLaunchKernelGGL(quant_block_tiles<1>, grid, dim3(256), 0, stream, x, rows, cols, q, scale);
    else
      hipLaunchKernelGGL(quant_block_tiles<0>, grid, dim3(256), 0, stream, x, rows, cols, q, scale);
  }
  return hipGetLastError();
}

}  // namespace moe

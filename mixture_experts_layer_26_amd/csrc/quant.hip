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

__device__ __forceinline__ float load_elem(const void* x, int xt, int64_t i) {
  return xt == 1 ? bf16_to_f32(static_cast<const uint16_t*>(x)[i]) : static_cast<const float*>(x)[i];
}

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

// 1 x 128 tiles: one wave per tile, two elements per lane
__global__ __launch_bounds__(256) void quant_row_tiles(const void* __restrict__ x, int xt,
                                                       int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ q,
                                                       float* __restrict__ scale) {
  const int lane = threadIdx.x % kWave;
  const int64_t tile = blockIdx.x * 4LL + threadIdx.x / kWave;
  const int64_t tiles_per_row = cols / 128;
  if (tile >= rows * tiles_per_row) return;
  const int64_t r = tile / tiles_per_row, cb = tile % tiles_per_row;
  const int64_t base = r * cols + cb * 128 + 2 * lane;
  const float a = load_elem(x, xt, base), b = load_elem(x, xt, base + 1);
  const float amax = wave_max(fmaxf(fabsf(a), fabsf(b)));
  const float s = amax / 448.0f;
  uint32_t pair = 0;
  if (s != 0.0f) pair = e4m3_pair(a / s, b / s);
  *reinterpret_cast<uint16_t*>(q + base) = static_cast<uint16_t>(pair);
  if (lane == 0) scale[tile] = s;
}

// 128 x 128 tiles: one workgroup of 256 threads per tile
__global__ __launch_bounds__(256) void quant_block_tiles(const void* __restrict__ x, int xt,
                                                         int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  __shared__ float wmax[4];
  const int64_t nbc = cols / 128;
  const int64_t br = blockIdx.x / nbc, bc = blockIdx.x % nbc;
  const int tid = threadIdx.x;
  // thread covers row (tid / 2) and columns 64 * (tid % 2) .. +64
  const int64_t r = br * 128 + tid / 2;
  const int64_t c0 = bc * 128 + 64 * (tid % 2);
  float m = 0.0f;
  for (int j = 0; j < 64; ++j) m = fmaxf(m, fabsf(load_elem(x, xt, r * cols + c0 + j)));
  m = wave_max(m);
  if (tid % kWave == 0) wmax[tid / kWave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax / 448.0f;
  for (int j = 0; j < 64; j += 2) {
    uint32_t pair = 0;
    if (s != 0.0f)
      pair = e4m3_pair(load_elem(x, xt, r * cols + c0 + j) / s, load_elem(x, xt, r * cols + c0 + j + 1) / s);
    *reinterpret_cast<uint16_t*>(q + r * cols + c0 + j) = static_cast<uint16_t>(pair);
  }
  if (tid == 0) scale[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_quantize_fp8(const void* x, int xt, int64_t rows, int64_t cols, int tile_r,
                               int tile_c, uint8_t* q, float* scale, hipStream_t stream) {
  (void)tile_c;
  if (tile_r == 1) {
    const int64_t tiles = rows * (cols / 128);
    hipLaunchKernelGGL(quant_row_tiles, dim3(static_cast<unsigned>((tiles + 3) / 4)), dim3(256), 0,
                       stream, x, xt, rows, cols, q, scale);
  } else {
    const int64_t tiles = (rows / 128) * (cols / 128);
    hipLaunchKernelGGL(quant_block_tiles, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream,
                       x, xt, rows, cols, q, scale);
  }
  return hipGetLastError();
}

}  // namespace moe

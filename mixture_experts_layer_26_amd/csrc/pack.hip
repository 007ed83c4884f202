// Tiled weight layout for the grouped expert GEMMs.
//
// An expert's [N, K] weight matrix (row n = output n, contiguous over K) is stored as
// [N/R][K/KS][R][KS]: for each tile of R output rows, the R rows' KS elements of one
// K-step (128 bytes: 64 bf16 or 128 fp8 codes) lie together. A K-step of a GEMM tile is
// then one contiguous block of R x 128 bytes instead of R pieces 128 bytes long and K
// elements apart, which keeps each CU's weight stream in few DRAM pages. R = 128 for the
// gate/up matrices (a gate/up tile takes 128 rows of each), 256 for the down matrix.
// Only the order of bytes changes; the GEMMs read the same values.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kStepBytes = 128;

__global__ void pack_weights_kernel(const unsigned char* __restrict__ src, unsigned char* __restrict__ dst,
                                    int64_t E, int64_t N, int64_t row_bytes, int R, int64_t chunks) {
  const int64_t kt_n = row_bytes / kStepBytes;  // K-steps per row
  const int64_t nt_n = N / R;                   // row tiles per expert
  for (int64_t o = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; o < chunks;
       o += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    // output chunk o -> (e, nt, kt, r, c) of [E][N/R][K/KS][R][8 chunks of 16 bytes]
    const int64_t c = o % 8;
    int64_t rest = o / 8;
    const int64_t r = rest % R;
    rest /= R;
    const int64_t kt = rest % kt_n;
    rest /= kt_n;
    const int64_t nt = rest % nt_n;
    const int64_t e = rest / nt_n;
    const int64_t s = ((e * N + nt * R + r) * row_bytes) + kt * kStepBytes + c * 16;
    st16(dst + o * 16, ld16(src + s));
  }
}

}  // namespace

hipError_t launch_pack_weights(const void* src, void* dst, int esz, int64_t E, int64_t N, int64_t K, int R,
                               hipStream_t stream) {
  const int64_t row_bytes = K * esz;
  const int64_t chunks = E * N * row_bytes / 16;
  const int64_t want = (chunks + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? (want > 0 ? want : 1) : 65536);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const unsigned char*>(src), static_cast<unsigned char*>(dst), E, N, row_bytes, R,
                     chunks);
  return hipGetLastError();
}

}  // namespace moe

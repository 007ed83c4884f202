// Grouped SwiGLU expert FFN in bf16 on gfx950 MFMA (fp32 accumulate).
//
// FFN_i of the DeepSeek-V3 explainer's equation for h'_t (method section 2), in the
// gated SiLU form y = W2 (SiLU(W1 x) * (W3 x)):
//   phase 1 (gated):  H[row, n] = SiLU(x_row . W1[n]) * (x_row . W3[n])  -> bf16
//   phase 2 (plain):  Y[row, n] = H_row . W2[n]
// Groups are the routed experts (rows = the expert's sorted pairs, x gathered from u
// through sorted_token) and the shared experts (rows = all tokens).
//
// Kernel shape: a persistent grid of 256 workgroups (one per CU), 4 waves each, walks a
// tile list built on the device from expert_offset: no host synchronisation. Tiles
// are 256 rows x 256 B-rows (phase 1: 128 gate + 128 up columns) with K-steps of 64,
// staged through XOR-swizzled LDS (double buffered) and consumed by
// v_mfma_f32_32x32x16_bf16; each wave owns a 128 x 128 block (16 MFMA tiles). The tile
// list is split into 8 contiguous chunks, one per XCD, so the tiles of one expert run
// side by side on one XCD and its weights and gathered rows are reused from that
// XCD's L2. MFMA blocks whose 32 rows are all past an expert's count are skipped.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 256;   // rows per tile
constexpr int BNB = 256;  // B rows per tile
constexpr int BK = 64;    // K per step
constexpr int kMaxGroups = 256 + 8;

struct Tile {
  int group;   // routed expert, or n_r + shared index
  int m0;      // first row of the tile within the group
  int n0;      // first output column
  int rows;    // valid rows in this tile
};

// Tile list: routed groups first (expert-major, then output-column tile, then row tile),
// then the shared groups. Built per workgroup in LDS from expert_offset.
struct TileMap {
  int cum[kMaxGroups + 1];  // first tile index of each group
  int mt[kMaxGroups];       // row tiles per group
  int total;
};

__device__ void build_tile_map(TileMap& tm, const int32_t* offset, int n_r, int n_groups_shared,
                               int64_t T, int ntn) {
  const int ng = n_r + n_groups_shared;
  for (int g = threadIdx.x; g < ng; g += kThreads) {
    const int64_t rows = g < n_r ? (offset[g + 1] - offset[g]) : T;
    tm.mt[g] = static_cast<int>((rows + BM - 1) / BM);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int g = 0; g < ng; ++g) {
      tm.cum[g] = acc;
      acc += tm.mt[g] * ntn;
    }
    tm.cum[ng] = acc;
    tm.total = acc;
  }
  __syncthreads();
}

__device__ __forceinline__ Tile tile_at(const TileMap& tm, int L, int ng, int ntn,
                                        const int32_t* offset, int n_r, int64_t T, int bn_out) {
  int lo = 0, hi = ng - 1;  // last group with cum[g] <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (tm.cum[mid] <= L) lo = mid; else hi = mid - 1;
  }
  Tile t;
  t.group = lo;
  const int local = L - tm.cum[lo];
  const int mt = tm.mt[lo];
  t.n0 = (local / mt) * bn_out;
  t.m0 = (local % mt) * BM;
  const int64_t rows = lo < n_r ? (offset[lo + 1] - offset[lo]) : T;
  const int64_t left = rows - t.m0;
  t.rows = static_cast<int>(left < BM ? left : BM);
  return t;
}

// LDS byte offset of 16-byte chunk c (0..7) of row r in a [rows][64] bf16 tile
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <bool GATED>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16(GemmArgs args) {
  __shared__ TileMap tm;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // LDS: A[2][BM][BK] then B[2][BNB][BK], bf16, XOR-swizzled 16-byte chunks
  auto lds_a = [&](int buf) { return smem + buf * (BM * BK * 2); };
  auto lds_b = [&](int buf) { return smem + 2 * BM * BK * 2 + buf * (BNB * BK * 2); };

  const int n_r = args.n_r;
  const int ngs = args.n_shared_groups;
  const int ng = n_r + ngs;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map(tm, args.offset, n_r, ngs, args.T, ntn);
  const int total = tm.total;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  // global->LDS copy assignment: chunk (tid % 8) of rows tid/8 + 32*i
  const int cc = tid % 8, cr = tid / 8;

  // XCD-contiguous walk over the tile list
  const int per_xcd_slots = gridDim.x / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int chunk = (total + 7) / 8;
  const int L_begin = xcd * chunk;
  int L_end = L_begin + chunk;
  if (L_end > total) L_end = total;

  for (int L = L_begin + slot; L < L_end; L += per_xcd_slots) {
    const Tile t = tile_at(tm, L, ng, ntn, args.offset, n_r, args.T, bn_out);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;  // shared group index
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    // A row pointers (rows past the tile's valid rows repeat its last valid row)
    const uint16_t* arow[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int r = cr + 32 * i;
      if (r >= t.rows) r = t.rows - 1;
      const int64_t m = t.m0 + r;
      if (routed) {
        const int64_t src = args.gather ? args.gather[row_base + m] : (row_base + m);
        arow[i] = args.a_routed + src * args.lda_routed + cc * 8;
      } else {
        arow[i] = args.a_shared + m * args.lda_shared + cc * 8;
      }
    }
    // B row pointers
    const uint16_t* brow[8];
    int64_t b_seg_stride = 0;  // phase 2 shared: next expert's W2 per K segment
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = cr + 32 * i;  // 0..255
      const uint16_t* base;
      int n;
      if (GATED) {
        const bool up = r >= 128;
        n = t.n0 + (r & 127);
        if (routed)
          base = (up ? args.b3_routed : args.b1_routed) + static_cast<int64_t>(t.group) * args.b_expert_stride;
        else
          base = (up ? args.b3_shared : args.b1_shared) + static_cast<int64_t>(sg) * args.b_expert_stride;
      } else {
        n = t.n0 + r;
        base = routed ? args.b1_routed + static_cast<int64_t>(t.group) * args.b_expert_stride
                      : args.b1_shared;
      }
      brow[i] = base + static_cast<int64_t>(n) * args.ldb + cc * 8;
    }
    if (!routed && !GATED) b_seg_stride = args.b_expert_stride;
    const int ktot = routed ? args.K : args.K * (GATED ? 1 : args.k_segments);
    const int nk = ktot / BK;
    const int kseg_steps = args.K / BK;  // K-steps per shared segment (phase 2)

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    // how many 32-row MFMA blocks of this wave hold valid rows
    int vblk = (t.rows - 128 * wm + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > 4 ? 4 : vblk);

    uint4 ra[8], rb[8];
    auto gload = [&](int kt) {
      int64_t boff = static_cast<int64_t>(kt) * BK;
      if (b_seg_stride) {
        const int seg = kt / kseg_steps;
        boff = static_cast<int64_t>(seg) * b_seg_stride + static_cast<int64_t>(kt - seg * kseg_steps) * BK;
      }
      const int64_t aoff = static_cast<int64_t>(kt) * BK;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ra[i] = ld16(arow[i] + aoff);
        rb[i] = ld16(brow[i] + boff);
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = cr + 32 * i;
        *reinterpret_cast<uint4*>(lds_a(buf) + swz(r, cc)) = ra[i];
        *reinterpret_cast<uint4*>(lds_b(buf) + swz(r, cc)) = rb[i];
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
      const unsigned char* la = lds_a(cur);
      const unsigned char* lb = lds_b(cur);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = 2 * s + lane / 32;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int r = 128 * wm + 32 * mb + lane % 32;
          af[mb] = *reinterpret_cast<const bf16x8*>(la + swz(r, c));
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          int r;
          if (GATED)
            r = (nb < 2 ? 0 : 128) + 64 * wn + 32 * (nb & 1) + lane % 32;
          else
            r = 128 * wn + 32 * nb + lane % 32;
          bfr[nb] = *reinterpret_cast<const bf16x8*>(lb + swz(r, c));
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb < vblk) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
              acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
          }
        }
      }
      if (kt + 1 < nk) lstore(cur ^ 1);
      __syncthreads();
    }

    // epilogue: C layout of the 32x32 MFMA -- lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4
    const int col_in = lane % 32;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb >= vblk) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 128 * wm + 32 * mb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
        if (i >= t.rows) continue;
        const int64_t m = t.m0 + i;
        if (GATED) {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int n = t.n0 + 64 * wn + 32 * nb + col_in;
            const float h = silu(acc[mb][nb][v]) * acc[mb][nb + 2][v];
            uint16_t* o = routed ? static_cast<uint16_t*>(args.out_routed) + (row_base + m) * args.ldo_routed + n
                                 : static_cast<uint16_t*>(args.out_shared) + m * args.ldo_shared +
                                       static_cast<int64_t>(sg) * args.N + n;
            *o = f32_to_bf16(h);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int n = t.n0 + 128 * wn + 32 * nb + col_in;
            const float y = acc[mb][nb][v];
            if (routed)
              static_cast<uint16_t*>(args.out_routed)[(row_base + m) * args.ldo_routed + n] = f32_to_bf16(y);
            else
              static_cast<float*>(args.out_shared)[m * args.ldo_shared + n] = y;
          }
        }
      }
    }
  }
}

}  // namespace

size_t ffn_bf16_lds_bytes() { return 2 * BM * BK * 2 + 2 * BNB * BK * 2; }

hipError_t launch_grouped_gemm_bf16(const GemmArgs& args, bool gated, int grid, hipStream_t stream) {
  const size_t lds = ffn_bf16_lds_bytes();
  const void* fn = gated ? reinterpret_cast<const void*>(grouped_gemm_bf16<true>)
                         : reinterpret_cast<const void*>(grouped_gemm_bf16<false>);
  hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  if (gated)
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3(grid), dim3(kThreads), lds, stream, args);
  else
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3(grid), dim3(kThreads), lds, stream, args);
  return hipGetLastError();
}

}  // namespace moe

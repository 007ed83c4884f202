// Grouped SwiGLU expert FFN in bf16 on gfx950 MFMA (fp32 accumulate).
//
// FFN_i of the DeepSeek-V3 explainer's equation for h'_t (method section 2), in the
// gated SiLU form y = W2 (SiLU(W1 x) * (W3 x)):
//   phase 1 (gated):  H[row, n] = SiLU(x_row . W1[n]) * (x_row . W3[n])  -> bf16
//   phase 2 (plain):  Y[row, n] = H_row . W2[n]
// Groups are the routed experts (rows = the expert's sorted pairs, x gathered from u
// through sorted_token) and the shared experts (rows = all tokens).
//
// Kernel shape: a persistent grid of one 8-wave workgroup per CU walks the device-built
// tile list (gemm_common.h). A tile is 256 rows x 256 weight rows (phase 1: 128 gate
// + 128 up columns) in K-steps of 64, staged through XOR-swizzled LDS (two stages) and
// consumed by v_mfma_f32_32x32x16_bf16. The waves form two groups of four, one wave of
// each group per SIMD; group g owns rows 128g.. of the tile and weight rows 128g..
// (gate rows for g = 0 and up rows for g = 1 in phase 1), each wave a 128 x 64 block
// (8 MFMA tiles). The groups ping-pong: while one runs the MFMAs of K-step k, the other
// stores its halves of step k+1 into the other LDS stage, so each SIMD's MFMA pipe is
// fed by one wave while its partner waits on memory. The K loop is specialised on the
// number of 32-row blocks of a wave that hold rows, so row blocks past an expert's
// count cost no MFMA work.
#include "gemm_common.h"
#include "launch.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int BK = 64;  // bf16 elements per K-step (128 bytes per row)

struct TileCtx {
  const uint16_t* arow[4];  // this thread's 4 A rows (its 16-byte chunk)
  const uint16_t* b;        // this thread's first B row (chunk); rows +32*i
  int64_t ldb;
  int64_t seg_stride;       // phase 2 shared: W2 stride per K segment, else 0
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;                   // K-steps
};

// MFMAs of one K-step from LDS stage (la, lb) for a wave holding NMB live 32-row
// blocks; the next sub-step's fragments are read while the current MFMAs run.
template <int NMB>
__device__ __forceinline__ void compute_step(const unsigned char* la, const unsigned char* lb, int arow0,
                                             const int (&brow)[2], int lane, f32x16 (&acc)[4][2]) {
  constexpr int NA = NMB > 0 ? NMB : 1;
  constexpr int NRD = NMB + 2;  // fragment reads per sub-step
  constexpr int NMF = NMB * 2;  // MFMAs per sub-step
  bf16x8 af[2][NA], bfr[2][2];
  auto rd = [&](int s, int buf) {
    const int ch = 2 * s + lane / 32;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      af[buf][mb] = *reinterpret_cast<const bf16x8*>(la + swz(arow0 + 32 * mb, ch));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) bfr[buf][nb] = *reinterpret_cast<const bf16x8*>(lb + swz(brow[nb], ch));
  };
  rd(0, 0);
  if (NMB > 0) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cur = s & 1;
    if (s + 1 < 4) rd(s + 1, (s + 1) & 1);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][mb], bfr[cur][nb], acc[mb][nb], 0, 0, 0);
    if (NMB > 0) {
      if (s + 1 < 4 && NMF >= NRD) {
        // the next sub-step's reads threaded between this sub-step's MFMAs
#pragma unroll
        for (int i = 0; i < NRD; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NMF > NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
      } else {
        if (s + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      }
    }
  }
}

// Ping-pong K loop. Group g stores its A rows 128g.. and B rows 128g.. of each stage.
// Global loads for a group's next step are issued at the start of its compute half and
// stored in its memory half; indices past the last step are clamped (harmless reloads).
template <bool GATED, int NMB>
__device__ __forceinline__ void mainloop(const TileCtx& c, unsigned char* smem, f32x16 (&acc)[4][2]) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = __builtin_amdgcn_readfirstlane(wave / 4), wn = wave % 4;
  const int gt = tid % 256, cc = gt % 8, cr = gt / 8;
  const int last = c.nk - 1;
  auto la = [&](int st) { return smem + st * kStageBytes; };
  auto lb = [&](int st) { return smem + 2 * kStageBytes + st * kStageBytes; };
  const int arow0 = 128 * g + lane % 32;
  int brow[2];
  if (GATED) {  // gate block and the matching up block
    brow[0] = 32 * wn + lane % 32;
    brow[1] = 128 + 32 * wn + lane % 32;
  } else {
    brow[0] = 64 * wn + lane % 32;
    brow[1] = 64 * wn + 32 + lane % 32;
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
    kt = kt < last ? kt : last;
    const int64_t aoff = static_cast<int64_t>(kt) * BK;
    const int64_t boff = b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, BK);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld16(c.arow[i] + aoff);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ld16(c.b + static_cast<int64_t>(32 * i) * c.ldb + boff);
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 128 * g + cr + 32 * i;
      *reinterpret_cast<uint4*>(la(st) + swz(r, cc)) = ra[i];
      *reinterpret_cast<uint4*>(lb(st) + swz(r, cc)) = rb[i];
    }
  };
  gload(0);
  lstore(0);
  if (g == 1) gload(1);
  __syncthreads();
  for (int kt = 0; kt < c.nk; ++kt) {
    const int cur = kt & 1;
    // first half: group 0 computes step kt, group 1 stores its halves of step kt+1
    if (g == 0) {
      gload(kt + 1);
      compute_step<NMB>(la(cur), lb(cur), arow0, brow, lane, acc);
    } else {
      lstore(cur ^ 1);
    }
    lds_barrier();
    // second half: group 1 computes step kt, group 0 stores its halves of step kt+1
    if (g == 1) {
      gload(kt + 2);
      compute_step<NMB>(la(cur), lb(cur), arow0, brow, lane, acc);
    } else {
      lstore(cur ^ 1);
    }
    lds_barrier();
  }
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16(GemmArgs args) {
  __shared__ TileMap tm;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int n_r = args.n_r;
  const int ng = n_r + args.n_shared_groups;
  const int bn_out = GATED ? BNB / 2 : BNB;
  build_tile_map(tm, args.offset, n_r, args.n_shared_groups, args.T, args.N / bn_out);

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = wave / 4, wn = wave % 4;
  const int gt = tid % 256, cc = gt % 8, gr = gt / 8;

  for_each_tile(tm.total, args.tile_counter, [&](int L) {
    const Tile t = tile_at(tm, L, ng, args.offset, n_r, args.T, bn_out);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;  // shared group index
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    TileCtx c;
    // A rows of this group's half (rows past the tile's valid rows repeat its last one)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int r = 128 * g + gr + 32 * i;
      if (r >= t.rows) r = t.rows - 1;
      const int64_t m = t.m0 + r;
      if (routed) {
        const int64_t src = args.gather ? args.gather[row_base + m] : (row_base + m);
        c.arow[i] = args.a_routed + src * args.lda_routed + cc * 8;
      } else {
        c.arow[i] = args.a_shared + m * args.lda_shared + cc * 8;
      }
    }
    // B rows of this group's half: gate (g = 0) / up (g = 1) rows when gated
    const int64_t eoff = static_cast<int64_t>(routed ? t.group : sg) * args.b_expert_stride;
    const uint16_t* base;
    int64_t nrow;
    if (GATED) {
      base = (g == 0 ? (routed ? args.b1_routed : args.b1_shared) : (routed ? args.b3_routed : args.b3_shared)) + eoff;
      nrow = t.n0 + gr;
    } else {
      base = routed ? args.b1_routed + eoff : args.b1_shared;
      nrow = t.n0 + 128 * g + gr;
    }
    c.b = base + nrow * args.ldb + cc * 8;
    c.ldb = args.ldb;
    c.seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = static_cast<uint32_t>((0x100000000ull + c.kseg_steps - 1) / c.kseg_steps);
    c.nk = (routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK;

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[a][0] = acc[a][1] = f32x16{};

    // live 32-row blocks of this wave (wave-uniform)
    int vblk = (t.rows - 128 * g + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > 4 ? 4 : vblk);
    vblk = __builtin_amdgcn_readfirstlane(vblk);
    switch (vblk) {  // every wave runs the same K loop; only the MFMA count differs
      case 4: mainloop<GATED, 4>(c, smem, acc); break;
      case 3: mainloop<GATED, 3>(c, smem, acc); break;
      case 2: mainloop<GATED, 2>(c, smem, acc); break;
      case 1: mainloop<GATED, 1>(c, smem, acc); break;
      default: mainloop<GATED, 0>(c, smem, acc); break;
    }

    // epilogue: C layout of the 32x32 MFMA -- lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4 of its 32x32 block
    const int col_in = lane % 32;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb >= vblk) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 128 * g + 32 * mb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
        if (i >= t.rows) continue;
        const int64_t m = t.m0 + i;
        if (GATED) {
          const int n = t.n0 + 32 * wn + col_in;
          const float h = silu(acc[mb][0][v]) * acc[mb][1][v];
          uint16_t* o = routed ? static_cast<uint16_t*>(args.out_routed) + (row_base + m) * args.ldo_routed + n
                               : static_cast<uint16_t*>(args.out_shared) + m * args.ldo_shared +
                                     static_cast<int64_t>(sg) * args.N + n;
          *o = f32_to_bf16(h);
        } else {
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int n = t.n0 + 64 * wn + 32 * nb + col_in;
            const float y = acc[mb][nb][v];
            if (routed)
              static_cast<uint16_t*>(args.out_routed)[(row_base + m) * args.ldo_routed + n] = f32_to_bf16(y);
            else
              static_cast<float*>(args.out_shared)[m * args.ldo_shared + n] = y;
          }
        }
      }
    }
  });
}

}  // namespace

size_t ffn_bf16_lds_bytes() { return 4 * kStageBytes; }

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

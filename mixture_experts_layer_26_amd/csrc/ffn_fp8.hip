// Grouped SwiGLU expert FFN with FP8 E4M3 operands on gfx950 (fp32 accumulate).
//
// FFN_i of the DeepSeek-V3 explainer's equation for h'_t (method section 2), with the
// FP8 scheme of its key ideas: activations in 1x128 tiles and weights in 128x128
// blocks, each with an fp32 scale (amax / 448, the quantisation pseudo-code of
// "DeepSeek モデルアーキテクチャ徹底解説"), products accumulated in fp32 and the
// partial sum of every 128-wide K block (the N_c = 128 interval) dequantised by the
// product of its two scales:
//   out[r, n] = sum_kb  s_a[r, kb] * s_w[n/128, kb] * (sum_{k in kb} qa[r, k] * qw[n, k])
// Phase 1 writes H = SiLU(gate) * up quantised per 1 x 128 (codes + fp32 scales);
// phase 2 writes y (bf16 routed rows, fp32 shared sum).
//
// The tile walk, tile claiming, LDS layout and ping-pong schedule are those of the bf16
// kernel (256 x 256 tiles, 128-byte rows per K-step, so one K-step is exactly one
// 128-wide scale block). The MFMA is v_mfma_scale_f32_16x16x128_f8f6f4 with unit
// (E8M0 = 127) scales: one instruction covers one scale block of a 16 x 16 output
// block, starting from zero, and its result is folded into the accumulator with one
// fp32 FMA per element: acc += blk * (s_a[row] * s_w). The fp32 scales are arbitrary
// (not powers of two), so they cannot ride in the MFMA's E8M0 scale operands.
#include "gemm_common.h"
#include "launch.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int BK = 128;  // fp8 elements (bytes) per K-step = one scale block
constexpr int kScaleBytes = BM * 4;  // one stage of A-row scales

struct TileCtx {
  const uint8_t* arow[4];   // this thread's 4 A rows (its 16-byte chunk)
  const uint8_t* b;         // this thread's first B row (chunk); rows +32*i
  const float* sa_row;      // A-row scales of row gr (threads with gt < 128: row 128g + gt)
  const float* sb[2];       // this wave's two B-scale rows (gate/up, or the wave's block)
  int64_t ldb;
  int64_t seg_stride;       // phase 2 shared: W2 stride per K segment, else 0
  int64_t sb_seg_stride;    // same for the W2 scales
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;
};

__device__ __forceinline__ i32x8 rd_frag(const unsigned char* base, int row, int q) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, 2 * q));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, 2 * q + 1));
  i32x8 f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// One K-step (one scale block) for a wave holding NM live 32-row blocks (2*NM 16-row
// MFMA blocks). sw[nb]: the weight scale of output block nb.
template <int NM>
__device__ __forceinline__ void compute_step(const unsigned char* la, const unsigned char* lb, const float* lsa,
                                             int arow0, const int (&brow)[4], const float (&sw)[4], int lane,
                                             f32x4 (&acc)[8][4]) {
  const int q = lane / 16;
  i32x8 bfr[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) bfr[nb] = rd_frag(lb, brow[nb], q);
#pragma unroll
  for (int mb = 0; mb < 2 * NM; ++mb) {
    const i32x8 af = rd_frag(la, arow0 + 16 * mb, q);
    // scales of this lane's 4 rows (16*mb + 4*q + v), contiguous in LDS
    const f32x4 sa = *reinterpret_cast<const f32x4*>(lsa + (arow0 - lane % 16) + 16 * mb + 4 * q);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x4 blk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[nb], f32x4{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(blk[v], sa[v] * sw[nb], acc[mb][nb][v]);
    }
  }
}

template <bool GATED, int NM>
__device__ __forceinline__ void mainloop(const TileCtx& c, unsigned char* smem, f32x4 (&acc)[8][4]) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = __builtin_amdgcn_readfirstlane(wave / 4), wn = wave % 4;
  const int gt = tid % 256, cc = gt % 8, cr = gt / 8;
  const int last = c.nk - 1;
  auto la = [&](int st) { return smem + st * kStageBytes; };
  auto lb = [&](int st) { return smem + 2 * kStageBytes + st * kStageBytes; };
  auto lsa = [&](int st) { return reinterpret_cast<float*>(smem + 4 * kStageBytes + st * kScaleBytes); };
  const int arow0 = 128 * g + lane % 16;
  int brow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (GATED)  // nb 0,1: gate rows; nb 2,3: the matching up rows
      brow[nb] = (nb < 2 ? 0 : 128) + 32 * wn + 16 * (nb & 1) + lane % 16;
    else
      brow[nb] = 64 * wn + 16 * nb + lane % 16;
  }
  uint4 ra[4], rb[4];
  float rs = 0.0f;
  auto gload = [&](int kt) {
    kt = kt < last ? kt : last;
    const int64_t aoff = static_cast<int64_t>(kt) * BK;
    const int64_t boff = b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, BK);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld16(c.arow[i] + aoff);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ld16(c.b + static_cast<int64_t>(32 * i) * c.ldb + boff);
    if (gt < 128) rs = c.sa_row[kt];
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 128 * g + cr + 32 * i;
      *reinterpret_cast<uint4*>(la(st) + swz(r, cc)) = ra[i];
      *reinterpret_cast<uint4*>(lb(st) + swz(r, cc)) = rb[i];
    }
    if (gt < 128) lsa(st)[128 * g + gt] = rs;
  };
  auto wscales = [&](int kt, float (&sw)[4]) {
    const int64_t o = b_offset(kt, c.kseg_steps, c.kseg_inv, c.sb_seg_stride, 1);
    const float s0 = c.sb[0][o], s1 = c.sb[1][o];
    sw[0] = sw[1] = s0;
    sw[2] = sw[3] = s1;
  };
  // In its memory half a group stores the registers loaded one K-step earlier, loads
  // the weight scales of its next compute half, then the tiles of the step after next
  // (in that order: the scales are waited for first, and loads complete in order).
  float sw[4];
  gload(0);
  lstore(0);
  if (g == 0) wscales(0, sw);
  gload(1);
  __syncthreads();
  for (int kt = 0; kt < c.nk; ++kt) {
    const int cur = kt & 1;
    if (g == 0) {
      compute_step<NM>(la(cur), lb(cur), lsa(cur), arow0, brow, sw, lane, acc);
    } else {
      lstore(cur ^ 1);
      wscales(kt, sw);
      gload(kt + 2);
    }
    lds_barrier();
    if (g == 1) {
      compute_step<NM>(la(cur), lb(cur), lsa(cur), arow0, brow, sw, lane, acc);
    } else {
      lstore(cur ^ 1);
      wscales(kt + 1 < last ? kt + 1 : last, sw);
      gload(kt + 2);
    }
    lds_barrier();
  }
}

__device__ __forceinline__ uint32_t e4m3(float x) {
  x = fminf(fmaxf(x, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false)) & 0xFFu;
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8(Fp8Args fa) {
  const GemmArgs& args = fa.g;
  __shared__ TileMap tm;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int n_r = args.n_r;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map(tm, args.offset, n_r, args.n_shared_groups, args.T, ntn);
  auto rows_of = [&](int grp) -> int64_t { return grp < n_r ? args.offset[grp + 1] - args.offset[grp] : args.T; };

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = wave / 4, wn = wave % 4;
  const int gt = tid % 256, cc = gt % 8, gr = gt / 8;
  const uint8_t* a_routed = reinterpret_cast<const uint8_t*>(args.a_routed);
  const uint8_t* a_shared = reinterpret_cast<const uint8_t*>(args.a_shared);

  for_each_tile(tm.total, args.sched, args.slot_stride, [&](int L) {
    const Tile t = tile_at(tm, L, n_r, bn_out, ntn, rows_of);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    TileCtx c;
    auto src_row = [&](int r) -> int64_t {  // A/scale row index of tile row r (clamped)
      if (r >= t.rows) r = t.rows - 1;
      const int64_t m = t.m0 + r;
      if (routed) return args.gather ? args.gather[row_base + m] : (row_base + m);
      return m;
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t src = src_row(128 * g + gr + 32 * i);
      c.arow[i] = (routed ? a_routed + src * args.lda_routed : a_shared + src * args.lda_shared) + cc * 16;
    }
    {
      const int64_t src = src_row(128 * g + (gt & 127));
      c.sa_row = routed ? fa.sa_routed + src * fa.ldsa_routed : fa.sa_shared + src * fa.ldsa_shared;
    }
    const int64_t eidx = routed ? t.group : sg;
    const int64_t eoff = eidx * args.b_expert_stride;
    const uint8_t* b1r = reinterpret_cast<const uint8_t*>(args.b1_routed);
    const uint8_t* b3r = reinterpret_cast<const uint8_t*>(args.b3_routed);
    const uint8_t* b1s = reinterpret_cast<const uint8_t*>(args.b1_shared);
    const uint8_t* b3s = reinterpret_cast<const uint8_t*>(args.b3_shared);
    const uint8_t* base;
    int64_t nrow;
    if (GATED) {
      base = (g == 0 ? (routed ? b1r : b1s) : (routed ? b3r : b3s)) + eoff;
      nrow = t.n0 + gr;
    } else {
      base = routed ? b1r + eoff : b1s;
      nrow = t.n0 + 128 * g + gr;
    }
    c.b = base + nrow * args.ldb + cc * 16;
    c.ldb = args.ldb;
    // weight-scale rows: [expert][N/128][K/128]
    const int64_t sbe = (routed || GATED) ? eidx * fa.sb_expert_stride : 0;
    if (GATED) {
      const int64_t nblk = t.n0 / 128;
      c.sb[0] = (routed ? fa.sb1_routed : fa.sb1_shared) + sbe + nblk * fa.kblocks;
      c.sb[1] = (routed ? fa.sb3_routed : fa.sb3_shared) + sbe + nblk * fa.kblocks;
    } else {
      const int64_t nblk = t.n0 / 128 + wn / 2;  // the wave's 64 columns lie in one block
      c.sb[0] = c.sb[1] = (routed ? fa.sb1_routed : fa.sb1_shared) + sbe + nblk * fa.kblocks;
    }
    c.seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.sb_seg_stride = (!routed && !GATED) ? fa.sb_expert_stride : 0;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = static_cast<uint32_t>((0x100000000ull + c.kseg_steps - 1) / c.kseg_steps);
    c.nk = (routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK;

    f32x4 acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{};

    int vblk = (t.rows - 128 * g + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > 4 ? 4 : vblk);
    vblk = __builtin_amdgcn_readfirstlane(vblk);
    switch (vblk) {
      case 4: mainloop<GATED, 4>(c, smem, acc); break;
      case 3: mainloop<GATED, 3>(c, smem, acc); break;
      case 2: mainloop<GATED, 2>(c, smem, acc); break;
      case 1: mainloop<GATED, 1>(c, smem, acc); break;
      default: mainloop<GATED, 0>(c, smem, acc); break;
    }

    // epilogue: C layout of the 16x16 MFMA -- lane holds column lane%16 and rows
    // 4*(lane/16) + v of its 16x16 block
    const int col_in = lane % 16, q = lane / 16;
    if (GATED) {
      // H = SiLU(gate) * up, then per-row 1x128 quantisation over the tile's 128 gate
      // columns (spread over the 4 waves of the group): amax per row via LDS
      float* amaxbuf = reinterpret_cast<float*>(smem);  // [4 waves][256 rows]
      float h[8][2][4];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float m = 0.0f;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            h[mb][nb][v] = silu(acc[mb][nb][v]) * acc[mb][nb + 2][v];
            m = fmaxf(m, fabsf(h[mb][nb][v]));
          }
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
          if (col_in == 0) amaxbuf[wn * 256 + 128 * g + 16 * mb + 4 * q + v] = m;
        }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = 128 * g + 16 * mb + 4 * q + v;
          const float amax = fmaxf(fmaxf(amaxbuf[i], amaxbuf[256 + i]), fmaxf(amaxbuf[512 + i], amaxbuf[768 + i]));
          if (i >= t.rows) continue;
          const float s = amax / 448.0f;
          const int64_t m = t.m0 + i;
          uint8_t* orow;
          float* srow;
          if (routed) {
            orow = reinterpret_cast<uint8_t*>(args.out_routed) + (row_base + m) * args.ldo_routed;
            srow = fa.os_routed + (row_base + m) * fa.ldos_routed;
          } else {
            orow = reinterpret_cast<uint8_t*>(args.out_shared) + m * args.ldo_shared +
                   static_cast<int64_t>(sg) * args.N;
            srow = fa.os_shared + m * fa.ldos_shared + static_cast<int64_t>(sg) * (args.N / 128);
          }
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int n = t.n0 + 32 * wn + 16 * nb + col_in;
            orow[n] = static_cast<uint8_t>(s == 0.0f ? 0u : e4m3(h[mb][nb][v] / s));
          }
          if (wn == 0 && col_in == 0) srow[t.n0 / 128] = s;
        }
      }
      __syncthreads();  // amaxbuf (LDS stage 0) is reused by the next tile
    } else {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        if (mb >= 2 * vblk) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int i = 128 * g + 16 * mb + 4 * q + v;
          if (i >= t.rows) continue;
          const int64_t m = t.m0 + i;
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int n = t.n0 + 64 * wn + 16 * nb + col_in;
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

size_t ffn_fp8_lds_bytes() { return 4 * kStageBytes + 2 * kScaleBytes; }

hipError_t launch_grouped_gemm_fp8(const Fp8Args& args, bool gated, int grid, hipStream_t stream) {
  const size_t lds = ffn_fp8_lds_bytes();
  const void* fn = gated ? reinterpret_cast<const void*>(grouped_gemm_fp8<true>)
                         : reinterpret_cast<const void*>(grouped_gemm_fp8<false>);
  hipError_t err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (err != hipSuccess) return err;
  if (gated)
    hipLaunchKernelGGL(grouped_gemm_fp8<true>, dim3(grid), dim3(kThreads), lds, stream, args);
  else
    hipLaunchKernelGGL(grouped_gemm_fp8<false>, dim3(grid), dim3(kThreads), lds, stream, args);
  return hipGetLastError();
}

}  // namespace moe

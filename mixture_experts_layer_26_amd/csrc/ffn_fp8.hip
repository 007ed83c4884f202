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

constexpr int BK = 128;                 // fp8 elements (bytes) per K-step = one scale block
constexpr int kOperand = BM * BK;       // 32 KB: one operand of one stage
constexpr int kScaleBytes = BM * 4;     // A-row scales of one stage
constexpr int kStageSize = 2 * kOperand + kScaleBytes;

// The two stages (A rows, B rows, A-row scales), one LDS array so that every load
// destination is a wave base plus a constant.
__shared__ __attribute__((aligned(16))) unsigned char stages[2 * kStageSize];

template <int ST>
__device__ __forceinline__ unsigned char* stage() {
  return stages + ST * kStageSize;
}

typedef __attribute__((address_space(3))) unsigned char* lds_ptr;

// One global_load_lds_dwordx4: lane i copies the 16 bytes at gptr (its own address) to
// LDS byte base + OFF + 16 i. M0 holds the LDS address (one wait state after writing
// it). The instruction is written out rather than taken from the builtin so that the
// compiler adds no wait of its own before the LDS reads; the waits are the explicit
// ones in step_barrier. Nothing else in these kernels uses M0.
template <int OFF>
__device__ __forceinline__ void dma16(const void* gptr, uint32_t base) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(base), "n"(OFF)
               : "memory");
}

// The same with 4 bytes per lane (lane i writes LDS byte base + OFF + 4 i).
template <int OFF>
__device__ __forceinline__ void dma4(const void* gptr, uint32_t base) {
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(base), "n"(OFF)
               : "memory");
}

struct TileCtx {
  uint32_t lds_wave;        // LDS address of this wave's rows (32 wave) in stage 0
  uint32_t lds_scale;       // waves 0..3: LDS address of row scales 64 wave.. in stage 0
  bool load_a;              // this wave's 32 A rows hold at least one of the tile's rows
  bool load_scale;          // waves 0..3 load the A-row scales (one row per lane)
  const uint8_t* a[4];      // this lane's four A rows (chunk included)
  const uint8_t* b;         // this lane's first B row (chunk included); row j: + 8 j ldb,
  int64_t ldb8;             //   and + odd_chunk for odd j (8 rows on, the swizzle term
  int odd_chunk;            //   (row/2)%8 differs by 4: the chunk index flips bit 2)
  const float* sa_row;      // threads 0..255: A-row scales of tile row tid (K-block 0)
  const float* sb[2];       // this wave's two B-scale rows (gate/up, or the wave's block)
  int64_t seg_stride;       // phase 2 shared: W2 stride per K segment, else 0
  int bstep;                // bytes from one K-step of a B row to the next
  int64_t sb_seg_stride;    // same for the W2 scales
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;
};

// Direct loads of K-step kt into stage ST: wave w fills A rows and B rows 32w..32w+31,
// four 8-row instructions each; lane i writes row 8j + i/8, 16-byte slot i%8, whose
// global chunk was chosen when the pointers were made. A wave whose A rows all lie past
// the tile's rows loads no A.
template <int ST>
__device__ __forceinline__ void dma_step(const TileCtx& c, int kt) {
  const int64_t aoff = static_cast<int64_t>(kt) * BK;
  const int64_t boff = b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, c.bstep);
  if (c.load_a) {
    dma16<ST * kStageSize + 0 * 8 * BK>(c.a[0] + aoff, c.lds_wave);
    dma16<ST * kStageSize + 1 * 8 * BK>(c.a[1] + aoff, c.lds_wave);
    dma16<ST * kStageSize + 2 * 8 * BK>(c.a[2] + aoff, c.lds_wave);
    dma16<ST * kStageSize + 3 * 8 * BK>(c.a[3] + aoff, c.lds_wave);
  }
  dma16<ST * kStageSize + kOperand + 0 * 8 * BK>(c.b + (boff + 0 * c.ldb8), c.lds_wave);
  dma16<ST * kStageSize + kOperand + 1 * 8 * BK>(c.b + (boff + 1 * c.ldb8 + c.odd_chunk), c.lds_wave);
  dma16<ST * kStageSize + kOperand + 2 * 8 * BK>(c.b + (boff + 2 * c.ldb8), c.lds_wave);
  dma16<ST * kStageSize + kOperand + 3 * 8 * BK>(c.b + (boff + 3 * c.ldb8 + c.odd_chunk), c.lds_wave);
  if (c.load_scale) dma4<ST * kStageSize>(c.sa_row + kt, c.lds_scale);
}

// A 16 x 128 fp8 fragment (rows row.., this lane's 32 bytes of K) from a swizzled stage.
__device__ __forceinline__ i32x8 rd_frag(const unsigned char* base, int row, int q) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, 2 * q));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, 2 * q + 1));
  i32x8 f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// Scheduling fence: the compiler moves no instruction across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// One K-step (one scale block) from stage ST for a wave holding NM live 32-row blocks
// (2*NM 16-row MFMA blocks). sw[p]: the weight scale of output blocks 2p, 2p+1. The
// MFMAs of a block start from a zero that an empty asm statement produces after the
// previous block's accumulators are final, so the compiler cannot hoist all MFMAs of
// the step ahead of their scaling (which would hold 32 MFMA results at once).
template <int ST, int NM>
__device__ __forceinline__ void compute_step(int arow0, const int (&brow)[4], const float (&sw)[2], int lane,
                                             f32x4 (&acc)[8][4]) {
  if constexpr (NM == 0) return;
  const unsigned char* la = stage<ST>();
  const unsigned char* lb = la + kOperand;
  const float* lsa = reinterpret_cast<const float*>(la + 2 * kOperand);
  const int q = lane / 16;
  i32x8 bfr[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) bfr[nb] = rd_frag(lb, brow[nb], q);
#pragma unroll
  for (int mb = 0; mb < 2 * NM; ++mb) {
    f32x4 zero = {};
    if (mb > 0)
      asm volatile("" : "+v"(zero) : "v"(acc[mb - 1][0]), "v"(acc[mb - 1][1]), "v"(acc[mb - 1][2]), "v"(acc[mb - 1][3]));
    const i32x8 af = rd_frag(la, arow0 + 16 * mb, q);
    // scales of this lane's 4 rows (16*mb + 4*q + v), contiguous in LDS
    const f32x4 sa = *reinterpret_cast<const f32x4*>(lsa + (arow0 - lane % 16) + 16 * mb + 4 * q);
    f32x4 prod[2];  // row scale x weight scale, per pair of output blocks
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int v = 0; v < 4; ++v) prod[p][v] = sa[v] * sw[p];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const f32x4 blk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[nb], zero, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mb][nb][v] = fmaf(blk[v], prod[nb / 2][v], acc[mb][nb][v]);
    }
  }
}

// Workgroup barrier at the end of a K-step: this wave's loads of the next step have
// landed (vmcnt(0)), its row scale of the next step is written to LDS, and its LDS
// operations are done; after the barrier every wave's part of the next step is in LDS
// and no wave reads the current stage any more.
__device__ __forceinline__ void step_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Weight scales of K-step kt for this wave's two pairs of output blocks.
__device__ __forceinline__ void wscales(const TileCtx& c, int kt, float (&sw)[2]) {
  const int64_t o = b_offset(kt, c.kseg_steps, c.kseg_inv, c.sb_seg_stride, 1);
  sw[0] = c.sb[0][o];
  sw[1] = c.sb[1][o];
}

// One K-step s from stage ST = s % 2. When MORE, step s+1 (tiles and row scales by
// DMA, the weight scales into sw for the next step) is loaded into the other stage
// while this one is computed.
template <int ST, int NM, bool MORE>
__device__ __forceinline__ void k_step(const TileCtx& c, int s, int arow0, const int (&brow)[4], int lane,
                                       float (&sw)[2], f32x4 (&acc)[8][4]) {
  float swn[2];
  if constexpr (MORE) {
    dma_step<(ST + 1) % 2>(c, s + 1);
    wscales(c, s + 1, swn);
  }
  fence();
  compute_step<ST, NM>(arow0, brow, sw, lane, acc);
  fence();
  if constexpr (MORE) {
    sw[0] = swn[0];
    sw[1] = swn[1];
  }
  step_barrier();
}

// The K loop of one tile: stage s % 2 is computed while step s+1 is loaded into the
// other stage. With an odd number of steps the first runs from stage 1, so the rest
// pair up (stage 0, stage 1). On exit no load is in flight and every wave is past the
// last read of the stages.
template <bool GATED, int NM>
__device__ __forceinline__ void mainloop(const TileCtx& c, f32x4 (&acc)[8][4]) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = wave / 4, wn = wave % 4;
  const int arow0 = 128 * g + lane % 16;
  int brow[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    if (GATED)  // nb 0,1: gate rows; nb 2,3: the matching up rows
      brow[nb] = (nb < 2 ? 0 : 128) + 32 * wn + 16 * (nb & 1) + lane % 16;
    else
      brow[nb] = 64 * wn + 16 * nb + lane % 16;
  }
  float sw[2];
  wscales(c, 0, sw);
  int s = 0;
  if (c.nk & 1) {  // odd: step 0 from stage 1, the rest in pairs as below
    dma_step<1>(c, 0);
    step_barrier();
    k_step<1, NM, true>(c, 0, arow0, brow, lane, sw, acc);
    s = 1;
  } else {
    dma_step<0>(c, 0);
    step_barrier();
  }
  for (; s + 2 < c.nk; s += 2) {
    k_step<0, NM, true>(c, s, arow0, brow, lane, sw, acc);
    k_step<1, NM, true>(c, s + 1, arow0, brow, lane, sw, acc);
  }
  k_step<0, NM, true>(c, s, arow0, brow, lane, sw, acc);
  k_step<1, NM, false>(c, s + 1, arow0, brow, lane, sw, acc);
}

__device__ __forceinline__ uint32_t e4m3(float x) {
  x = fminf(fmaxf(x, -448.0f), 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(x, x, 0, false)) & 0xFFu;
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_fp8(Fp8Args fa) {
  const GemmArgs& args = fa.g;
  __shared__ TileMap tm;

  const int n_r = args.n_r;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map(tm, args.offset, n_r, args.n_shared_groups, args.T, ntn);
  auto rows_of = [&](int grp) -> int64_t { return grp < n_r ? args.offset[grp + 1] - args.offset[grp] : args.T; };

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = wave / 4, wn = wave % 4;
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
    const int64_t eidx = routed ? t.group : sg;
    const int64_t eoff = eidx * args.b_expert_stride;
    const uint8_t* b1r = reinterpret_cast<const uint8_t*>(args.b1_routed);
    const uint8_t* b3r = reinterpret_cast<const uint8_t*>(args.b3_routed);
    const uint8_t* b1s = reinterpret_cast<const uint8_t*>(args.b1_shared);
    const uint8_t* b3s = reinterpret_cast<const uint8_t*>(args.b3_shared);
    c.load_a = __builtin_amdgcn_readfirstlane(32 * wave < t.rows ? 1 : 0) != 0;
    {
      const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(stages)));
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      c.lds_wave = lds0 + static_cast<uint32_t>(32 * wv * BK);
      c.lds_scale = lds0 + static_cast<uint32_t>(2 * kOperand + 4 * kWave * wv);
      c.load_scale = wv < BM / kWave;
    }
    // this lane's load rows: 32*wave + 8j + lane/8 of the tile, slot lane%8, holding
    // global chunk slot ^ ((row/2)%8) (the swizzle of swz)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * wave + 8 * j + lane / 8;
      const int chunk = (lane % 8) ^ ((r >> 1) & 7);
      const int64_t src = src_row(r);
      c.a[j] = (routed ? a_routed + src * args.lda_routed : a_shared + src * args.lda_shared) + chunk * 16;
    }
    {
      const int r = 32 * wave + lane / 8;
      const int chunk = (lane % 8) ^ ((r >> 1) & 7);
      const uint8_t* base;
      int64_t nrow;
      if (GATED) {  // tile rows 0..127 gate, 128..255 up (a wave's 32 rows lie in one)
        base = (r < 128 ? (routed ? b1r : b1s) : (routed ? b3r : b3s)) + eoff;
        nrow = t.n0 + (r & 127);
      } else {
        base = routed ? b1r + eoff : b1s;
        nrow = t.n0 + r;
      }
      if (args.b_tiled) {  // [E][N/R][K/128][R][128]: one K-step of the tile is R contiguous rows
        constexpr int R = GATED ? 128 : 256;
        c.b = base + (t.n0 / R) * (args.ldb / BK) * (R * BK) + static_cast<int64_t>(nrow - t.n0) * BK + chunk * 16;
        c.ldb8 = 8 * BK;
      } else {
        c.b = base + nrow * args.ldb + chunk * 16;
        c.ldb8 = 8 * args.ldb;
      }
      c.odd_chunk = ((chunk ^ 4) - chunk) * 16;
    }
    {
      const int64_t src = src_row(tid & (BM - 1));
      c.sa_row = routed ? fa.sa_routed + src * fa.ldsa_routed : fa.sa_shared + src * fa.ldsa_shared;
    }
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
    c.bstep = args.b_tiled ? (GATED ? 128 : 256) * BK : BK;
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
    switch (vblk) {  // every wave runs the same loads and barriers; only the MFMA count differs
      case 4: mainloop<GATED, 4>(c, acc); break;
      case 3: mainloop<GATED, 3>(c, acc); break;
      case 2: mainloop<GATED, 2>(c, acc); break;
      case 1: mainloop<GATED, 1>(c, acc); break;
      default: mainloop<GATED, 0>(c, acc); break;
    }

    // epilogue: C layout of the 16x16 MFMA -- lane holds column lane%16 and rows
    // 4*(lane/16) + v of its 16x16 block
    const int col_in = lane % 16, q = lane / 16;
    if (GATED) {
      // H = SiLU(gate) * up, then per-row 1x128 quantisation over the tile's 128 gate
      // columns (spread over the 4 waves of the group): amax per row via LDS
      float* amaxbuf = reinterpret_cast<float*>(stage<0>());  // [4 waves][256 rows]
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

size_t ffn_fp8_lds_bytes() { return 2 * kStageSize; }

hipError_t launch_grouped_gemm_fp8(const Fp8Args& args, bool gated, int grid, hipStream_t stream) {
  if (args.g.K % BK != 0) return hipErrorInvalidValue;
  if (gated)
    hipLaunchKernelGGL(grouped_gemm_fp8<true>, dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(grouped_gemm_fp8<false>, dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace moe

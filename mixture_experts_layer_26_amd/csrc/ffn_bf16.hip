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
// tile list in gangs (gemm_common.h). A tile is up to 256 rows x 256 weight rows (phase
// 1: 128 gate + 128 up columns). K advances in steps of 64 (128-byte rows) through two
// LDS stages filled by direct global-to-LDS loads (global_load_lds_dwordx4): no staging
// registers and no LDS store instructions; a stage is loaded one step before it is
// computed. One barrier per step, before its last 16-wide sub-step, so each wave reads
// the next step's first fragments while the MFMAs of the current one run. Every wave
// computes a 128 x 64 block with v_mfma_f32_32x32x16_bf16 (8 MFMA tiles): wave (g, wn)
// owns rows 128g.. of the tile and, in phase 1, gate rows 32wn.. and the matching up
// rows (so SiLU(gate) * up is formed in registers). The K loop is specialised on the
// number of 32-row blocks of a wave that hold rows, so row blocks past an expert's
// count cost no MFMA work. Weights are read row-major or in the tiled layout of
// pack.hip.
#include "gemm_common.h"
#include "launch.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int BK = 64;                  // bf16 per K-step: 128-byte rows (whole cache lines)
constexpr int kRow = 128;               // bytes per tile row per stage
constexpr int kOperand = BM * kRow;     // 32 KB: one operand of one stage
constexpr int kStages = 2;
constexpr int kSubs = BK / 16;          // MFMA sub-steps per K-step
constexpr int kDmaPerStep = 8;          // global_load_lds per wave per step (4 A + 4 B)

// The two stages.
__shared__ __attribute__((aligned(16))) unsigned char stage0[2 * kOperand];
__shared__ __attribute__((aligned(16))) unsigned char stage1[2 * kOperand];

template <int ST>
__device__ __forceinline__ unsigned char* stage() {
  if constexpr (ST == 0) return stage0;
  else return stage1;
}

typedef __attribute__((address_space(3))) unsigned char* lds_ptr;

// One global_load_lds_dwordx4: lane i copies the 16 bytes at gptr (its own address) to
// LDS byte lds + 16 i. M0 holds the LDS address (one wait state after writing it). The
// instruction is written out rather than taken from the builtin so that the compiler,
// which cannot follow which stage a load lands in across loop iterations, adds no wait
// of its own before the LDS reads; the waits are the explicit ones in step_barrier.
// Nothing else in these kernels uses M0.
__device__ __forceinline__ void dma16(const void* gptr, const unsigned char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0) : "memory");
}

struct TileCtx {
  bool load_a;           // this wave's 32 A rows hold at least one of the tile's rows
  const uint16_t* a[4];  // this lane's four A rows (chunk included)
  const uint16_t* b[4];  // this lane's four B rows (chunk included)
  int64_t seg_stride;    // phase 2 shared: W2 stride per K segment, else 0
  int bstep;             // elements from one K-step of a B row to the next
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;                // K-steps
};

// Direct loads of K-step kt into stage ST: wave w fills A rows and B rows 32w..32w+31,
// four 8-row instructions each; lane i writes row 8j + i/8 of its instruction's block,
// 16-byte slot i%8, whose global chunk was chosen when the pointers were made. A wave
// whose A rows all lie past the tile's rows loads no A (those LDS rows feed only
// outputs that are not stored).
template <int ST>
__device__ __forceinline__ void dma_step(const TileCtx& c, int kt, int wave) {
  unsigned char* st = stage<ST>();
  const int64_t aoff = static_cast<int64_t>(kt) * BK;
  const int64_t boff = b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, c.bstep);
  if (c.load_a) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(c.a[j] + aoff, st + (32 * wave + 8 * j) * kRow);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) dma16(c.b[j] + boff, st + kOperand + (32 * wave + 8 * j) * kRow);
}

// Fragments of one 16-wide sub-step of stage ST for a wave holding NMB live 32-row
// blocks: NMB A fragments (rows arow0 + 32 mb) and two B fragments (rows brow).
template <int NMB>
struct Frags {
  bf16x8 a[NMB > 0 ? NMB : 1];
  bf16x8 b[2];
};

template <int ST, int NMB>
__device__ __forceinline__ void read_frags(Frags<NMB>& f, int sub, int arow0, const int (&brow)[2], int lane) {
  const unsigned char* la = stage<ST>();
  const unsigned char* lb = la + kOperand;
  const int ch = 2 * sub + lane / 32;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) f.a[mb] = *reinterpret_cast<const bf16x8*>(la + swz(arow0 + 32 * mb, ch));
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) f.b[nb] = *reinterpret_cast<const bf16x8*>(lb + swz(brow[nb], ch));
}

// MFMA i (0 .. 2 NMB - 1) of a sub-step: row block i / 2, column block i % 2.
template <int NMB>
__device__ __forceinline__ void mfma_one(const Frags<NMB>& f, f32x16 (&acc)[4][2], int i) {
  const int mb = i / 2, nb = i % 2;
  acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mb], f.b[nb], acc[mb][nb], 0, 0, 0);
}

template <int NMB>
__device__ __forceinline__ void mfma_sub(const Frags<NMB>& f, f32x16 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 2 * NMB; ++i) mfma_one(f, acc, i);
}

// Scheduling fence: the compiler moves no instruction across it, so the order written
// below (MFMAs, barrier, loads, reads) is the order issued.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Wait until this wave's LDS reads have returned and its loads of the next step have
// landed (NEWER loads issued after them may stay in flight), then the workgroup
// barrier: after it every wave's part of the next step is in LDS and no wave reads the
// current step's stage any more. Loads complete in order, so any extra memory
// operation only makes the wait stricter.
template <int NEWER>
__device__ __forceinline__ void step_barrier() {
  if constexpr (NEWER == 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (NEWER == 4)
    asm volatile("s_waitcnt vmcnt(4)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
static_assert(kDmaPerStep == 8, "step_barrier's wait counts assume 8 loads per step (4 without A)");

// One K-step s from stage ST = s % 2, four 16-wide sub-steps. Fragment sets f0 and f1
// alternate: each sub-step's MFMAs run while the sub-step after next is read. On entry
// sub-steps 0 and 1 have been requested. The barrier sits before the last sub-step: the
// wave has then issued every read of stage ST, so after it stage ST takes the load of
// step s+2 (when DMA) and the next step's first two sub-steps are read from the other
// stage (loaded one step ago, landed; when READ) while the last sub-step runs.
template <int ST, int NMB, bool DMA, bool READ>
__device__ __forceinline__ void k_step(const TileCtx& c, int s, int wave, int arow0, const int (&brow)[2],
                                       int lane, Frags<NMB>& f0, Frags<NMB>& f1, f32x16 (&acc)[4][2]) {
  constexpr int NMF = 2 * NMB;
  mfma_sub(f0, acc);
  fence();
  read_frags<ST, NMB>(f0, 2, arow0, brow, lane);
  fence();
  mfma_sub(f1, acc);
  fence();
  read_frags<ST, NMB>(f1, 3, arow0, brow, lane);
  fence();
  mfma_sub(f0, acc);
  fence();
  step_barrier<0>();
  fence();
  if constexpr (NMF > 0) mfma_one(f1, acc, 0);
  fence();
  if constexpr (DMA) dma_step<ST>(c, s + kStages, wave);
  fence();
  if constexpr (NMF > 1) mfma_one(f1, acc, 1);
  fence();
  if constexpr (READ) read_frags<(ST + 1) % kStages, NMB>(f0, 0, arow0, brow, lane);
  fence();
#pragma unroll
  for (int i = 2; i < NMF; ++i) mfma_one(f1, acc, i);
  fence();
  if constexpr (READ) read_frags<(ST + 1) % kStages, NMB>(f1, 1, arow0, brow, lane);
  fence();
}

// The K loop of one tile. nk is even (K is a multiple of 128): the loop runs all but
// the last two steps, which load nothing. On exit no load is in flight and every wave
// is past the last read of the stages.
template <int NMB>
__device__ __forceinline__ void mainloop(const TileCtx& c, f32x16 (&acc)[4][2], int arow0, const int (&brow)[2]) {
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  dma_step<0>(c, 0, wave);
  dma_step<1>(c, 1, wave);
  // step 0 landed; step 1 (8 loads, or 4 without A) in flight
  if (c.load_a)
    step_barrier<kDmaPerStep>();
  else
    step_barrier<kDmaPerStep / 2>();
  Frags<NMB> f0, f1;
  read_frags<0, NMB>(f0, 0, arow0, brow, lane);
  read_frags<0, NMB>(f1, 1, arow0, brow, lane);
  int s = 0;
  for (; s < c.nk - kStages; s += kStages) {
    k_step<0, NMB, true, true>(c, s, wave, arow0, brow, lane, f0, f1, acc);
    k_step<1, NMB, true, true>(c, s + 1, wave, arow0, brow, lane, f0, f1, acc);
  }
  k_step<0, NMB, false, true>(c, s, wave, arow0, brow, lane, f0, f1, acc);
  k_step<1, NMB, false, false>(c, s + 1, wave, arow0, brow, lane, f0, f1, acc);
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16(GemmArgs args) {
  __shared__ TileMap tm;

  const int n_r = args.n_r;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map(tm, args.offset, n_r, args.n_shared_groups, args.T, ntn);
  auto rows_of = [&](int grp) -> int64_t { return grp < n_r ? args.offset[grp + 1] - args.offset[grp] : args.T; };

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = wave / 4, wn = wave % 4;

  for_each_tile(tm.total, args.sched, args.slot_stride, [&](int L) {
    const Tile t = tile_at(tm, L, n_r, bn_out, ntn, rows_of);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;  // shared group index
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    TileCtx c;
    // this lane's load rows: 32*wave + 8j + lane/8 of the tile, slot lane%8, holding
    // global chunk slot ^ ((row/2)%8) (the swizzle of swz)
    const int64_t eoff = static_cast<int64_t>(routed ? t.group : sg) * args.b_expert_stride;
    c.load_a = __builtin_amdgcn_readfirstlane(32 * wave < t.rows ? 1 : 0) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 32 * wave + 8 * j + lane / 8;
      const int chunk = (lane % 8) ^ ((r >> 1) & 7);
      // A row (rows past the tile's valid rows repeat its last one)
      const int ra = r < t.rows ? r : t.rows - 1;
      const int64_t m = t.m0 + ra;
      if (routed) {
        const int64_t src = args.gather ? args.gather[row_base + m] : (row_base + m);
        c.a[j] = args.a_routed + src * args.lda_routed + chunk * 8;
      } else {
        c.a[j] = args.a_shared + m * args.lda_shared + chunk * 8;
      }
      // B row: tile rows 0..127 gate and 128..255 up when gated
      const uint16_t* base;
      int64_t nrow;
      if (GATED) {
        const bool up = r >= 128;
        base = (up ? (routed ? args.b3_routed : args.b3_shared) : (routed ? args.b1_routed : args.b1_shared)) + eoff;
        nrow = t.n0 + (r & 127);
      } else {
        base = routed ? args.b1_routed + eoff : args.b1_shared;
        nrow = t.n0 + r;
      }
      if (args.b_tiled) {  // [E][N/R][K/64][R][64]: one K-step of the tile is R contiguous rows
        constexpr int R = GATED ? 128 : 256;
        c.b[j] = base + (t.n0 / R) * (args.ldb / BK) * (R * BK) + static_cast<int64_t>(nrow - t.n0) * BK + chunk * 8;
      } else {
        c.b[j] = base + nrow * args.ldb + chunk * 8;
      }
    }
    c.seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.bstep = args.b_tiled ? (GATED ? 128 : 256) * BK : BK;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = kseg_recip(c.kseg_steps);
    c.nk = (routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK;

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[a][0] = acc[a][1] = f32x16{};

    const int arow0 = 128 * g + lane % 32;
    int brow[2];
    if (GATED) {  // gate block and the matching up block
      brow[0] = 32 * wn + lane % 32;
      brow[1] = 128 + 32 * wn + lane % 32;
    } else {
      brow[0] = 64 * wn + lane % 32;
      brow[1] = 64 * wn + 32 + lane % 32;
    }
    // live 32-row blocks of this wave (wave-uniform)
    int vblk = (t.rows - 128 * g + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > 4 ? 4 : vblk);
    vblk = __builtin_amdgcn_readfirstlane(vblk);
    switch (vblk) {  // every wave runs the same loads and barriers; only the MFMA count differs
      case 4: mainloop<4>(c, acc, arow0, brow); break;
      case 3: mainloop<3>(c, acc, arow0, brow); break;
      case 2: mainloop<2>(c, acc, arow0, brow); break;
      case 1: mainloop<1>(c, acc, arow0, brow); break;
      default: mainloop<0>(c, acc, arow0, brow); break;
    }

    // epilogue. C layout of the 32x32 MFMA: lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4 of its 32x32 block.
    const int col_in = lane % 32;
    if (GATED || routed) {
      // bf16 outputs go through LDS (the stages are free once the K loop is done): group
      // g writes its 128 rows as a [128][W] bf16 tile into stage g, then its 256 threads
      // store whole rows with 16-byte stores. Rows whose bit 2 is set have their 64-byte
      // halves swapped, so the two half-waves' 2-byte writes (rows r and r+4) fall in
      // different banks.
      constexpr int W = GATED ? BNB / 2 : BNB;  // output columns of the tile
      constexpr int pitch = 2 * W;               // bytes per row
      unsigned char* ep = g == 0 ? stage<0>() : stage<1>();
      auto eoff = [](int r, int byte) { return r * pitch + (byte ^ (((r >> 2) & 1) << 6)); };
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb >= vblk) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * mb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
          if (GATED) {
            const float h = silu(acc[mb][0][v]) * acc[mb][1][v];
            *reinterpret_cast<uint16_t*>(ep + eoff(r, 2 * (32 * wn + col_in))) = f32_to_bf16(h);
          } else {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
              *reinterpret_cast<uint16_t*>(ep + eoff(r, 2 * (64 * wn + 32 * nb + col_in))) =
                  f32_to_bf16(acc[mb][nb][v]);
          }
        }
      }
      __syncthreads();
      const int gt = tid % 256;
      constexpr int cpr = pitch / 16;  // 16-byte chunks per row
      const int rows_g = t.rows - 128 * g;
      for (int idx = gt; idx < 128 * cpr; idx += 256) {
        const int r = idx / cpr, ch = idx % cpr;
        if (r >= rows_g) break;
        const uint4 val = *reinterpret_cast<const uint4*>(ep + eoff(r, 16 * ch));
        const int64_t m = t.m0 + 128 * g + r;
        uint16_t* dst = routed ? static_cast<uint16_t*>(args.out_routed) + (row_base + m) * args.ldo_routed
                               : static_cast<uint16_t*>(args.out_shared) + m * args.ldo_shared +
                                     static_cast<int64_t>(sg) * args.N;
        st16(dst + t.n0 + 8 * ch, val);
      }
    } else {
      // fp32 shared-expert sum: direct stores
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb >= vblk) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = 128 * g + 32 * mb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
          if (i >= t.rows) continue;
          const int64_t m = t.m0 + i;
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            const int n = t.n0 + 64 * wn + 32 * nb + col_in;
            static_cast<float*>(args.out_shared)[m * args.ldo_shared + n] = acc[mb][nb][v];
          }
        }
      }
    }
  });
}

}  // namespace

size_t ffn_bf16_lds_bytes() { return kStages * 2 * kOperand; }

hipError_t launch_grouped_gemm_bf16(const GemmArgs& args, bool gated, int grid, hipStream_t stream) {
  if (args.K % (kStages * BK) != 0) return hipErrorInvalidValue;
  if (gated)
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace moe

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
// tile list in gangs (gemm_common.h). A phase-1 tile is up to 320 rows x 256 weight rows
// (128 gate + 128 up columns): at V3 prefill the routed experts hold about 185..345 rows,
// so with 320-row tiles most experts are one row block and their weights pass through the
// L1 once, where 256-row tiles split about 120 of the 256 experts in two. K advances in
// steps of 64 (128-byte rows) through two LDS stages filled by direct global-to-LDS loads (global_load_lds_dwordx4): no staging
// registers and no LDS store instructions; a stage is loaded one step before it is
// computed. One barrier per step, before its last 16-wide sub-step, so each wave reads
// the next step's first fragments while the MFMAs of the current one run. In phase 1
// every wave computes a 160 x 64 block with v_mfma_f32_32x32x16_bf16 (10 MFMA tiles):
// wave (g, wn) owns rows 160g.. of the tile and gate rows 32wn.. with the matching up
// rows (so SiLU(gate) * up is formed in registers). Phase 2 keeps 256-row tiles (waves
// of 128 x 64, 8 MFMA tiles): at 320 rows its kernel, which also carries the shared
// experts' segmented K range and fp32 epilogue, spilled registers inside the K loop. The K loop is specialised on the
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
constexpr int kOpB = BNB * kRow;        // 32 KB: the B rows of one stage
constexpr int kStages = 2;
constexpr int kSubs = BK / 16;          // MFMA sub-steps per K-step
constexpr int kDmaB = BNB / 64;         // B loads (global_load_lds of 8 rows) per wave per step

// Tile geometry for TRW tile rows: two wave groups of TRW / 2 rows, each wave a
// TRW / 2 x 64 block of 32 x 32 MFMA tiles. Phase 1 uses 320 rows, phase 2 256 (at 320 the
// down-projection spilled registers inside its K loop).
template <int TRW>
struct Geo {
  static constexpr int GR = TRW / 2;      // rows per wave group
  static constexpr int kMB = GR / 32;     // 32-row blocks per wave
  static constexpr int kOpA = TRW * kRow; // the A rows of one stage
  static constexpr int kDmaA = TRW / 64;  // A loads per wave per step
};
constexpr int kTR1 = 320, kTR2 = 256;     // tile rows of phase 1 and phase 2
constexpr int kStageSz = Geo<kTR1>::kOpA + kOpB;  // 72 KB

// The two stages.
__shared__ __attribute__((aligned(16))) unsigned char stage0[kStageSz];
__shared__ __attribute__((aligned(16))) unsigned char stage1[kStageSz];

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

template <int TRW>
struct TileCtx {
  bool load_a;                // this wave's A rows hold at least one of the tile's rows
  const uint16_t* abase;      // wave-uniform base of the A operand
  uint32_t a[Geo<TRW>::kDmaA];  // this lane's A rows: element offsets from abase (chunk included)
  const uint16_t* bbase;      // wave-uniform base of this wave's B rows
  uint32_t b[kDmaB];          // this lane's four B rows: element offsets from bbase (chunk included)
  int64_t seg_stride;    // phase 2 shared: W2 stride per K segment, else 0
  int bstep;             // elements from one K-step of a B row to the next
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;                // K-steps
};

// Direct loads of K-step kt into stage ST: wave w fills A rows 8 kDmaA w.. (kDmaA 8-row
// instructions: 40 rows in phase 1, 32 in phase 2) and B rows 32w..32w+31 (four); lane i
// writes row 8j + i/8 of its
// instruction's block, 16-byte slot i%8, whose global chunk was chosen when the pointers
// were made. A wave whose A rows all lie past the tile's rows loads no A (those LDS rows
// feed only outputs that are not stored).
template <int ST, int TRW>
__device__ __forceinline__ void dma_step(const TileCtx<TRW>& c, int kt, int wave) {
  constexpr int kDmaA = Geo<TRW>::kDmaA, kOpA = Geo<TRW>::kOpA;
  unsigned char* st = stage<ST>();
  const int64_t aoff = static_cast<int64_t>(kt) * BK;
  const int64_t boff = b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, c.bstep);
  if (c.load_a) {
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) dma16(c.abase + (aoff + c.a[j]), st + (8 * kDmaA * wave + 8 * j) * kRow);
  }
#pragma unroll
  for (int j = 0; j < kDmaB; ++j) dma16(c.bbase + (boff + c.b[j]), st + kOpA + (8 * kDmaB * wave + 8 * j) * kRow);
}

// Fragments of one 16-wide sub-step of stage ST for a wave holding NMB live 32-row
// blocks: NMB A fragments (rows arow0 + 32 mb) and two B fragments (rows brow).
template <int NMB>
struct Frags {
  bf16x8 a[NMB > 0 ? NMB : 1];
  bf16x8 b[2];
};

template <int ST, int TRW, int NMB>
__device__ __forceinline__ void read_frags(Frags<NMB>& f, int sub, int arow0, const int (&brow)[2], int lane) {
  const unsigned char* la = stage<ST>();
  const unsigned char* lb = la + Geo<TRW>::kOpA;
  const int ch = 2 * sub + lane / 32;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) f.a[mb] = *reinterpret_cast<const bf16x8*>(la + swz(arow0 + 32 * mb, ch));
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) f.b[nb] = *reinterpret_cast<const bf16x8*>(lb + swz(brow[nb], ch));
}

// MFMA i (0 .. 2 NMB - 1) of a sub-step: row block i / 2, column block i % 2.
template <int KMB, int NMB>
__device__ __forceinline__ void mfma_one(const Frags<NMB>& f, f32x16 (&acc)[KMB][2], int i) {
  const int mb = i / 2, nb = i % 2;
  acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[mb], f.b[nb], acc[mb][nb], 0, 0, 0);
}

template <int KMB, int NMB>
__device__ __forceinline__ void mfma_sub(const Frags<NMB>& f, f32x16 (&acc)[KMB][2]) {
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
  static_assert(NEWER >= 0 && NEWER < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(NEWER) : "memory");
}

// One K-step s from stage ST = s % 2, four 16-wide sub-steps. Fragment sets f0 and f1
// alternate: each sub-step's MFMAs run while the sub-step after next is read. On entry
// sub-steps 0 and 1 have been requested. The barrier sits before the last sub-step: the
// wave has then issued every read of stage ST, so after it stage ST takes the load of
// step s+2 (when DMA) and the next step's first two sub-steps are read from the other
// stage (loaded one step ago, landed; when READ) while the last sub-step runs.
template <int ST, int TRW, int NMB, bool DMA, bool READ>
__device__ __forceinline__ void k_step(const TileCtx<TRW>& c, int s, int wave, int arow0, const int (&brow)[2],
                                       int lane, Frags<NMB>& f0, Frags<NMB>& f1,
                                       f32x16 (&acc)[Geo<TRW>::kMB][2]) {
  constexpr int NMF = 2 * NMB;
  mfma_sub(f0, acc);
  fence();
  read_frags<ST, TRW, NMB>(f0, 2, arow0, brow, lane);
  fence();
  mfma_sub(f1, acc);
  fence();
  read_frags<ST, TRW, NMB>(f1, 3, arow0, brow, lane);
  fence();
  mfma_sub(f0, acc);
  fence();
  step_barrier<0>();
  fence();
  if constexpr (NMF > 0) mfma_one(f1, acc, 0);
  fence();
  if constexpr (DMA) dma_step<ST, TRW>(c, s + kStages, wave);
  fence();
  if constexpr (NMF > 1) mfma_one(f1, acc, 1);
  fence();
  if constexpr (READ) read_frags<(ST + 1) % kStages, TRW, NMB>(f0, 0, arow0, brow, lane);
  fence();
#pragma unroll
  for (int i = 2; i < NMF; ++i) mfma_one(f1, acc, i);
  fence();
  if constexpr (READ) read_frags<(ST + 1) % kStages, TRW, NMB>(f1, 1, arow0, brow, lane);
  fence();
}

// The K loop of one tile. nk is even (K is a multiple of 128): the loop runs all but
// the last two steps, which load nothing. On exit no load is in flight and every wave
// is past the last read of the stages.
template <int TRW, int NMB>
__device__ __forceinline__ void mainloop(const TileCtx<TRW>& c, f32x16 (&acc)[Geo<TRW>::kMB][2], int arow0,
                                         const int (&brow)[2]) {
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  dma_step<0, TRW>(c, 0, wave);
  dma_step<1, TRW>(c, 1, wave);
  // step 0 landed; step 1 (kDmaA + 4 loads, or 4 without A) in flight
  if (c.load_a)
    step_barrier<Geo<TRW>::kDmaA + kDmaB>();
  else
    step_barrier<kDmaB>();
  Frags<NMB> f0, f1;
  read_frags<0, TRW, NMB>(f0, 0, arow0, brow, lane);
  read_frags<0, TRW, NMB>(f1, 1, arow0, brow, lane);
  int s = 0;
  for (; s < c.nk - kStages; s += kStages) {
    k_step<0, TRW, NMB, true, true>(c, s, wave, arow0, brow, lane, f0, f1, acc);
    k_step<1, TRW, NMB, true, true>(c, s + 1, wave, arow0, brow, lane, f0, f1, acc);
  }
  k_step<0, TRW, NMB, false, true>(c, s, wave, arow0, brow, lane, f0, f1, acc);
  k_step<1, TRW, NMB, false, false>(c, s + 1, wave, arow0, brow, lane, f0, f1, acc);
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16(GemmArgs args) {
  __shared__ TileMap tm;
  constexpr int TR = GATED ? kTR1 : kTR2;
  using G = Geo<TR>;
  constexpr int GR = G::GR, kMB = G::kMB, kDmaA = G::kDmaA;

  const int n_r = args.n_r;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map<TR>(tm, args.offset, n_r, args.n_shared_groups, args.T, ntn);
  auto rows_of = [&](int grp) -> int64_t { return grp < n_r ? args.offset[grp + 1] - args.offset[grp] : args.T; };

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = wave / 4, wn = wave % 4;

  for_each_tile(tm.total, args.sched, args.slot_stride, [&](int L) {
    const Tile t = tile_at(tm, L, n_r, bn_out, ntn, rows_of);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;  // shared group index
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    TileCtx<TR> c;
    // this lane's load rows: 8*kDmaA*wave + 8j + lane/8 of the tile's A rows and 32*wave + 8j +
    // lane/8 of its B rows, slot lane%8, holding global chunk slot ^ ((row/2)%8) (the
    // swizzle of swz)
    const int64_t eoff = static_cast<int64_t>(routed ? t.group : sg) * args.b_expert_stride;
    c.load_a = __builtin_amdgcn_readfirstlane(8 * kDmaA * wave < t.rows ? 1 : 0) != 0;
    // element offsets fit 32 bits: moe_grouped_ffn rejects bf16 operands of 2^32 elements or more
    c.abase = routed ? args.a_routed : args.a_shared;
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) {
      const int r = 8 * kDmaA * wave + 8 * j + lane / 8;
      const int chunk = (lane % 8) ^ ((r >> 1) & 7);
      // rows past the tile's valid rows repeat its last one
      const int ra = r < t.rows ? r : t.rows - 1;
      const int64_t m = t.m0 + ra;
      const int64_t src = routed ? (args.gather ? args.gather[row_base + m] : (row_base + m)) : m;
      c.a[j] = static_cast<uint32_t>(src * (routed ? args.lda_routed : args.lda_shared) + chunk * 8);
    }
    {
      // B rows 32*wave..: in phase 1 waves 0..3 hold gate rows and 4..7 up rows, so the
      // matrix is wave-uniform
      const bool up = GATED && wave >= 4;
      const uint16_t* base = GATED ? (up ? (routed ? args.b3_routed : args.b3_shared)
                                         : (routed ? args.b1_routed : args.b1_shared)) + eoff
                                   : (routed ? args.b1_routed + eoff : args.b1_shared);
      constexpr int R = GATED ? 128 : 256;  // tiled layout: [E][N/R][K/64][R][64]
      c.bbase = args.b_tiled ? base + (t.n0 / R) * (args.ldb / BK) * (R * BK) : base;
#pragma unroll
      for (int j = 0; j < kDmaB; ++j) {
        const int r = 8 * kDmaB * wave + 8 * j + lane / 8;
        const int chunk = (lane % 8) ^ ((r >> 1) & 7);
        const int64_t nrow = t.n0 + (GATED ? (r & 127) : r);
        c.b[j] = static_cast<uint32_t>(args.b_tiled ? (nrow - t.n0) * BK + chunk * 8 : nrow * args.ldb + chunk * 8);
      }
    }
    c.seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.bstep = args.b_tiled ? (GATED ? 128 : 256) * BK : BK;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = kseg_recip(c.kseg_steps);
    c.nk = (routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK;

    f32x16 acc[kMB][2];
#pragma unroll
    for (int a = 0; a < kMB; ++a) acc[a][0] = acc[a][1] = f32x16{};

    const int arow0 = GR * g + lane % 32;
    int brow[2];
    if (GATED) {  // gate block and the matching up block
      brow[0] = 32 * wn + lane % 32;
      brow[1] = 128 + 32 * wn + lane % 32;
    } else {
      brow[0] = 64 * wn + lane % 32;
      brow[1] = 64 * wn + 32 + lane % 32;
    }
    // live 32-row blocks of this wave (wave-uniform)
    int vblk = (t.rows - GR * g + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > kMB ? kMB : vblk);
    vblk = __builtin_amdgcn_readfirstlane(vblk);
    static_assert(kMB == 4 || kMB == 5, "the K loop is specialised for 0..kMB live row blocks");
    switch (vblk) {  // every wave runs the same loads and barriers; only the MFMA count differs
      case 5:
        if constexpr (kMB >= 5) mainloop<TR, (kMB >= 5 ? 5 : 4)>(c, acc, arow0, brow);
        break;
      case 4: mainloop<TR, 4>(c, acc, arow0, brow); break;
      case 3: mainloop<TR, 3>(c, acc, arow0, brow); break;
      case 2: mainloop<TR, 2>(c, acc, arow0, brow); break;
      case 1: mainloop<TR, 1>(c, acc, arow0, brow); break;
      default: mainloop<TR, 0>(c, acc, arow0, brow); break;
    }

    // epilogue. C layout of the 32x32 MFMA: lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4 of its 32x32 block.
    const int col_in = lane % 32;
    if (GATED || routed) {
      // bf16 outputs go through LDS (the stages are free once the K loop is done): group
      // g writes its rows as a [rows][W] bf16 tile into stage g, then its 256 threads
      // store whole rows with 16-byte stores, in passes of as many row blocks as a stage
      // holds (one pass in both phases: 160 rows of 256 B, 128 rows of 512 B). Rows whose
      // bit 2 is set have their 64-byte halves swapped, so
      // the two half-waves' 2-byte writes (rows r and r+4) fall in different banks.
      constexpr int W = GATED ? BNB / 2 : BNB;  // output columns of the tile
      constexpr int pitch = 2 * W;               // bytes per row
      constexpr int kFit = kStageSz / (32 * pitch);
      constexpr int kPassMB = kMB < kFit ? kMB : kFit;  // row blocks per pass
      constexpr int kPasses = (kMB + kPassMB - 1) / kPassMB;
      static_assert(kPassMB * 32 * pitch <= kStageSz, "a pass fits in a stage");
      unsigned char* ep = g == 0 ? stage<0>() : stage<1>();
      auto eoff = [](int r, int byte) { return r * pitch + (byte ^ (((r >> 2) & 1) << 6)); };
      const int gt = tid % 256;
      constexpr int cpr = pitch / 16;  // 16-byte chunks per row
      const int rows_g = t.rows - GR * g;
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        const int mb0 = pass * kPassMB;
        if (pass > 0) __syncthreads();  // the previous pass's rows have been stored
#pragma unroll
        for (int mb = mb0; mb < mb0 + kPassMB && mb < kMB; ++mb) {
          if (mb >= vblk) continue;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = 32 * (mb - mb0) + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);  // row of the pass
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
        const int prow0 = 32 * mb0;  // the pass's first row within the group
        const int nrows = (kMB - mb0 < kPassMB ? kMB - mb0 : kPassMB) * 32;
        for (int idx = gt; idx < nrows * cpr; idx += 256) {
          const int r = idx / cpr, ch = idx % cpr;
          if (prow0 + r >= rows_g) break;
          const uint4 val = *reinterpret_cast<const uint4*>(ep + eoff(r, 16 * ch));
          const int64_t m = t.m0 + GR * g + prow0 + r;
          uint16_t* dst = routed ? static_cast<uint16_t*>(args.out_routed) + (row_base + m) * args.ldo_routed
                                 : static_cast<uint16_t*>(args.out_shared) + m * args.ldo_shared +
                                       static_cast<int64_t>(sg) * args.N;
          st16(dst + t.n0 + 8 * ch, val);
        }
      }
    } else {
      // fp32 shared-expert sum: direct stores
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        if (mb >= vblk) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int i = GR * g + 32 * mb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
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

size_t ffn_bf16_lds_bytes() { return kStages * kStageSz; }

hipError_t launch_grouped_gemm_bf16(const GemmArgs& args, bool gated, int grid, hipStream_t stream) {
  if (args.K % (kStages * BK) != 0) return hipErrorInvalidValue;
  if (gated)
    hipLaunchKernelGGL(grouped_gemm_bf16<true>, dim3(grid), dim3(kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(grouped_gemm_bf16<false>, dim3(grid), dim3(kThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace moe

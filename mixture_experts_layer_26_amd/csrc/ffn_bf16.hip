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
// tile list in gangs (gemm_common.h). A tile is up to TRW rows x 256 weight rows (phase 1:
// 128 gate + 128 up columns; phase 2: 256 output columns). Two tile shapes:
// - large batches: 320-row tiles, two LDS stages. At V3 prefill the routed experts hold
//   about 185..345 rows, so most experts are one row block and their weights pass through
//   the L1 once, where 256-row tiles split about 120 of the 256 experts in two.
// - batches of at most 128 tokens (decode): 128-row tiles, so every group is one row
//   block, and three LDS stages. These launches stream the weights once and do little MFMA
//   work; the third stage keeps two K-steps of weights in flight per CU across each
//   barrier instead of one.
// K advances in steps of 64 (128-byte rows) through a ring of LDS stages filled by direct
// global-to-LDS loads (global_load_lds_dwordx4): no staging registers and no LDS store
// instructions. One barrier per step, before its last 16-wide sub-step, so each wave reads
// the next step's first fragments while the MFMAs of the current one run. Every wave
// computes a TRW/2 x 64 block with v_mfma_f32_32x32x16_bf16: wave (g, wn) owns rows
// g*TRW/2.. of the tile; in phase 1 gate rows 32wn.. with the matching up rows (so
// SiLU(gate) * up is formed in registers), in phase 2 output columns 64wn... The load
// addresses keep their wave-uniform part in SGPRs (one VGPR per loaded row), which leaves
// the K loops free of register spills at 320 rows in both phases. The K loop is
// specialised on the number of 32-row blocks of a wave that hold rows, so row blocks past
// an expert's count cost no MFMA work. Weights are read row-major or in the tiled layout
// of pack.hip. Phase 2 writes its outputs (y_routed, the fp32 shared sum) with the
// non-temporal policy: the combine reads them once, from HBM at prefill sizes, and
// streaming them past the L2 measured faster in both (V3 prefill bf16: down-projection
// 0.5-0.8%, combine 5-8%; decode down-projection 1.4%). H keeps the default policy (no
// change measured), and so do the FP8 kernel's outputs (the policy made its
// down-projection 8% slower).
#include "gemm_common.h"
#include "launch.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int BK = 64;                  // bf16 per K-step: 128-byte rows (whole cache lines)
constexpr int kRow = 128;               // bytes per tile row per stage
constexpr int kOpB = BNB * kRow;        // 32 KB: the B rows of one stage
constexpr int kSubs = BK / 16;          // MFMA sub-steps per K-step
constexpr int kDmaB = BNB / 64;         // B loads (global_load_lds of 8 rows) per wave per step

// Tile geometry for TRW tile rows and S stages: two wave groups of TRW / 2 rows, each wave
// a TRW / 2 x 64 block of 32 x 32 MFMA tiles.
template <int TRW, int S>
struct Geo {
  static constexpr int GR = TRW / 2;      // rows per wave group
  static constexpr int kMB = GR / 32;     // 32-row blocks per wave
  static constexpr int kOpA = TRW * kRow; // the A rows of one stage
  static constexpr int kDmaA = TRW / 64;  // A loads per wave per step
  static constexpr int kStage = kOpA + kOpB;
  static constexpr int kS = S;
};
using GeoLarge = Geo<320, 2>;  // 2 x 72 KB
using GeoSmall = Geo<128, 3>;  // 3 x 48 KB; every group of a batch of <= 128 tokens is one block
static_assert(GeoSmall::GR * 2 == kSmallBatchRows, "the small tiles hold a whole small batch");

// The ring of S stages of one geometry (one LDS array per geometry: a kernel allocates
// only the ring it uses).
template <class G>
__device__ __forceinline__ unsigned char* ring() {
  __shared__ __attribute__((aligned(16))) unsigned char r[G::kS * G::kStage];
  return r;
}

template <class G, int ST>
__device__ __forceinline__ unsigned char* stage() {
  return ring<G>() + ST * G::kStage;
}

typedef __attribute__((address_space(3))) unsigned char* lds_ptr;

// One global_load_lds_dwordx4 in its SGPR-base form: lane i copies the 16 bytes at
// sbase + voff (sbase wave-uniform in SGPRs, voff the lane's 32-bit byte offset) to LDS
// byte lds + 16 i. M0 holds the LDS address (one wait state after writing it). The
// instruction is written out rather than taken from the builtin so that the compiler,
// which cannot follow which stage a load lands in across loop iterations, adds no wait
// of its own before the LDS reads; the waits are the explicit ones in step_barrier.
// Keeping the wave-uniform part of every address in SGPRs leaves one VGPR per loaded row
// (a 64-bit per-lane address would take two, plus the temporaries of its add), and a
// K-step moves the base with scalar adds. M0 is declared clobbered, so the compiler keeps
// no value of its own in M0 across the statement (clang warns that M0 is a reserved
// register; the clobber is what tells its M0-initialisation passes that the statement
// writes it).
// The A rows are re-read by many workgroups through the L2 and take the default cache
// policy (the non-temporal policy on them took V3 prefill to 8.5 ms).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t voff, const unsigned char* sbase, const unsigned char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// The same for a weight row, whose cache policy depends on the tile's group: non-temporal
// (stream != 0) for groups of one row block, whose weight bytes one workgroup reads once;
// streaming them with that policy measured faster in every phase (V3 decode 3.86 -> 3.67
// ms, V3 prefill 7.08 -> 6.86 ms). Weights that several row blocks read (the shared
// experts', a large expert's) keep the default policy, so that the blocks after the first
// find them in the L2 (with the policy on them too, the shared expert's gate/up weights
// came from HBM once per row block). The choice is a scalar branch inside the statement,
// between two copies of the load, so the compiler sees one instruction and its register
// allocation of the K loop is the same as with a fixed policy (two copies of the K loop
// spilled). SCC is clobbered by the compare.
__device__ __forceinline__ void dma16_w(uint32_t voff, const unsigned char* sbase, const unsigned char* lds,
                                        uint32_t stream) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  const uint32_t st = __builtin_amdgcn_readfirstlane(stream);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_cmp_eq_u32 %3, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "global_load_lds_dwordx4 %0, %1 nt\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "global_load_lds_dwordx4 %0, %1\n"
      "2:" ::"v"(voff),
      "s"(sbase), "s"(m0), "s"(st)
      : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// A wave-uniform pointer made explicit (both halves read from the first lane), so that it
// can sit in SGPRs as the base of dma16.
__device__ __forceinline__ const unsigned char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<const unsigned char*>((hi << 32) | lo);
}

template <class G>
struct TileCtx {
  bool load_a;                  // this wave's A rows hold at least one of the tile's rows
  uint32_t b_stream;            // 1: the group has one row block, its weights are read once
  const unsigned char* abase;   // wave-uniform: K-step 0 of the A rows
  uint32_t a[G::kDmaA];         // this lane's A rows: byte offsets from abase (chunk included)
  const unsigned char* bbase;   // wave-uniform: K-step 0 of this wave's B rows
  uint32_t b[kDmaB];            // this lane's four B rows: byte offsets from bbase (chunk included)
  int64_t seg_stride;    // phase 2 shared: W2 stride per K segment (elements), else 0
  int bstep;             // elements from one K-step of a B row to the next
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;                // K-steps
};

// Direct loads of K-step kt into stage ST: wave w fills A rows 8 kDmaA w.. (kDmaA 8-row
// instructions: 40 rows with 320-row tiles, 16 with 128-row tiles) and B rows 32w..32w+31
// (four); lane i writes row 8j + i/8 of its instruction's block, 16-byte slot i%8, whose
// global chunk was chosen when the offsets were made. A wave whose A rows all lie past the
// tile's rows loads no A (those LDS rows feed only outputs that are not stored).
template <int ST, class G>
__device__ __forceinline__ void dma_step(const TileCtx<G>& c, int kt, int wave) {
  constexpr int kDmaA = G::kDmaA, kOpA = G::kOpA;
  unsigned char* st = stage<G, ST>();
  const unsigned char* ak = c.abase + static_cast<int64_t>(kt) * (BK * 2);
  const unsigned char* bk = c.bbase + 2 * b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, c.bstep);
  if (c.load_a) {
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) dma16(c.a[j], ak, st + (8 * kDmaA * wave + 8 * j) * kRow);
  }
#pragma unroll
  for (int j = 0; j < kDmaB; ++j) dma16_w(c.b[j], bk, st + kOpA + (8 * kDmaB * wave + 8 * j) * kRow, c.b_stream);
}

// Fragments of one 16-wide sub-step of stage ST for a wave holding NMB live 32-row
// blocks: NMB A fragments (rows arow0 + 32 mb) and two B fragments (rows brow).
template <int NMB>
struct Frags {
  bf16x8 a[NMB > 0 ? NMB : 1];
  bf16x8 b[2];
};

template <int ST, class G, int NMB>
__device__ __forceinline__ void read_frags(Frags<NMB>& f, int sub, int arow0, const int (&brow)[2], int lane) {
  const unsigned char* la = stage<G, ST>();
  const unsigned char* lb = la + G::kOpA;
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

// Wait until at most N of this wave's loads are in flight. Loads complete in order, so
// with N = the loads issued after those of a step, that step has landed; any extra memory
// operation only makes the wait stricter.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this wave's LDS reads have returned and its loads of the next step have
// landed, with `steps` later K-steps of its loads left in flight (0 .. S - 1; a wave issues
// kDmaB loads per step, plus kDmaA when it loads A), then the workgroup barrier: after it
// every wave's part of the next step is in LDS and no wave reads the current step's stage
// any more. The branches choose only the count of the load wait (their conditions are
// wave-uniform); the barrier itself is issued once, unconditionally.
template <class G>
__device__ __forceinline__ void step_barrier(int steps, bool load_a) {
  constexpr int LB = kDmaB, LAB = G::kDmaA + kDmaB;
  static_assert(G::kS <= 3, "wait counts written out for up to two later steps");
  if (steps <= 0)
    wait_vm<0>();
  else if (steps == 1)
    load_a ? wait_vm<LAB>() : wait_vm<LB>();
  else
    load_a ? wait_vm<2 * LAB>() : wait_vm<2 * LB>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One K-step s from stage ST = s % S, four 16-wide sub-steps. Fragment sets f0 and f1
// alternate: each sub-step's MFMAs run while the sub-step after next is read. On entry
// sub-steps 0 and 1 have been requested, steps up to s + S - 1 have been loaded or are in
// flight, and `newer` of them lie beyond s + 1. The barrier sits before the last sub-step:
// the wave has then issued every read of stage ST, and step s + 1 has landed; after it
// stage ST takes the load of step s + S (when dma) and the next step's first two
// sub-steps are read (when read) while the last sub-step runs.
template <int ST, class G, int NMB>
__device__ __forceinline__ void k_step(const TileCtx<G>& c, int s, int wave, int arow0, const int (&brow)[2],
                                       int lane, Frags<NMB>& f0, Frags<NMB>& f1, f32x16 (&acc)[G::kMB][2],
                                       bool dma, bool read, int newer) {
  constexpr int NMF = 2 * NMB, S = G::kS, NX = (ST + 1) % S;
  static_assert(kSubs == 4, "a K-step is four 16-wide sub-steps, read in alternating fragment sets");
  mfma_sub(f0, acc);
  fence();
  read_frags<ST, G, NMB>(f0, 2, arow0, brow, lane);
  fence();
  mfma_sub(f1, acc);
  fence();
  read_frags<ST, G, NMB>(f1, 3, arow0, brow, lane);
  fence();
  mfma_sub(f0, acc);
  fence();
  step_barrier<G>(newer, c.load_a);
  fence();
  if constexpr (NMF > 0) mfma_one(f1, acc, 0);
  fence();
  if (dma) dma_step<ST, G>(c, s + S, wave);
  fence();
  if constexpr (NMF > 1) mfma_one(f1, acc, 1);
  fence();
  if (read) read_frags<NX, G, NMB>(f0, 0, arow0, brow, lane);
  fence();
#pragma unroll
  for (int i = 2; i < NMF; ++i) mfma_one(f1, acc, i);
  fence();
  if (read) read_frags<NX, G, NMB>(f1, 1, arow0, brow, lane);
  fence();
}

// Steps base + I, base + I + 1, ... below base + R (base a multiple of S, R <= 2S - 1): the
// tail of the K loop, whose loads and waits depend on how many steps remain.
template <int I, class G, int NMB>
__device__ __forceinline__ void tail_steps(const TileCtx<G>& c, int base, int R, int wave, int arow0,
                                           const int (&brow)[2], int lane, Frags<NMB>& f0, Frags<NMB>& f1,
                                           f32x16 (&acc)[G::kMB][2]) {
  constexpr int S = G::kS;
  if constexpr (I < 2 * S - 1) {
    if (I < R) {
      const int left = R - I;  // steps from this one to the end
      const int newer = left - 2 < S - 2 ? left - 2 : S - 2;
      k_step<I % S, G, NMB>(c, base + I, wave, arow0, brow, lane, f0, f1, acc, left > S, left > 1, newer);
      tail_steps<I + 1, G, NMB>(c, base, R, wave, arow0, brow, lane, f0, f1, acc);
    }
  }
}

template <int J, class G>
__device__ __forceinline__ void prologue_dma(const TileCtx<G>& c, int wave) {
  if constexpr (J < G::kS) {
    if (J < c.nk) {
      dma_step<J, G>(c, J, wave);
      prologue_dma<J + 1, G>(c, wave);
    }
  }
}

template <int I, class G, int NMB>
__device__ __forceinline__ void body_steps(const TileCtx<G>& c, int s, int wave, int arow0, const int (&brow)[2],
                                           int lane, Frags<NMB>& f0, Frags<NMB>& f1, f32x16 (&acc)[G::kMB][2]) {
  if constexpr (I < G::kS) {
    k_step<I, G, NMB>(c, s + I, wave, arow0, brow, lane, f0, f1, acc, true, true, G::kS - 2);
    body_steps<I + 1, G, NMB>(c, s, wave, arow0, brow, lane, f0, f1, acc);
  }
}

// The K loop of one tile: steps 0 .. S-1 are loaded up front, and step s loads step s + S
// into the stage it has just finished. The loop runs S steps at a time while every one of
// them loads; the last S .. 2S - 1 steps (or all, for a short K) go through tail_steps. On
// exit no load is in flight and every wave is past the last read of the stages.
template <class G, int NMB>
__device__ __forceinline__ void mainloop(const TileCtx<G>& c, f32x16 (&acc)[G::kMB][2], int arow0,
                                         const int (&brow)[2]) {
  constexpr int S = G::kS;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  prologue_dma<0, G>(c, wave);
  // step 0 landed; steps 1 .. min(S, nk) - 1 in flight
  step_barrier<G>((c.nk < S ? c.nk : S) - 1, c.load_a);
  Frags<NMB> f0, f1;
  read_frags<0, G, NMB>(f0, 0, arow0, brow, lane);
  read_frags<0, G, NMB>(f1, 1, arow0, brow, lane);
  int s = 0;
  for (; s + 2 * S <= c.nk; s += S) body_steps<0, G, NMB>(c, s, wave, arow0, brow, lane, f0, f1, acc);
  tail_steps<0, G, NMB>(c, s, c.nk - s, wave, arow0, brow, lane, f0, f1, acc);
}

// PRE (phase 1 only): also store the pre-activations a and v in fp32 (the backward's
// recompute). A separate instance, so that the forward's keeps its register allocation.
template <bool GATED, class G, bool PRE>
__global__ __launch_bounds__(kThreads) void grouped_gemm_bf16(GemmArgs args) {
  __shared__ TileMap tm;
  constexpr int TR = 2 * G::GR;
  constexpr int GR = G::GR, kMB = G::kMB, kDmaA = G::kDmaA;

  const int n_r = args.n_r;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map<TR, GATED>(tm, args.offset, n_r, args.n_shared_groups, args.T, ntn);
  auto rows_of = [&](int grp) -> int64_t { return grp < n_r ? args.offset[grp + 1] - args.offset[grp] : args.T; };

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = wave / 4, wn = wave % 4;

  for_each_tile(tm.total, args.sched, args.slot_stride, [&](int L) {
    const Tile t = tile_at(tm, L, n_r, bn_out, ntn, rows_of);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;  // shared group index
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    TileCtx<G> c;
    // this lane's load rows: 8*kDmaA*wave + 8j + lane/8 of the tile's A rows and 32*wave + 8j +
    // lane/8 of its B rows, slot lane%8, holding global chunk slot ^ ((row/2)%8) (the
    // swizzle of swz). Offsets are in bytes from a wave-uniform base: the gathered rows of
    // phase 1 from u itself (moe_grouped_ffn refuses u of 2^31 elements or more, so they fit
    // 32 bits), every other A operand from the tile's first row, B from the tile's weights.
    const int64_t eoff = static_cast<int64_t>(routed ? t.group : sg) * args.b_expert_stride;
    c.load_a = __builtin_amdgcn_readfirstlane(8 * kDmaA * wave < t.rows ? 1 : 0) != 0;
    c.b_stream = __builtin_amdgcn_readfirstlane(tm.mt[t.group] == 1 ? 1 : 0);
    const bool gathered = routed && args.gather != nullptr;
    const int64_t lda = routed ? args.lda_routed : args.lda_shared;
    {
      const uint16_t* a0 = routed ? args.a_routed : args.a_shared;
      const int64_t first = gathered ? 0 : (routed ? row_base : 0) + t.m0;  // row of A at offset 0
      c.abase = uniform_ptr(a0 + first * lda);
    }
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) {
      const int r = 8 * kDmaA * wave + 8 * j + lane / 8;
      const int chunk = (lane % 8) ^ ((r >> 1) & 7);
      // rows past the tile's valid rows repeat its last one
      const int ra = r < t.rows ? r : t.rows - 1;
      const int64_t row = gathered ? args.gather[row_base + t.m0 + ra] : ra;
      c.a[j] = static_cast<uint32_t>(2 * (row * lda + chunk * 8));
    }
    {
      // B rows 32*wave..: in phase 1 waves 0..3 hold gate rows and 4..7 up rows, so the
      // matrix is wave-uniform
      const bool up = GATED && wave >= 4;
      const uint16_t* base = GATED ? (up ? (routed ? args.b3_routed : args.b3_shared)
                                         : (routed ? args.b1_routed : args.b1_shared)) + eoff
                                   : (routed ? args.b1_routed + eoff : args.b1_shared);
      constexpr int R = GATED ? 128 : 256;  // tiled layout: [E][N/R][K/64][R][64]
      c.bbase = uniform_ptr(args.b_tiled ? base + (t.n0 / R) * (args.ldb / BK) * (R * BK) : base + t.n0 * args.ldb);
#pragma unroll
      for (int j = 0; j < kDmaB; ++j) {
        const int r = 8 * kDmaB * wave + 8 * j + lane / 8;
        const int chunk = (lane % 8) ^ ((r >> 1) & 7);
        const int64_t nrow = GATED ? (r & 127) : r;  // weight row within the tile
        c.b[j] = static_cast<uint32_t>(2 * (args.b_tiled ? nrow * BK + chunk * 8 : nrow * args.ldb + chunk * 8));
      }
    }
    c.seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.bstep = args.b_tiled ? (GATED ? 128 : 256) * BK : BK;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = kseg_recip(c.kseg_steps);
    // wave-uniform (it sets the K loop's loads and waits)
    c.nk = __builtin_amdgcn_readfirstlane((routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK);

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
    static_assert(kMB >= 2 && kMB <= 5, "the K loop is specialised for 0..kMB live row blocks");
    switch (vblk) {  // every wave runs the same loads and barriers; only the MFMA count differs
      case 5:
        if constexpr (kMB >= 5) mainloop<G, (kMB >= 5 ? 5 : 1)>(c, acc, arow0, brow);
        break;
      case 4:
        if constexpr (kMB >= 4) mainloop<G, (kMB >= 4 ? 4 : 1)>(c, acc, arow0, brow);
        break;
      case 3:
        if constexpr (kMB >= 3) mainloop<G, (kMB >= 3 ? 3 : 1)>(c, acc, arow0, brow);
        break;
      case 2: mainloop<G, 2>(c, acc, arow0, brow); break;
      case 1: mainloop<G, 1>(c, acc, arow0, brow); break;
      default: mainloop<G, 0>(c, acc, arow0, brow); break;
    }

    // epilogue. C layout of the 32x32 MFMA: lane holds column lane%32 and rows
    // 8*(v/4) + 4*(lane/32) + v%4 of its 32x32 block.
    const int col_in = lane % 32;
    if (GATED || routed) {
      // bf16 outputs go through LDS (the stages are free once the K loop is done): group
      // g writes its rows as a [rows][W] bf16 tile into stage g, then its 256 threads
      // store whole rows with 16-byte stores, in passes of as many row blocks as a stage
      // holds (320-row tiles, phase 1: one pass of 160 rows of 256 B; phase 2: 128 + 32 rows
      // of 512 B; 128-row tiles: one pass). Rows whose bit 2 is set have their 64-byte halves
      // swapped, so the two half-waves' 2-byte writes (rows r and r+4) fall in different banks.
      constexpr int W = GATED ? BNB / 2 : BNB;  // output columns of the tile
      constexpr int pitch = 2 * W;               // bytes per row
      constexpr int kFit = G::kStage / (32 * pitch);
      constexpr int kPassMB = kMB < kFit ? kMB : kFit;  // row blocks per pass
      constexpr int kPasses = (kMB + kPassMB - 1) / kPassMB;
      static_assert(kPassMB * 32 * pitch <= G::kStage, "a pass fits in a stage");
      unsigned char* ep = g == 0 ? stage<G, 0>() : stage<G, 1>();
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
          if constexpr (GATED)
            st16(dst + t.n0 + 8 * ch, val);
          else  // y_routed: read back once, by the combine, from HBM
            __builtin_nontemporal_store(__builtin_bit_cast(i32x4, val), reinterpret_cast<i32x4*>(dst + t.n0 + 8 * ch));
        }
      }
      if constexpr (GATED && PRE) {
        // the pre-activations a and v in fp32, straight from the accumulators: lane column
        // 32 wn + col_in, 128 contiguous bytes per row
        float* pa = routed ? args.pre_gate_routed : args.pre_gate_shared;
        float* pv = routed ? args.pre_up_routed : args.pre_up_shared;
        {
          const int64_t ld = routed ? args.ldo_routed : args.ldo_shared;
          const int64_t col = t.n0 + 32 * wn + col_in + (routed ? 0 : static_cast<int64_t>(sg) * args.N);
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) {
            if (mb >= vblk) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int i = GR * g + 32 * mb + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
              if (i >= t.rows) continue;
              const int64_t o = ((routed ? row_base : 0) + t.m0 + i) * ld + col;
              pa[o] = acc[mb][0][v];
              pv[o] = acc[mb][1][v];
            }
          }
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
            __builtin_nontemporal_store(acc[mb][nb][v], static_cast<float*>(args.out_shared) + m * args.ldo_shared + n);
          }
        }
      }
    }
  });
}

}  // namespace

size_t ffn_bf16_lds_bytes() {
  const size_t a = GeoLarge::kS * GeoLarge::kStage, b = GeoSmall::kS * GeoSmall::kStage;
  return a > b ? a : b;
}

hipError_t launch_grouped_gemm_bf16(const GemmArgs& args, bool gated, int grid, hipStream_t stream) {
  if (args.K % (2 * BK) != 0) return hipErrorInvalidValue;
  const bool small = args.T <= kSmallBatchRows;  // every group fits one 128-row tile
  const bool pre = gated && args.pre_gate_routed != nullptr;
  if (pre && (!args.pre_up_routed || !args.pre_gate_shared || !args.pre_up_shared)) return hipErrorInvalidValue;
  const dim3 g(grid), b(kThreads);
  if (pre && small)
    hipLaunchKernelGGL((grouped_gemm_bf16<true, GeoSmall, true>), g, b, 0, stream, args);
  else if (pre)
    hipLaunchKernelGGL((grouped_gemm_bf16<true, GeoLarge, true>), g, b, 0, stream, args);
  else if (gated && small)
    hipLaunchKernelGGL((grouped_gemm_bf16<true, GeoSmall, false>), g, b, 0, stream, args);
  else if (gated)
    hipLaunchKernelGGL((grouped_gemm_bf16<true, GeoLarge, false>), g, b, 0, stream, args);
  else if (small)
    hipLaunchKernelGGL((grouped_gemm_bf16<false, GeoSmall, false>), g, b, 0, stream, args);
  else
    hipLaunchKernelGGL((grouped_gemm_bf16<false, GeoLarge, false>), g, b, 0, stream, args);
  return hipGetLastError();
}

}  // namespace moe

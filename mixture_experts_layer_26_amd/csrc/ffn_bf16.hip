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
// are 256 rows x 256 B-rows (phase 1: 128 gate + 128 up columns) with K-steps of 64;
// global loads run two K-steps ahead in registers, then go through XOR-swizzled LDS
// (double buffered) to v_mfma_f32_32x32x16_bf16; each wave owns a 128 x 128 block
// (16 MFMA tiles) and reads the next sub-step's fragments while the current MFMAs
// run. The tile list is split into 8
// contiguous chunks, one per XCD, so the tiles of one expert run side by side on one
// XCD and its weights and gathered rows are reused from that XCD's L2. The K loop is
// specialised on the number of 32-row blocks of a wave that hold rows, so row blocks
// past an expert's count cost no MFMA work.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

// Tuning knobs (compile-time): waves along N (2: 4 waves of 128x128; 4: 8 waves of
// 128x64), register stages of global prefetch (1 or 2), double-buffered MFMA
// fragments, and explicit interleaving of LDS reads with MFMAs.
#ifndef MOE_GEMM_WN
#define MOE_GEMM_WN 4
#endif
#ifndef MOE_GEMM_STAGES
#define MOE_GEMM_STAGES 1
#endif
#ifndef MOE_GEMM_FRAGDB
#define MOE_GEMM_FRAGDB 1
#endif
#ifndef MOE_GEMM_SCHED
#define MOE_GEMM_SCHED 1
#endif
#ifndef MOE_GEMM_PF
#define MOE_GEMM_PF 1
#endif
constexpr int WN = MOE_GEMM_WN;            // waves along N
constexpr int kThreads = 64 * 2 * WN;      // 2 waves along M
constexpr int NBW = 256 / WN / 32;         // 32-column MFMA blocks per wave
constexpr int CPT = 2048 / kThreads;       // 16-byte chunks per thread per operand per K-step
constexpr int RSTEP = kThreads / 8;        // row step between a thread's chunks
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
#ifndef MOE_GEMM_SWZ
#define MOE_GEMM_SWZ 1
#endif
__device__ __forceinline__ int swz(int r, int c) {
  return r * 128 + ((c ^ (MOE_GEMM_SWZ ? ((r >> 1) & 7) : (r & 7))) << 4);
}

// Per-workgroup state of one tile's main loop.
struct TileCtx {
  const uint16_t* arow[CPT];  // this thread's A rows (chunk cc)
  const uint16_t* b1;         // this thread's first B row (chunk cc); rows cr + RSTEP*i
  const uint16_t* b3;         // gated: the up-projection rows (B rows 128..255)
  const uint16_t* pf;         // row whose cache line this thread prefetches
  bool pf_is_b;               // pf is a weight (B) row, else an activation (A) row
  int64_t ldb;
  int64_t b_seg_stride;       // phase 2 shared: W2 stride per K segment, else 0
  int kseg_steps;             // K-steps per shared segment
  uint32_t kseg_inv;          // ceil(2^32 / kseg_steps)
  int nk;                     // K-steps
};

// Element offset of K-step kt in a B row. For the shared down-projection the K range
// runs over the shared experts' segments (seg = kt / kseg_steps selects the expert);
// elsewhere kseg_steps == nk, so seg is 0 and the offset is kt * BK.
// (The quotient uses a precomputed reciprocal: exact for kt, kseg_steps < 2^16.)
__device__ __forceinline__ int64_t b_offset(const TileCtx& c, int kt) {
  const int seg = static_cast<int>(__umulhi(static_cast<uint32_t>(kt), c.kseg_inv));
  return static_cast<int64_t>(seg) * c.b_seg_stride + static_cast<int64_t>(kt - seg * c.kseg_steps) * BK;
}

// One K-step's global->register stage.
struct Stage {
  uint4 a[CPT], b[CPT];
};

template <bool GATED>
__device__ __forceinline__ void gload(const TileCtx& c, int kt, Stage& st) {
  const int64_t aoff = static_cast<int64_t>(kt) * BK;
  const int64_t boff = b_offset(c, kt);
#pragma unroll
  for (int i = 0; i < CPT; ++i) st.a[i] = ld16(c.arow[i] + aoff);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int r = i * RSTEP;  // row offset of chunk i from the thread's first row
    const uint16_t* base = (GATED && r >= 128) ? c.b3 + (r - 128) * c.ldb : c.b1 + r * c.ldb;
    st.b[i] = ld16(base + boff);
  }
}

__device__ __forceinline__ void lstore(unsigned char* la, unsigned char* lb, const Stage& st, int cr, int cc) {
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int r = cr + RSTEP * i;
    *reinterpret_cast<uint4*>(la + swz(r, cc)) = st.a[i];
    *reinterpret_cast<uint4*>(lb + swz(r, cc)) = st.b[i];
  }
}

// MFMAs of one K-step on LDS stage (la, lb) for a wave holding NMB live 32-row blocks.
template <int NMB>
__device__ __forceinline__ void compute_step(const unsigned char* la, const unsigned char* lb, int arow0,
                                             const int (&brow)[NBW], int lane, f32x16 (&acc)[4][NBW]) {
  constexpr int NA = NMB > 0 ? NMB : 1;
  constexpr int NF = MOE_GEMM_FRAGDB ? 2 : 1;
  bf16x8 af[NF][NA], bfr[NF][NBW];
  auto rd = [&](int s, int buf) {
    const int ch = 2 * s + lane / 32;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
      af[buf][mb] = *reinterpret_cast<const bf16x8*>(la + swz(arow0 + 32 * mb, ch));
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) bfr[buf][nb] = *reinterpret_cast<const bf16x8*>(lb + swz(brow[nb], ch));
  };
  constexpr int NRD = NMB + NBW;     // fragment reads per sub-step
  constexpr int NMF = NMB * NBW;     // MFMAs per sub-step
  if (MOE_GEMM_FRAGDB) {
    rd(0, 0);
    if (MOE_GEMM_SCHED && NMB > 0) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int cur = MOE_GEMM_FRAGDB ? (s & 1) : 0;
    if (MOE_GEMM_FRAGDB) {
      if (s + 1 < 4) rd(s + 1, (s + 1) & 1);
    } else {
      rd(s, 0);
    }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][mb], bfr[cur][nb], acc[mb][nb], 0, 0, 0);
    if (MOE_GEMM_SCHED && NMB > 0) {
      if (MOE_GEMM_FRAGDB && s + 1 < 4 && NMF >= NRD) {
        // next sub-step's reads threaded between this sub-step's MFMAs
#pragma unroll
        for (int i = 0; i < NRD; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NMF > NRD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
      } else {
        if (!MOE_GEMM_FRAGDB || s + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
      }
    }
  }
}

// Main loop over K: LDS double buffer plus MOE_GEMM_STAGES register stages of global
// prefetch (loads for step kt + MOE_GEMM_STAGES are issued while step kt computes).
template <bool GATED, int NMB>
__device__ __forceinline__ void mainloop(const TileCtx& c, unsigned char* smem, f32x16 (&acc)[4][NBW]) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int cc = tid % 8, cr = tid / 8;
  unsigned char* la0 = smem;
  unsigned char* la1 = smem + BM * BK * 2;
  unsigned char* lb0 = smem + 2 * BM * BK * 2;
  unsigned char* lb1 = lb0 + BNB * BK * 2;
  const int arow0 = 128 * wm + lane % 32;
  int brow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (GATED) {
      const int j = nb % (NBW / 2);
      brow[nb] = (nb < NBW / 2 ? 0 : 128) + 32 * (NBW / 2) * wn + 32 * j + lane % 32;
    } else {
      brow[nb] = (256 / WN) * wn + 32 * nb + lane % 32;
    }
  }
#if MOE_GEMM_STAGES == 2
  Stage s0, s1;
  gload<GATED>(c, 0, s0);
  if (c.nk > 1) gload<GATED>(c, 1, s1);
  lstore(la0, lb0, s0, cr, cc);
  lds_barrier();
  if (c.nk > 2) gload<GATED>(c, 2, s0);
  for (int kt = 0; kt < c.nk; kt += 2) {
    compute_step<NMB>(la0, lb0, arow0, brow, lane, acc);
    if (kt + 1 < c.nk) lstore(la1, lb1, s1, cr, cc);
    lds_barrier();
    if (kt + 3 < c.nk) gload<GATED>(c, kt + 3, s1);
    if (kt + 1 >= c.nk) break;
    compute_step<NMB>(la1, lb1, arow0, brow, lane, acc);
    if (kt + 2 < c.nk) lstore(la0, lb0, s0, cr, cc);
    lds_barrier();
    if (kt + 4 < c.nk) gload<GATED>(c, kt + 4, s0);
  }
#else
  // One register stage, and an L2 prefetch kPfDist K-steps ahead: each thread touches
  // one 128-byte line per step (waves 0-3: the tile's 256 weight rows; waves 4-7: its
  // 256 activation rows). The word a prefetch returns is folded into `sink` one
  // iteration later, by when it has arrived, so no prefetch is waited on early.
  // Indices past the last K-step are clamped, so the loop body has no branches.
  constexpr int kPfDist = 4;
  const int last = c.nk - 1;
  uint32_t sink = 0;
  auto touch = [&](int kt) -> uint32_t {
    kt = kt < last ? kt : last;
    const int64_t off = c.pf_is_b ? b_offset(c, kt) : static_cast<int64_t>(kt) * BK;
    return MOE_GEMM_PF ? *reinterpret_cast<const uint32_t*>(c.pf + off) : 0u;
  };
  Stage st;
  gload<GATED>(c, 0, st);
  lstore(la0, lb0, st, cr, cc);
  uint32_t pf = touch(kPfDist - 1);
  lds_barrier();
  for (int kt = 0; kt < c.nk; ++kt) {
    const bool odd = kt & 1;
    gload<GATED>(c, kt < last ? kt + 1 : last, st);
    sink ^= pf;
    pf = touch(kt + kPfDist);
    compute_step<NMB>(odd ? la1 : la0, odd ? lb1 : lb0, arow0, brow, lane, acc);
    lstore(odd ? la0 : la1, odd ? lb0 : lb1, st, cr, cc);  // after the last step: unused
    lds_barrier();
  }
  sink ^= pf;
  // never true for real data (keeps the prefetch loads alive)
  if (sink == 0x7FC00001u && c.nk < 0) acc[0][0][0] += 1.0f;
#endif
}

#ifndef MOE_GEMM_PINGPONG
#define MOE_GEMM_PINGPONG 1
#endif

// Ping-pong main loop (8 waves). Group g (waves 4g..4g+3, one wave on each SIMD)
// owns tile rows 128g..128g+127 and B rows 128g..128g+127 (for the gated phase: the
// gate rows for g = 0, the up rows for g = 1). The two groups alternate half-steps:
// while one group runs the MFMAs of K-step k, the other writes its halves of step
// k+1 into the other LDS stage, so each SIMD's MFMA pipe is fed by one wave while its
// partner waits on memory. Global loads for a group's next step are issued at the
// start of its compute half. Indices past the end are clamped (harmless reloads).
template <bool GATED, int NMB>
__device__ __forceinline__ void mainloop_pp(const TileCtx& c, unsigned char* smem, f32x16 (&acc)[4][NBW]) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int g = __builtin_amdgcn_readfirstlane(wave / 4), wn = wave % 4;
  const int gt = tid % 256, cc = gt % 8, cr = gt / 8;
  const int last = c.nk - 1;
  auto la = [&](int st) { return smem + st * (BM * BK * 2); };
  auto lb = [&](int st) { return smem + 2 * BM * BK * 2 + st * (BNB * BK * 2); };
  const int arow0 = 128 * g + lane % 32;
  int brow[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    if (GATED) {
      const int j = nb % (NBW / 2);
      brow[nb] = (nb < NBW / 2 ? 0 : 128) + 32 * (NBW / 2) * wn + 32 * j + lane % 32;
    } else {
      brow[nb] = 64 * wn + 32 * nb + lane % 32;
    }
  }
  uint4 ra[4], rb[4];
  auto gload = [&](int kt) {
    kt = kt < last ? kt : last;
    const int64_t aoff = static_cast<int64_t>(kt) * BK;
    const int64_t boff = b_offset(c, kt);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ld16(c.arow[i] + aoff);
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[i] = ld16(c.b1 + static_cast<int64_t>(32 * i) * c.ldb + boff);
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
  lds_barrier();
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
  const int ngs = args.n_shared_groups;
  const int ng = n_r + ngs;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map(tm, args.offset, n_r, ngs, args.T, ntn);
  const int total = tm.total;

  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int cc = tid % 8, cr = tid / 8;

  // Tile claiming: the tile list is cut into 8 contiguous chunks, one per XCD. A
  // workgroup claims tiles of its own XCD's chunk from that chunk's counter, so the
  // tiles in flight on an XCD are always neighbours in the list (the same expert's
  // column tiles and row tiles), whose gathered rows and weights its L2 then serves to
  // several CUs. When the chunk runs out it helps the other XCDs' chunks. The
  // counters only decide which CU computes a tile, never what a tile computes.
  __shared__ int claim;
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  xcc &= 7;
  const int chunk = (total + 7) / 8;
  int o = 0;
  while (o < 8) {
    const int x = (static_cast<int>(xcc) + o) & 7;
    if (tid == 0) claim = atomicAdd(args.tile_counter + x, 1);
    __syncthreads();
    const int local = claim;
    __syncthreads();
    const int L = x * chunk + local;
    if (local >= chunk || L >= total) {
      ++o;
      continue;
    }
    const Tile t = tile_at(tm, L, ng, ntn, args.offset, n_r, args.T, bn_out);
    const bool routed = t.group < n_r;
    const int sg = t.group - n_r;  // shared group index
    const int64_t row_base = routed ? args.offset[t.group] : 0;

    TileCtx c;
    // A rows (rows past the tile's valid rows repeat its last valid row)
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
#if MOE_GEMM_PINGPONG
      int r = 128 * (wave / 4) + (tid % 256) / 8 + 32 * i;  // this group's half of the rows
#else
      int r = cr + RSTEP * i;
#endif
      if (r >= t.rows) r = t.rows - 1;
      const int64_t m = t.m0 + r;
      if (routed) {
        const int64_t src = args.gather ? args.gather[row_base + m] : (row_base + m);
        c.arow[i] = args.a_routed + src * args.lda_routed + cc * 8;
      } else {
        c.arow[i] = args.a_shared + m * args.lda_shared + cc * 8;
      }
    }
    const int64_t eoff = static_cast<int64_t>(routed ? t.group : sg) * args.b_expert_stride;
#if MOE_GEMM_PINGPONG
    {
      // this group's half of the B rows: gate (g = 0) / up (g = 1) rows when gated
      const int g = wave / 4, gr = (tid % 256) / 8;
      const uint16_t* base;
      int64_t nrow;
      if (GATED) {
        base = g == 0 ? (routed ? args.b1_routed : args.b1_shared) : (routed ? args.b3_routed : args.b3_shared);
        base += eoff;
        nrow = t.n0 + gr;
      } else {
        base = routed ? args.b1_routed + eoff : args.b1_shared;
        nrow = t.n0 + 128 * g + gr;
      }
      c.b1 = base + nrow * args.ldb + cc * 8;
      c.b3 = c.b1;
    }
#else
    if (GATED) {
      c.b1 = (routed ? args.b1_routed : args.b1_shared) + eoff + static_cast<int64_t>(t.n0 + cr) * args.ldb + cc * 8;
      c.b3 = (routed ? args.b3_routed : args.b3_shared) + eoff + static_cast<int64_t>(t.n0 + cr) * args.ldb + cc * 8;
    } else {
      c.b1 = (routed ? args.b1_routed + eoff : args.b1_shared) + static_cast<int64_t>(t.n0 + cr) * args.ldb + cc * 8;
      c.b3 = c.b1;
    }
#endif
    if (tid < BNB) {  // waves 0-3: one weight row of the tile each
      const int r = tid;
      const int64_t nrow = t.n0 + (GATED ? (r & 127) : r);
      const uint16_t* base = GATED ? (r >= 128 ? (routed ? args.b3_routed : args.b3_shared)
                                               : (routed ? args.b1_routed : args.b1_shared))
                                   : (routed ? args.b1_routed : args.b1_shared);
      c.pf = base + ((routed || GATED) ? eoff : 0) + nrow * args.ldb;
      c.pf_is_b = true;
    } else {  // waves 4-7: one activation row of the tile each
      int r = tid - BNB;
      if (r >= t.rows) r = t.rows - 1;
      const int64_t m = t.m0 + r;
      if (routed) {
        const int64_t src = args.gather ? args.gather[row_base + m] : (row_base + m);
        c.pf = args.a_routed + src * args.lda_routed;
      } else {
        c.pf = args.a_shared + m * args.lda_shared;
      }
      c.pf_is_b = false;
    }
    c.ldb = args.ldb;
    c.b_seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = static_cast<uint32_t>((0x100000000ull + c.kseg_steps - 1) / c.kseg_steps);
    c.nk = (routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK;

    f32x16 acc[4][NBW];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NBW; ++b) acc[a][b] = f32x16{};

    // live 32-row blocks of this wave (wave-uniform)
    int vblk = (t.rows - 128 * wm + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > 4 ? 4 : vblk);
    vblk = __builtin_amdgcn_readfirstlane(vblk);
    // every wave runs the same K loop (barriers); only the MFMA count differs
#if MOE_GEMM_PINGPONG
    switch (vblk) {
      case 4: mainloop_pp<GATED, 4>(c, smem, acc); break;
      case 3: mainloop_pp<GATED, 3>(c, smem, acc); break;
      case 2: mainloop_pp<GATED, 2>(c, smem, acc); break;
      case 1: mainloop_pp<GATED, 1>(c, smem, acc); break;
      default: mainloop_pp<GATED, 0>(c, smem, acc); break;
    }
#else
    switch (vblk) {
      case 4: mainloop<GATED, 4>(c, smem, acc); break;
      case 3: mainloop<GATED, 3>(c, smem, acc); break;
      case 2: mainloop<GATED, 2>(c, smem, acc); break;
      case 1: mainloop<GATED, 1>(c, smem, acc); break;
      default: mainloop<GATED, 0>(c, smem, acc); break;
    }
#endif

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
          for (int nb = 0; nb < NBW / 2; ++nb) {
            const int n = t.n0 + 32 * (NBW / 2) * wn + 32 * nb + col_in;
            const float h = silu(acc[mb][nb][v]) * acc[mb][nb + NBW / 2][v];
            uint16_t* o = routed ? static_cast<uint16_t*>(args.out_routed) + (row_base + m) * args.ldo_routed + n
                                 : static_cast<uint16_t*>(args.out_shared) + m * args.ldo_shared +
                                       static_cast<int64_t>(sg) * args.N + n;
            *o = f32_to_bf16(h);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            const int n = t.n0 + (256 / WN) * wn + 32 * nb + col_in;
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

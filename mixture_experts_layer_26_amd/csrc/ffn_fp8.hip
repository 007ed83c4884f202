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
// The tile walk, tile claiming and LDS layout are those of the bf16 kernel, with tiles of
// up to 320 rows x 256 weight rows in both phases (at V3 prefill most experts, 185..345
// rows, are then one row block and their weights pass through the L1 once) and 128-byte
// rows per K-step, so one K-step is exactly one 128-wide scale block. There are two
// stages: step s+1 is loaded while step s is computed. The MFMA is
// v_mfma_scale_f32_16x16x128_f8f6f4 with unit (E8M0 = 127) scales: one instruction
// covers one scale block of a 16 x 16 output block, starting from zero, and its result
// is folded into the accumulator with one fp32 FMA per element:
// acc += blk * (s_a[row] * s_w). The fp32 scales are arbitrary (not powers of two), so
// they cannot ride in the MFMA's E8M0 scale operands. The A-row scales arrive in LDS
// with the tiles (K-block-major in memory, so a step's scales of a tile are contiguous);
// the weight scales are read by scalar loads.
#include "gemm_common.h"
#include "launch.h"

namespace moe {

namespace {

using namespace gemm;

constexpr int BK = 128;                 // fp8 elements (bytes) per K-step = one scale block
constexpr int TR = 320;                 // tile rows (A rows per tile)
constexpr int GR = TR / 2;              // rows per wave group
constexpr int kRB = GR / 16;            // 16-row MFMA blocks per wave
constexpr int kNM = GR / 32;            // 32-row blocks per wave
constexpr int kDmaA = TR / 64;          // A loads (8 rows each) per wave per step
constexpr int kOpA = TR * BK;           // 40 KB: the A rows of one stage
constexpr int kOpB = BNB * BK;          // 32 KB: the B rows of one stage
// A-row scales of one stage: slot GS g + 12 c + mb holds the scale of row GR g + 16 mb + c
// (c = 0..15, mb = 0..kRB-1; slots 10 and 11 of each 12 are padding), so that a lane's
// scales of its row blocks are contiguous and 16-byte aligned, and the 16 lanes that read
// one 16-byte piece each (at a 48-byte stride) fall in 16 different 4-bank groups.
constexpr int kScalePitch = 12;
constexpr int GS = 16 * kScalePitch;    // scale slots per wave group
constexpr int kScaleSlots = 2 * GS;     // 384: six 64-lane loads
constexpr int kScaleBytes = kScaleSlots * 4;
constexpr int kStageSize = kOpA + kOpB + kScaleBytes;
static_assert(kRB <= kScalePitch, "a lane's row scales fit its slot run");
static_assert(kStageSize % 16 == 0, "16-byte aligned stages");

// The two stages (A rows, B rows, A-row scales), one LDS array so that every load
// destination is a wave base plus a constant.
__shared__ __attribute__((aligned(16))) unsigned char stages[2 * kStageSize];

template <int ST>
__device__ __forceinline__ unsigned char* stage() {
  return stages + ST * kStageSize;
}

typedef __attribute__((address_space(3))) unsigned char* lds_ptr;

// Weight scales are wave-uniform and read-only in these kernels, so they are read
// through the constant address space with a wave-uniform address: the loads become
// scalar loads, whose waits count on lgkmcnt. A vector load here would be waited for
// with a vmcnt that the compiler sizes without the DMA loads it cannot see, so the
// wait would also cover the next step's tile loads and stall the step's MFMAs on them.
typedef const __attribute__((address_space(4))) float* scale_ptr;

__device__ __forceinline__ scale_ptr uniform_scales(const float* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return (scale_ptr)((hi << 32) | lo);
}

// One global_load_lds_dwordx4 in its SGPR-base form: lane i copies the 16 bytes at
// sbase + voff (sbase wave-uniform in SGPRs, voff the lane's 32-bit byte offset) to LDS
// byte lbase + OFF + 16 i. M0 holds the LDS address (one wait state after writing it).
// The instruction is written out rather than taken from the builtin so that the compiler
// adds no wait of its own before the LDS reads; the waits are the explicit ones in
// step_barrier. Keeping the wave-uniform part of every address in SGPRs leaves one VGPR
// per loaded row, and a K-step moves the bases with scalar adds. The statement writes M0
// and SCC (the add), and declares both clobbered, so the compiler keeps no value of its
// own in either across it (clang warns that M0 is a reserved register; the clobber is
// what tells its M0-initialisation passes that the statement writes it). NT sets the
// non-temporal cache policy, used for the weight codes: each is read by one workgroup or
// the few of a gang close together in time, and streaming them with that policy measured
// faster (V3 prefill 4.45 -> 4.33 ms); A rows, re-read by many workgroups through the L2,
// keep the default policy (with it set on them, 4.76 ms).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int OFF, bool NT>
__device__ __forceinline__ void dma16(uint32_t voff, const unsigned char* sbase, uint32_t lbase) {
  if constexpr (NT)
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
                 "s"(lbase), "n"(OFF)
                 : "memory", "m0", "scc");
  else
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lbase), "n"(OFF)
                 : "memory", "m0", "scc");
}

// The same with 4 bytes per lane (lane i writes LDS byte lbase + OFF + 4 i).
template <int OFF>
__device__ __forceinline__ void dma4(uint32_t voff, const unsigned char* sbase, uint32_t lbase) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lbase), "n"(OFF)
               : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

// A wave-uniform pointer made explicit (both halves read from the first lane), so that it
// can sit in SGPRs as the base of dma16 and dma4.
__device__ __forceinline__ const unsigned char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<const unsigned char*>((hi << 32) | lo);
}

struct TileCtx {
  uint32_t lds_a;             // LDS address of this wave's A rows (8 kDmaA wave..) in stage 0
  uint32_t lds_b;             // LDS address of this wave's B rows (32 wave..) in stage 0
  uint32_t lds_scale;         // waves 0..5: LDS address of scale slots 64 wave.. in stage 0
  bool load_a;                // this wave's A rows hold at least one of the tile's rows
  bool load_scale;            // waves 0..5 load the A-row scales (one slot per lane)
  const unsigned char* abase; // wave-uniform: K-step 0 of the A rows
  uint32_t a[kDmaA];          // this lane's A rows: byte offsets from abase (chunk included)
  const unsigned char* bbase; // wave-uniform: K-step 0 of this wave's B rows
  uint32_t b[4];              // this lane's four B rows: byte offsets from bbase (chunk included)
  const unsigned char* sbase; // wave-uniform: K block 0 of the A-row scales
  uint32_t s;                 // threads 0..255: byte offset of the scale of the row LDS slot tid holds
  int64_t sa_step;            // bytes from one K block of the row scales to the next
  scale_ptr sb[2];            // this wave's two B-scale rows (gate/up, or the wave's block)
  int64_t seg_stride;         // phase 2 shared: W2 stride per K segment, else 0
  int bstep;                  // bytes from one K-step of a B row to the next
  int64_t sb_seg_stride;      // same for the W2 scales
  int kseg_steps;
  uint32_t kseg_inv;
  int nk;
};

// Direct loads of K-step kt into stage ST: wave w fills A rows 8 kDmaA w.. (kDmaA 8-row
// instructions) and B rows 32w..32w+31 (four); lane i writes row 8j + i/8 of its
// instruction's block, 16-byte slot i%8, whose global chunk was chosen when the offsets
// were made. A wave whose A rows all lie past the tile's rows loads no A.
template <int ST, int J = 0>
__device__ __forceinline__ void dma_a(const TileCtx& c, const unsigned char* ak) {
  if constexpr (J < kDmaA) {
    dma16<ST * kStageSize + J * 8 * BK, false>(c.a[J], ak, c.lds_a);
    dma_a<ST, J + 1>(c, ak);
  }
}

template <int ST>
__device__ __forceinline__ void dma_step(const TileCtx& c, int kt) {
  if (kt >= c.nk) return;  // past the last step (a K loop of one step)
  const unsigned char* ak = c.abase + static_cast<int64_t>(kt) * BK;
  const unsigned char* bk = c.bbase + b_offset(kt, c.kseg_steps, c.kseg_inv, c.seg_stride, c.bstep);
  if (c.load_a) dma_a<ST>(c, ak);
  dma16<ST * kStageSize + 0 * 8 * BK, true>(c.b[0], bk, c.lds_b);  // lds_b includes the A region
  dma16<ST * kStageSize + 1 * 8 * BK, true>(c.b[1], bk, c.lds_b);
  dma16<ST * kStageSize + 2 * 8 * BK, true>(c.b[2], bk, c.lds_b);
  dma16<ST * kStageSize + 3 * 8 * BK, true>(c.b[3], bk, c.lds_b);
  if (c.load_scale) dma4<ST * kStageSize>(c.s, c.sbase + kt * c.sa_step, c.lds_scale);
}

// A 16 x 128 fp8 fragment (rows row.., this lane's 32 bytes of K) from a swizzled stage.
// Lane group q (lanes 16q..16q+15) takes the 16-byte chunks q and q + 4 of its row, i.e.
// K elements 16q.. and 64 + 16q.., for the weight and the activation fragments alike: the
// MFMA pairs the same K elements of both operands, so the 128-wide block's sum is the same
// set of products in another order. Chunks 2q and 2q + 1 (K elements 32q..32q+31) cost 4
// bank-conflict cycles per ds_read_b128 under the (row/2)%8 swizzle, chunks q and q + 4
// none (SQ_LDS_BANK_CONFLICT, measured with an in-bounds probe of both patterns).
__device__ __forceinline__ i32x8 rd_frag(const unsigned char* base, int row, int q) {
  const uint4 lo = *reinterpret_cast<const uint4*>(base + swz(row, q));
  const uint4 hi = *reinterpret_cast<const uint4*>(base + swz(row, q + 4));
  i32x8 f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// Scheduling fence: the compiler moves no instruction across it.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// One K-step (one scale block) from stage ST for a wave holding NM live 32-row blocks
// (2*NM 16-row MFMA blocks, 4 column blocks each: 8*NM MFMAs). sw[p]: the weight scale
// of column blocks 2p, 2p+1. The weight fragment is the MFMA's first operand, so a
// lane's result holds 4 consecutive output columns of one token row (16*mb + lane%16)
// and the fold needs one row scale per lane and block: acc += blk * (s_a[row] * s_w).
// Each MFMA covers one scale block from zero. MFMAs and folds are software-pipelined:
// MFMA j is issued before the fold of MFMA j-1, so the fold's VALU work runs while the
// matrix core computes, and an empty asm statement ties MFMA j's A operand to the fold
// of MFMA j-2, so at most two MFMA results are held at once and the compiler cannot
// hoist the step's MFMAs ahead of their folds. The activation fragment of block mb+1 is
// read from LDS while block mb is computed.
template <int ST, int NM>
__device__ __forceinline__ void compute_step(int arow0, const int (&brow)[4], int lsa_off, const float (&sw)[2],
                                             int lane, f32x4 (&acc)[kRB][4]) {
  if constexpr (NM == 0) return;
  constexpr int NMF = 8 * NM;
  const unsigned char* la = stage<ST>();
  const unsigned char* lb = la + kOpA;
  const int q = lane / 16;
  // this lane's row scales of blocks 0..2NM-1, contiguous in LDS (see the DMA's slot order)
  const float* lsa = reinterpret_cast<const float*>(lb + kOpB) + lsa_off;
  float sa[NM > 0 ? 4 * ((2 * NM + 3) / 4) : 4];
#pragma unroll
  for (int p = 0; p < (2 * NM + 3) / 4; ++p) {
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(lsa + 4 * p);
#pragma unroll
    for (int v = 0; v < 4; ++v) sa[4 * p + v] = s4[v];
  }
  // weight fragments of column blocks 0, 1 first; those of blocks 2, 3 are read while
  // the first MFMA runs, which shortens the LDS burst at the start of the step
  i32x8 bfr[4];
  bfr[0] = rd_frag(lb, brow[0], q);
  bfr[1] = rd_frag(lb, brow[1], q);
  i32x8 af = rd_frag(la, arow0, q);
  i32x8 af_next;
  float prod[2][2];  // [block parity][column pair]: row scale x weight scale
  prod[0][0] = sa[0] * sw[0];
  prod[0][1] = sa[0] * sw[1];
  f32x4 blk[2];
  // Issue order, pinned by fences: MFMA j, then the fold of MFMA j-1 (its result is
  // ready by the time MFMA j has been accepted), so the fold's VALU work overlaps MFMA j.
#pragma unroll
  for (int j = 0; j <= NMF; ++j) {
    const int mb = j / 4, nb = j % 4;
    if (j < NMF) {
      if (nb == 0 && mb > 0) af = af_next;
      if (j >= 2) {  // ties the activation fragment (in place, no copy) to the fold of MFMA j-2
        const int mp = (j - 2) / 4, np = (j - 2) % 4;
        asm volatile("" : "+v"(af) : "v"(acc[mp][np]));
      }
      blk[j & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[nb], af, f32x4{}, 0, 0, 0, 127, 0, 127);
      fence();
      if (j == 0) {
        bfr[2] = rd_frag(lb, brow[2], q);
        bfr[3] = rd_frag(lb, brow[3], q);
      }
      if (nb == 0 && mb + 1 < 2 * NM) af_next = rd_frag(la, arow0 + 16 * (mb + 1), q);
      if (nb == 3 && mb + 1 < 2 * NM) {
        prod[(mb + 1) & 1][0] = sa[mb + 1] * sw[0];
        prod[(mb + 1) & 1][1] = sa[mb + 1] * sw[1];
      }
    }
    if (j >= 1) {  // fold MFMA j-1
      const int mp = (j - 1) / 4, np = (j - 1) % 4;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        acc[mp][np][v] = fmaf(blk[(j - 1) & 1][v], prod[mp & 1][np / 2], acc[mp][np][v]);
    }
    fence();
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
  if (kt >= c.nk) kt = c.nk - 1;  // past the last step: any valid scale (not used)
  const int64_t o = b_offset(kt, c.kseg_steps, c.kseg_inv, c.sb_seg_stride, 1);
  sw[0] = c.sb[0][o];
  sw[1] = c.sb[1][o];
}

// One K-step s from stage ST = s % 2. When MORE, step s+1 (tiles and row scales by
// DMA, the weight scales into sw for the next step) is loaded into the other stage
// while this one is computed.
template <int ST, int NM, bool MORE>
__device__ __forceinline__ void k_step(const TileCtx& c, int s, int arow0, const int (&brow)[4], int lsa_off,
                                       int lane, float (&sw)[2], f32x4 (&acc)[kRB][4]) {
  if constexpr (MORE) dma_step<(ST + 1) % 2>(c, s + 1);
  fence();
  compute_step<ST, NM>(arow0, brow, lsa_off, sw, lane, acc);
  fence();
  // the next step's weight scales: scalar loads issued after this step's last use of sw,
  // so that no wait for them falls among this step's LDS reads; the barrier's lgkmcnt(0)
  // covers them
  if constexpr (MORE) wscales(c, s + 1, sw);
  fence();
  step_barrier();
}

// The K loop of one tile: stage s % 2 is computed while step s+1 is loaded into the
// other stage. With an odd number of steps (more than one) the first runs from stage 1,
// so the rest pair up (stage 0, stage 1). On exit no load is in flight and every wave
// is past the last read of the stages.
template <bool GATED, int NM>
__device__ __forceinline__ void mainloop(const TileCtx& c, f32x4 (&acc)[kRB][4]) {
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = wave / 4, wn = wave % 4;
  const int arow0 = GR * g + lane % 16;
  const int lsa_off = GS * g + kScalePitch * (lane % 16);  // row scales of rows arow0 + 16 mb
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
    k_step<1, NM, true>(c, 0, arow0, brow, lsa_off, lane, sw, acc);  // nk = 1: loads nothing more
    s = 1;
  } else {
    dma_step<0>(c, 0);
    step_barrier();
  }
  for (; s + 2 < c.nk; s += 2) {
    k_step<0, NM, true>(c, s, arow0, brow, lsa_off, lane, sw, acc);
    k_step<1, NM, true>(c, s + 1, arow0, brow, lsa_off, lane, sw, acc);
  }
  if (s < c.nk) {  // not for a single step
    k_step<0, NM, true>(c, s, arow0, brow, lsa_off, lane, sw, acc);
    k_step<1, NM, false>(c, s + 1, arow0, brow, lsa_off, lane, sw, acc);
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

  const int n_r = args.n_r;
  const int bn_out = GATED ? BNB / 2 : BNB;
  const int ntn = args.N / bn_out;
  build_tile_map<TR, GATED>(tm, args.offset, n_r, args.n_shared_groups, args.T, ntn);
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
    // Load offsets are bytes from wave-uniform bases: the gathered rows of phase 1 from the
    // quantised u itself (T * d bytes; moe_grouped_ffn refuses FP8 shapes where that reaches
    // 2^32), every other A operand from the tile's first row, B from the tile's weights.
    const bool gathered = routed && args.gather != nullptr;
    const int64_t lda = routed ? args.lda_routed : args.lda_shared;
    auto a_row = [&](int r) -> int64_t {  // A row of tile row r (clamped), relative to abase
      if (r >= t.rows) r = t.rows - 1;
      return gathered ? args.gather[row_base + t.m0 + r] : r;
    };
    {
      const uint8_t* a0 = routed ? a_routed : a_shared;
      const int64_t first = gathered ? 0 : (routed ? row_base : 0) + t.m0;  // row of A at offset 0
      c.abase = uniform_ptr(a0 + first * lda);
    }
    const int64_t eidx = routed ? t.group : sg;
    const int64_t eoff = eidx * args.b_expert_stride;
    const uint8_t* b1r = reinterpret_cast<const uint8_t*>(args.b1_routed);
    const uint8_t* b3r = reinterpret_cast<const uint8_t*>(args.b3_routed);
    const uint8_t* b1s = reinterpret_cast<const uint8_t*>(args.b1_shared);
    const uint8_t* b3s = reinterpret_cast<const uint8_t*>(args.b3_shared);
    c.load_a = __builtin_amdgcn_readfirstlane(8 * kDmaA * wave < t.rows ? 1 : 0) != 0;
    {
      const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(stages)));
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      c.lds_a = lds0 + static_cast<uint32_t>(8 * kDmaA * wv * BK);
      c.lds_b = lds0 + static_cast<uint32_t>(kOpA + 32 * wv * BK);
      c.lds_scale = lds0 + static_cast<uint32_t>(kOpA + kOpB + 4 * kWave * wv);
      c.load_scale = wv < kScaleSlots / kWave;
    }
    // this lane's load rows: 8 kDmaA wave + 8j + lane/8 of the tile's A rows (and 32 wave +
    // 8j + lane/8 of its B rows), slot lane%8, holding global chunk slot ^ ((row/2)%8) (the
    // swizzle of swz)
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) {
      const int r = 8 * kDmaA * wave + 8 * j + lane / 8;
      const int chunk = (lane % 8) ^ ((r >> 1) & 7);
      c.a[j] = static_cast<uint32_t>(a_row(r) * lda + chunk * 16);
    }
    {
      const uint8_t* base;
      if (GATED)  // tile rows 0..127 gate, 128..255 up (a wave's 32 rows lie in one)
        base = (wave < 4 ? (routed ? b1r : b1s) : (routed ? b3r : b3s)) + eoff;
      else
        base = routed ? b1r + eoff : b1s;
      constexpr int R = GATED ? 128 : 256;  // [E][N/R][K/128][R][128]: one K-step of the tile is R contiguous rows
      c.bbase = uniform_ptr(args.b_tiled ? base + (t.n0 / R) * (args.ldb / BK) * (R * BK) : base + t.n0 * args.ldb);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 32 * wave + 8 * j + lane / 8;
        const int chunk = (lane % 8) ^ ((r >> 1) & 7);
        const int64_t nrow = GATED ? (r & 127) : r;  // weight row within the tile
        c.b[j] = static_cast<uint32_t>((args.b_tiled ? nrow * BK : nrow * args.ldb) + chunk * 16);
      }
    }
    {  // scales are indexed by sorted row (routed) or token (shared), not by the gathered A row.
      // LDS slot GS g + 12 c + mb holds row GR g + 16 mb + c (padding slots: row GR g + c)
      const int slot = tid % kScaleSlots;
      const int sg2 = slot / GS, c12 = (slot % GS) / kScalePitch, mb = slot % kScalePitch;
      int r = GR * sg2 + 16 * (mb < kRB ? mb : 0) + c12;
      if (r >= t.rows) r = t.rows - 1;
      c.sbase = uniform_ptr(routed ? fa.sa_routed + row_base + t.m0 : fa.sa_shared + t.m0);
      c.s = static_cast<uint32_t>(4 * r);
      c.sa_step = 4 * (routed ? fa.ldsa_routed : fa.ldsa_shared);
    }
    // weight-scale rows: [expert][N/128][K/128]
    const int64_t sbe = (routed || GATED) ? eidx * fa.sb_expert_stride : 0;
    if (GATED) {
      const int64_t nblk = t.n0 / 128;
      c.sb[0] = uniform_scales((routed ? fa.sb1_routed : fa.sb1_shared) + sbe + nblk * fa.kblocks);
      c.sb[1] = uniform_scales((routed ? fa.sb3_routed : fa.sb3_shared) + sbe + nblk * fa.kblocks);
    } else {
      const int64_t nblk = t.n0 / 128 + wn / 2;  // the wave's 64 columns lie in one block
      c.sb[0] = c.sb[1] = uniform_scales((routed ? fa.sb1_routed : fa.sb1_shared) + sbe + nblk * fa.kblocks);
    }
    c.seg_stride = (!routed && !GATED) ? args.b_expert_stride : 0;
    c.bstep = args.b_tiled ? (GATED ? 128 : 256) * BK : BK;
    c.sb_seg_stride = (!routed && !GATED) ? fa.sb_expert_stride : 0;
    c.kseg_steps = args.K / BK;
    c.kseg_inv = kseg_recip(c.kseg_steps);
    c.nk = (routed ? args.K : args.K * (GATED ? 1 : args.k_segments)) / BK;

    f32x4 acc[kRB][4];
#pragma unroll
    for (int a = 0; a < kRB; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{};

    int vblk = (t.rows - GR * g + 31) / 32;
    vblk = vblk < 0 ? 0 : (vblk > kNM ? kNM : vblk);
    vblk = __builtin_amdgcn_readfirstlane(vblk);
    static_assert(kNM == 5, "the K loop is specialised for 0..5 live 32-row blocks");
    switch (vblk) {  // every wave runs the same loads and barriers; only the MFMA count differs
      case 5: mainloop<GATED, 5>(c, acc); break;
      case 4: mainloop<GATED, 4>(c, acc); break;
      case 3: mainloop<GATED, 3>(c, acc); break;
      case 2: mainloop<GATED, 2>(c, acc); break;
      case 1: mainloop<GATED, 1>(c, acc); break;
      default: mainloop<GATED, 0>(c, acc); break;
    }

    // epilogue: the MFMA took the weight fragment first, so a lane holds token row
    // GR g + 16 mb + lane%16 and, in each 16-column block nb, the 4 consecutive columns
    // 4 (lane/16) + v
    const int rc = lane % 16, q = lane / 16;
    if (GATED) {
      // H = SiLU(gate) * up, then per-row 1x128 quantisation over the tile's 128 gate
      // columns (spread over the 4 waves of the group): amax per row via LDS
      float* amaxbuf = reinterpret_cast<float*>(stage<0>());  // [4 waves][TR rows]
      float h[kRB][2][4];
#pragma unroll
      for (int mb = 0; mb < kRB; ++mb) {
        float m = 0.0f;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            h[mb][nb][v] = silu(acc[mb][nb][v]) * acc[mb][nb + 2][v];
            m = fmaxf(m, fabsf(h[mb][nb][v]));
          }
        m = fmaxf(m, __shfl_xor(m, 16, kWave));
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        if (q == 0) amaxbuf[wn * TR + GR * g + 16 * mb + rc] = m;
      }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < kRB; ++mb) {
        const int i = GR * g + 16 * mb + rc;
        const float amax =
            fmaxf(fmaxf(amaxbuf[i], amaxbuf[TR + i]), fmaxf(amaxbuf[2 * TR + i], amaxbuf[3 * TR + i]));
        if (i >= t.rows) continue;
        const float s = amax / 448.0f;
        const float rs = s == 0.0f ? 0.0f : 1.0f / s;  // H's codes: h * (1/s), one division per row
        const int64_t m = t.m0 + i;
        uint8_t* orow;
        float* srow;
        if (routed) {
          orow = reinterpret_cast<uint8_t*>(args.out_routed) + (row_base + m) * args.ldo_routed;
          srow = fa.os_routed + (t.n0 / 128) * fa.ldos_routed + row_base + m;
        } else {
          orow = reinterpret_cast<uint8_t*>(args.out_shared) + m * args.ldo_shared +
                 static_cast<int64_t>(sg) * args.N;
          srow = fa.os_shared + (static_cast<int64_t>(sg) * (args.N / 128) + t.n0 / 128) * fa.ldos_shared + m;
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          uint32_t codes = 0;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            codes |= e4m3(h[mb][nb][v] * rs) << (8 * v);
          *reinterpret_cast<uint32_t*>(orow + t.n0 + 32 * wn + 16 * nb + 4 * q) = codes;
        }
        if (wn == 0 && q == 0) *srow = s;
      }
      __syncthreads();  // amaxbuf (LDS stage 0) is reused by the next tile
    } else {
#pragma unroll
      for (int mb = 0; mb < kRB; ++mb) {
        if (mb >= 2 * vblk) continue;
        const int i = GR * g + 16 * mb + rc;
        if (i >= t.rows) continue;
        const int64_t m = t.m0 + i;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = t.n0 + 64 * wn + 16 * nb + 4 * q;
          if (routed) {
            uint2 o;
            o.x = pack_bf16x2(acc[mb][nb][0], acc[mb][nb][1]);
            o.y = pack_bf16x2(acc[mb][nb][2], acc[mb][nb][3]);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(args.out_routed) + (row_base + m) * args.ldo_routed + n) = o;
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(args.out_shared) + m * args.ldo_shared + n) =
                make_float4(acc[mb][nb][0], acc[mb][nb][1], acc[mb][nb][2], acc[mb][nb][3]);
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

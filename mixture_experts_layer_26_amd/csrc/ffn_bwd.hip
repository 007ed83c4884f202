// Backward of the grouped SwiGLU experts (bf16 operands, fp32 accumulation, bf16
// gradients: the quantisation section of "DeepSeek モデルアーキテクチャ徹底解説" computes
// the backward's gradients in BF16).
//
// For one expert with rows X (the tokens routed to it, in sorted-row order), output
// gradient dY, a = X W1^T, v = X W3^T, h = SiLU(a) v and y = h W2^T:
//   dh = dY W2,  da = dh v SiLU'(a),  dv = dh SiLU(a),  dX = da W1 + dv W3,
//   dW1 = da^T X,  dW3 = dv^T X,  dW2 = dY^T h.
// Five launches, each a grid of output tiles (v_mfma_f32_32x32x16_bf16, each wave a grid
// of 32 x 32 blocks), K through a ring of LDS stages filled by global_load_lds_dwordx4
// (no staging registers):
//   kAV:     256 rows x 128 d_ff tiles on 8 waves, K = d in steps of 64: a and v in two
//            accumulators; the epilogue stores h (bf16, as the forward forms it) and a, v
//            (fp32, for the next launch).
//   kDh:     256 rows x 256 d_ff tiles on 8 waves (128 d_ff when d_ff % 256 != 0), K = d in
//            steps of 64: dh; the epilogue reads a and v and stores da and dv in bf16.
//   kDx:     256 rows x 256 d tiles on 8 waves, K = d_ff in steps of 32 (the shared
//            experts' K ranges one after another): dX = da W1 + dv W3.
//   kDw13:   128 d_ff x 128 d tiles per expert on 4 waves, K = the expert's rows: dW1, dW3
//            (two workgroups per CU hide the short K loops' ends better than one of 8 waves).
//   kDw2:    256 d x 128 d_ff tiles per expert on 8 waves, K = the expert's rows: dW2.
// The tile shapes trade FLOP per staged byte, which bounds these loops (the L1 keeps a
// fixed number of line requests in flight), against workgroups per CU, which hide the
// ends of short K loops.
// The routed rows of X are read from a sorted copy of u (gathered once per call), so no
// index lookups sit in the K loops.
// Operands whose K is contiguous in memory (X in kAV, dY in kDh, da, dv in kDx, the rows
// of W1/W3 in kAV) are staged as [rows][BK k] and read with ds_read_b128. Operands
// whose K runs across rows (W2 in kDh, W1/W3 in kDx, everything in the weight
// gradients) are staged as they lie, [BK k][columns], and read with
// ds_read_b64_tr_b16, which hands each lane four consecutive k of one column: within
// 16 lanes, lane i receives column i of the 4 x 16 block whose rows the lanes'
// addresses name (lane j points at row j / 4, columns 4 (j % 4) .. + 3). Two such reads
// give the 8 consecutive k of an MFMA operand fragment.
#include "device.h"
#include "launch.h"

namespace moe {

namespace {

enum { kDx = 1, kDw13 = 2, kDw2 = 3, kAV = 4, kDh = 5, kDh128 = 6 };
// modes whose row tiles span d_ff columns, one group per shared expert
template <int MODE> constexpr bool kRowsByFf = MODE == kAV || MODE == kDh || MODE == kDh128;

// Per mode: NA A operands (M side) and NB B operands (N side) with their K-major flags;
// NACC accumulators; a WM x WN grid of waves, each NMB x NNB blocks of 32 x 32, so the
// tile is TM = 32 WM NMB rows by TN = 32 WN NNB columns; kOcc: waves per SIMD the
// register budget is held to; NST: LDS stages in the load ring (NST - 1 K-steps in
// flight); BK: K per step. Operands whose K runs along their rows take whole 128-byte
// lines per row with BK = 64; with BK = 32 each line is requested twice, a step apart.
template <int MODE> struct Cfg;
template <> struct Cfg<kAV> {  // A: X (K-contiguous); B: W1, W3 (K-contiguous)
  static constexpr int NA = 1, NB = 2, NACC = 2, WM = 4, WN = 2, NMB = 2, NNB = 2, kOcc = 2, NST = 2, BK = 64;
  static constexpr bool a_km = false;
  static constexpr bool b_km(int) { return false; }
};
template <> struct Cfg<kDh> {  // A: dY (K-contiguous); B: W2 (K-major)
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 2, WN = 4, NMB = 4, NNB = 2, kOcc = 2, NST = 2, BK = 64;
  static constexpr bool a_km = false;
  static constexpr bool b_km(int) { return true; }
};
template <> struct Cfg<kDh128> {  // as kDh, 128 d_ff columns per tile
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 4, WN = 2, NMB = 2, NNB = 2, kOcc = 2, NST = 2, BK = 64;
  static constexpr bool a_km = false;
  static constexpr bool b_km(int) { return true; }
};
template <> struct Cfg<kDx> {  // A: da, dv (K-contiguous); B: W1, W3 (K-major)
  static constexpr int NA = 2, NB = 2, NACC = 1, WM = 2, WN = 4, NMB = 4, NNB = 2, kOcc = 2, NST = 2, BK = 32;
  static constexpr bool a_km = false;
  static constexpr bool b_km(int) { return true; }
};
template <> struct Cfg<kDw13> {  // A: da, dv; B: X (all K-major)
  static constexpr int NA = 2, NB = 1, NACC = 2, WM = 2, WN = 2, NMB = 2, NNB = 2, kOcc = 2, NST = 3, BK = 32;
  static constexpr bool a_km = true;
  static constexpr bool b_km(int) { return true; }
};
template <> struct Cfg<kDw2> {  // A: dY; B: h (K-major)
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 4, WN = 2, NMB = 2, NNB = 2, kOcc = 2, NST = 3, BK = 32;
  static constexpr bool a_km = true;
  static constexpr bool b_km(int) { return true; }
};
template <int MODE> constexpr int kWaves = Cfg<MODE>::WM * Cfg<MODE>::WN;
template <int MODE> constexpr int kTM = 32 * Cfg<MODE>::WM * Cfg<MODE>::NMB;
template <int MODE> constexpr int kTN = 32 * Cfg<MODE>::WN * Cfg<MODE>::NNB;
// bytes of operand op's tile in one stage, and its offset in the stage
template <int MODE> constexpr int op_bytes(int op) {
  return (op < Cfg<MODE>::NA ? kTM<MODE> : kTN<MODE>) * Cfg<MODE>::BK * 2;
}
template <int MODE> constexpr int op_offset(int op) {
  int o = 0;
  for (int i = 0; i < op; ++i) o += op_bytes<MODE>(i);
  return o;
}
template <int MODE> constexpr int kStageBytes = op_offset<MODE>(Cfg<MODE>::NA + Cfg<MODE>::NB);

// LDS offsets. K-contiguous tile [128 rows][BK k]: 2 BK-byte rows; 16-byte chunk c of row r
// at chunk c ^ ((r >> 2) & 3) (BK = 32) or c ^ ((r >> 1) & 7) (BK = 64), so the 32 rows of a
// fragment read cover all banks.
template <int BK>
__device__ __forceinline__ int kc_swz(int r) { return BK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
template <int BK>
__device__ __forceinline__ int kc_off(int r, int c) { return r * (2 * BK) + ((c ^ kc_swz<BK>(r)) << 4); }
// K-major tile [BK k][W columns]: RB = 2 W-byte rows, 64-byte unit q of row k at q ^ (k & 3),
// so the 4 rows of one transposed read fall in different banks.
template <int RB>
__device__ __forceinline__ int km_off(int k, int byte) { return k * RB + ((((byte >> 6) ^ (k & 3))) << 6) + (byte & 63); }

typedef short v4s __attribute__((ext_vector_type(4)));

// MFMA fragment (8 consecutive k of row/column `lane % 32` of a 32-block) of sub-step s.
template <int BK>
__device__ __forceinline__ bf16x8 frag_kc(const unsigned char* t, int r0, int s, int lane) {
  return *reinterpret_cast<const bf16x8*>(t + kc_off<BK>(r0 + lane % 32, 2 * s + lane / 32));
}
template <int RB>
__device__ __forceinline__ bf16x8 frag_km(const unsigned char* t, int c0, int s, int lane) {
  const int g = lane / 16, j = lane % 16;
  const int col = c0 + 16 * (g % 2) + 4 * (j % 4);
  const int k = 16 * s + 8 * (g / 2) + j / 4;
  typedef __attribute__((address_space(3))) v4s lds_v4s;  // the tile lives in LDS
  unsigned char* p = const_cast<unsigned char*>(t);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + km_off<RB>(k, 2 * col)));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + km_off<RB>(k + 4, 2 * col)));
  typedef short v8s __attribute__((ext_vector_type(8)));
  const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, both);
}

// Tile order for the L2s. Workgroup b runs on XCD b % 8 (dispatch is round-robin over
// the 8 XCDs). Chunks of 32 consecutive tiles go to one XCD and the chunks alternate over
// the XCDs, so tiles that share an operand (the column tiles of a row block, and the row
// blocks of one expert) run on one XCD and share its L2, while the tiles -- real ones and
// the empty ones at the end of an upper-bound grid alike -- spread evenly over the XCDs.
// The grid is a multiple of 256, so this is a permutation of the tile indices.
// Measured per launch at V3 prefill, it helps the a/v (6.89 -> 6.78 ms), dh (3.70 -> 3.57)
// and dW2 (4.71 -> 4.48) launches and hurts dW1/dW3 (9.06 -> 9.49); dX is unchanged. The
// launches that gain use it.
constexpr int kChunk = 32;
template <int MODE> constexpr bool kChunked = MODE == kAV || MODE == kDh || MODE == kDh128 || MODE == kDw2;
template <int MODE>
__device__ __forceinline__ int chunked_tile(int b) {
  if constexpr (!kChunked<MODE>) return b;
  const int x = b % 8, j = b / 8;
  return ((j / kChunk) * 8 + x) * kChunk + j % kChunk;
}
inline unsigned grid_of(int64_t tiles) { return static_cast<unsigned>((tiles + 8 * kChunk - 1) / (8 * kChunk) * (8 * kChunk)); }

// Where a tile's rows, weights and outputs are.
struct Ctx {
  int g;          // group: routed expert (< n_r) or shared expert / shared group
  bool shared;
  int64_t row0;   // first row of the group in the routed row space (routed) or 0 (shared)
  int rows;       // rows of the group (kDw*: the K extent) or valid rows of the tile (row-tile modes)
  int64_t m0;     // tile's first row within the group (row-tile modes), else 0
  int c0;         // tile's first output column (kAV, kDh: d_ff; kDx: d)
  int mo, no;     // kDw*: tile's first output row / column
  int nk;         // K-steps
};

// Row tiles of kAV / kDh / kDx: groups are the routed experts, then the shared groups
// (kAV, kDh: each shared expert; kDx: one group for all of them). The offsets are copied
// to LDS (soff, n_r + 1 entries) and one thread walks the groups. Returns false past
// the last tile.
template <int MODE>
__device__ bool decode_row_tile(const BwdArgs& a, int id, Ctx& c, int* sh, int* soff) {
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>;
  const int nsg = a.n_s == 0 ? 0 : (kRowsByFf<MODE> ? a.n_s : 1);
  const int ntn = (kRowsByFf<MODE> ? a.F : a.d) / TN;
  for (int i = threadIdx.x; i <= a.n_r; i += blockDim.x) soff[i] = a.offset[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    int base = 0, found = -1, rb = 0;
    for (int g = 0; g < a.n_r + nsg && found < 0; ++g) {
      const int r = g < a.n_r ? soff[g + 1] - soff[g] : static_cast<int>(a.T);
      const int n = ((r + TM - 1) / TM) * ntn;
      if (id < base + n) {
        found = g;
        rb = id - base;
      }
      base += n;
    }
    sh[0] = found;
    sh[1] = rb;
  }
  __syncthreads();
  const int g = sh[0], rb = sh[1];
  if (g < 0) return false;
  c.g = g;
  c.shared = g >= a.n_r;
  const int r = c.shared ? static_cast<int>(a.T) : soff[g + 1] - soff[g];
  c.row0 = c.shared ? 0 : soff[g];
  c.m0 = static_cast<int64_t>(rb / ntn) * TM;
  c.c0 = (rb % ntn) * TN;
  c.rows = r - static_cast<int>(c.m0) < TM ? r - static_cast<int>(c.m0) : TM;
  return true;
}

// Global address of the 16 bytes one lane copies for operand op at K-step kt.
// K-contiguous operands: (x, y) = (tile row, 8-element chunk of the step's BK k); rows past
// the tile's rows repeat its last row (they feed only outputs that are not stored).
// K-major operands: (x, y) = (K-row of the step, first of 8 columns); K-rows past the
// group's rows (weight gradients) read the zeroed 16 bytes at a.zero.
template <int MODE>
__device__ __forceinline__ const uint16_t* src(const BwdArgs& a, const Ctx& c, bool is_a, int op, int x, int y,
                                               int kt) {
  const int64_t F = a.F, d = a.d;
  if constexpr (MODE == kAV) {
    if (is_a) {  // X (sorted copy), row x of the tile, k = BK kt + 8 y
      const int64_t row = c.m0 + (x < c.rows ? x : c.rows - 1);
      const int64_t k = static_cast<int64_t>(Cfg<MODE>::BK) * kt + 8 * y;
      return c.shared ? a.u + row * d + k : a.xs + (c.row0 + row) * d + k;
    }
    // W1 / W3 row c0 + x, k contiguous
    const int e = c.shared ? c.g - a.n_r : c.g;
    const uint16_t* w = c.shared ? (op == 0 ? a.w1s : a.w3s) : (op == 0 ? a.w1r : a.w3r);
    return w + static_cast<int64_t>(e) * F * d + (c.c0 + x) * d + static_cast<int64_t>(Cfg<MODE>::BK) * kt + 8 * y;
  } else if constexpr (MODE == kDh || MODE == kDh128) {
    if (is_a) {  // dY, row x of the tile, k = BK kt + 8 y
      const int64_t row = c.m0 + (x < c.rows ? x : c.rows - 1);
      const int64_t k = static_cast<int64_t>(Cfg<MODE>::BK) * kt + 8 * y;
      return c.shared ? a.dout + row * d + k : a.dy_routed + (c.row0 + row) * d + k;
    }
    // W2 [d][d_ff]: K-row BK kt + x, columns c0 + y
    const int e = c.shared ? c.g - a.n_r : c.g;
    const uint16_t* w = c.shared ? a.w2s : a.w2r;
    const int64_t k = static_cast<int64_t>(Cfg<MODE>::BK) * kt + x;
    return w + static_cast<int64_t>(e) * d * F + k * F + c.c0 + y;
  } else if constexpr (MODE == kDx) {
    const int64_t kk = static_cast<int64_t>(Cfg<MODE>::BK) * kt;  // K position (shared: across the experts)
    if (is_a) {  // da / dv row x
      const int64_t row = c.m0 + (x < c.rows ? x : c.rows - 1);
      const int64_t k = kk + 8 * y;
      if (c.shared) return (op == 0 ? a.da_s : a.dv_s) + row * (a.n_s * F) + k;
      return (op == 0 ? a.da_r : a.dv_r) + (c.row0 + row) * F + k;
    }
    // W1 / W3 [d_ff][d]: K-row j, columns c0 + y
    const int64_t seg = c.shared ? kk / F : c.g;
    const int64_t j = kk - (c.shared ? seg * F : 0) + x;
    const uint16_t* w = c.shared ? (op == 0 ? a.w1s : a.w3s) : (op == 0 ? a.w1r : a.w3r);
    return w + seg * F * d + j * d + c.c0 + y;
  } else {
    // weight gradients: K-row = row BK kt + x of the group, columns y
    const int64_t row = static_cast<int64_t>(Cfg<MODE>::BK) * kt + x;
    if (row >= c.rows) return a.zero;
    const int s = c.shared ? c.g - a.n_r : 0;
    if constexpr (MODE == kDw13) {
      if (is_a) {  // da / dv columns mo.. (d_ff)
        if (c.shared) return (op == 0 ? a.da_s : a.dv_s) + row * (a.n_s * F) + s * F + c.mo + y;
        return (op == 0 ? a.da_r : a.dv_r) + (c.row0 + row) * F + c.mo + y;
      }
      // X columns no.. (d)
      return c.shared ? a.u + row * d + c.no + y : a.xs + (c.row0 + row) * d + c.no + y;
    } else {
      if (is_a) {  // dY columns mo.. (d)
        if (c.shared) return a.dout + row * d + c.mo + y;
        return a.dy_routed + (c.row0 + row) * d + c.mo + y;
      }
      if (c.shared) return a.h_s + row * (a.n_s * F) + s * F + c.no + y;  // h columns no.. (d_ff)
      return a.h_r + (c.row0 + row) * F + c.no + y;
    }
  }
}

typedef __attribute__((address_space(3))) unsigned char* lds_ptr;

// One global_load_lds_dwordx4: lane i copies the 16 bytes at gptr (its own address) to
// LDS byte lds + 16 i. M0 holds the LDS address (one wait state after writing it). The
// instruction is written out so that the compiler adds no wait of its own before the LDS
// reads; the waits are the explicit ones in ring_wait.
__device__ __forceinline__ void dma16(const void* gptr, const unsigned char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0) : "memory");
}

// Loads of K-step kt into one stage: each operand's tile is split evenly over the waves,
// 64 16-byte slots per instruction (slot = per-wave share * w + 64 i + lane). The lane
// picks the global chunk whose swizzled LDS position is its slot.
template <int MODE>
__device__ __forceinline__ void dma_step(const BwdArgs& a, const Ctx& c, int kt, unsigned char* stage, int w,
                                         int lane) {
  constexpr int NA = Cfg<MODE>::NA, NB = Cfg<MODE>::NB, BK = Cfg<MODE>::BK, NW = kWaves<MODE>;
#pragma unroll
  for (int op = 0; op < NA + NB; ++op) {
    const bool km = op < NA ? Cfg<MODE>::a_km : Cfg<MODE>::b_km(op - NA);
    const int width = op < NA ? kTM<MODE> : kTN<MODE>;  // tile rows (K-contig.) or columns (K-major)
    const int per_wave = op_bytes<MODE>(op) / 16 / NW;   // slots
#pragma unroll
    for (int i = 0; i < per_wave / 64; ++i) {
      const int slot = per_wave * w + 64 * i + lane;
      int x, y;
      if (km) {  // slot = (width / 8) k + 4 (unit ^ (k & 3)) + 16-byte piece of the unit
        const int spr = width / 8;
        x = slot / spr;
        const int ws = slot % spr;
        y = (((ws / 4) ^ (x & 3)) * 32) + (ws % 4) * 8;
      } else {  // slot = (BK / 8) r + (chunk ^ swizzle(r))
        x = slot / (BK / 8);
        y = (slot % (BK / 8)) ^ kc_swz<BK>(x);
      }
      dma16(src<MODE>(a, c, op < NA, op < NA ? op : op - NA, x, y, kt),
            stage + op_offset<MODE>(op) + (per_wave * w + 64 * i) * 16);
    }
  }
}

template <int MODE>
constexpr int loads_per_step() {
  int n = 0;
  for (int op = 0; op < Cfg<MODE>::NA + Cfg<MODE>::NB; ++op) n += op_bytes<MODE>(op) / 16 / kWaves<MODE> / 64;
  return n;
}

// Wait until this wave's loads of the oldest stage in flight have landed (the N loads
// issued after them may stay in flight), then the workgroup barrier.
template <int N>
__device__ __forceinline__ void ring_wait() {
  if constexpr (N == 0)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int MODE>
__device__ __forceinline__ void compute(const unsigned char* base,
                                        f32x16 (&acc)[Cfg<MODE>::NACC][Cfg<MODE>::NMB][Cfg<MODE>::NNB], int wm,
                                        int wn, int lane) {
  constexpr int NA = Cfg<MODE>::NA, NB = Cfg<MODE>::NB, BK = Cfg<MODE>::BK;
  constexpr int NMB = Cfg<MODE>::NMB, NNB = Cfg<MODE>::NNB;
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>;
  const int r0 = (TM / Cfg<MODE>::WM) * wm, n0 = (TN / Cfg<MODE>::WN) * wn;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    bf16x8 fa[NA][NMB], fb[NB][NNB];
#pragma unroll
    for (int op = 0; op < NA; ++op)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const unsigned char* t = base + op_offset<MODE>(op);
        fa[op][mb] = Cfg<MODE>::a_km ? frag_km<2 * TM>(t, r0 + 32 * mb, s, lane)
                                     : frag_kc<BK>(t, r0 + 32 * mb, s, lane);
      }
#pragma unroll
    for (int op = 0; op < NB; ++op)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const unsigned char* t = base + op_offset<MODE>(NA + op);
        fb[op][nb] = Cfg<MODE>::b_km(op) ? frag_km<2 * TN>(t, n0 + 32 * nb, s, lane)
                                         : frag_kc<BK>(t, n0 + 32 * nb, s, lane);
      }
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        // the n-side fragment goes first, so each lane's accumulator holds 4 consecutive
        // output columns of one output row (see the epilogue)
        if constexpr (MODE == kAV) {
          acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][nb], fa[0][mb], acc[0][mb][nb], 0, 0, 0);
          acc[1][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][nb], fa[0][mb], acc[1][mb][nb], 0, 0, 0);
        } else if constexpr (MODE == kDx) {
          acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][nb], fa[0][mb], acc[0][mb][nb], 0, 0, 0);
          acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][nb], fa[1][mb], acc[0][mb][nb], 0, 0, 0);
        } else if constexpr (MODE == kDw13) {
          acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][nb], fa[0][mb], acc[0][mb][nb], 0, 0, 0);
          acc[1][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][nb], fa[1][mb], acc[1][mb][nb], 0, 0, 0);
        } else {
          acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0][nb], fa[0][mb], acc[0][mb][nb], 0, 0, 0);
        }
      }
  }
}

template <int MODE>
__global__ __launch_bounds__(64 * kWaves<MODE>, Cfg<MODE>::kOcc) void ffn_bwd_kernel(BwdArgs a) {
  constexpr int NACC = Cfg<MODE>::NACC, NMB = Cfg<MODE>::NMB, NNB = Cfg<MODE>::NNB;
  constexpr int NST = Cfg<MODE>::NST, BK = Cfg<MODE>::BK;
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>;
  constexpr int kStage = kStageBytes<MODE>;
  constexpr int ND = loads_per_step<MODE>();  // loads per wave per K-step
  __shared__ __align__(16) unsigned char lds[NST * kStage];
  // the tile decoder's scratch lives in the last stage, which no load touches before the
  // ring's first barrier
  int* sh = reinterpret_cast<int*>(lds + (NST - 1) * kStage);
  int* soff = sh + 2;
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = w / Cfg<MODE>::WN, wn = w % Cfg<MODE>::WN;

  Ctx c{};
  if constexpr (kRowsByFf<MODE> || MODE == kDx) {
    if (!decode_row_tile<MODE>(a, chunked_tile<MODE>(blockIdx.x), c, sh, soff)) return;
    if constexpr (kRowsByFf<MODE>)
      c.nk = a.d / BK;
    else
      c.nk = (c.shared ? a.n_s * a.F : a.F) / BK;
  } else {
    // per group: (M / TM) x (N / TN) tiles; M = d_ff, N = d (kDw13) or M = d, N = d_ff
    const int mt = (MODE == kDw13 ? a.F : a.d) / TM, nt = (MODE == kDw13 ? a.d : a.F) / TN;
    const int id = chunked_tile<MODE>(blockIdx.x);
    if (id >= (a.n_r + a.n_s) * mt * nt) return;  // the grid's rounding
    c.g = id / (mt * nt);
    const int rest = id % (mt * nt);
    c.mo = (rest / nt) * TM;
    c.no = (rest % nt) * TN;
    c.shared = c.g >= a.n_r;
    c.row0 = c.shared ? 0 : a.offset[c.g];
    c.rows = c.shared ? static_cast<int>(a.T) : a.offset[c.g + 1] - a.offset[c.g];
    c.nk = (c.rows + BK - 1) / BK;
  }

  f32x16 acc[NACC][NMB][NNB];
#pragma unroll
  for (int x = 0; x < NACC; ++x)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[x][mb][nb][v] = 0.0f;

  // load ring: steps 0 .. NST - 2 first; at step kt, once step kt has landed, the load of
  // step kt + NST - 1 goes into the stage step kt - 1 was read from (every wave is past
  // that read: it came before the barrier)
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0)
    if (s0 < c.nk) dma_step<MODE>(a, c, s0, lds + s0 * kStage, w, lane);
  for (int kt = 0; kt < c.nk; ++kt) {
    if (NST == 3 && kt + 1 < c.nk)
      ring_wait<ND>();  // step kt + 1's loads may stay in flight
    else
      ring_wait<0>();
    if (kt + NST - 1 < c.nk) dma_step<MODE>(a, c, kt + NST - 1, lds + ((kt + NST - 1) % NST) * kStage, w, lane);
    compute<MODE>(lds + (kt % NST) * kStage, acc, wm, wn, lane);
  }

  // epilogue. The MFMA's first operand indexes the output rows of its 32x32 result and the
  // second the columns: with the n-side fragment first, lane l holds output row m =
  // l % 32 of its 32-row block and columns n = 8 (v / 4) + 4 (l / 32) + v % 4 of its
  // 32-column block, i.e. 4 consecutive columns per group of 4 v: one 8-byte store each.
  const int m_in = lane % 32;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = (TM / Cfg<MODE>::WM) * wm + 32 * mb + m_in;
        const int n = (TN / Cfg<MODE>::WN) * wn + 32 * nb + 8 * p + 4 * (lane / 32);
        if constexpr (kRowsByFf<MODE>) {
          if (r >= c.rows) continue;
          const int64_t row = c.m0 + r;
          const int64_t col = c.c0 + n;
          int64_t o;
          if (c.shared)
            o = row * (a.n_s * static_cast<int64_t>(a.F)) + static_cast<int64_t>(c.g - a.n_r) * a.F + col;
          else
            o = (c.row0 + row) * a.F + col;
          if constexpr (MODE == kAV) {  // h = SiLU(a) v as the forward forms it; a, v kept in fp32
            float hv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float av = acc[0][mb][nb][4 * p + q], vv = acc[1][mb][nb][4 * p + q];
              hv[q] = av * fast_sigmoid(av) * vv;
            }
            *reinterpret_cast<uint2*>((c.shared ? a.h_s : a.h_r) + o) =
                make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
            const f32x16& x0 = acc[0][mb][nb];
            const f32x16& x1 = acc[1][mb][nb];
            *reinterpret_cast<float4*>((c.shared ? a.a_s : a.a_r) + o) =
                make_float4(x0[4 * p], x0[4 * p + 1], x0[4 * p + 2], x0[4 * p + 3]);
            *reinterpret_cast<float4*>((c.shared ? a.v_s : a.v_r) + o) =
                make_float4(x1[4 * p], x1[4 * p + 1], x1[4 * p + 2], x1[4 * p + 3]);
          } else {  // da = dh v SiLU'(a), dv = dh SiLU(a)
            const float4 a4 = *reinterpret_cast<const float4*>((c.shared ? a.a_s : a.a_r) + o);
            const float4 v4 = *reinterpret_cast<const float4*>((c.shared ? a.v_s : a.v_r) + o);
            const float aa[4] = {a4.x, a4.y, a4.z, a4.w}, vv4[4] = {v4.x, v4.y, v4.z, v4.w};
            float dav[4], dvv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float av = aa[q], vv = vv4[q];
              const float dh = acc[0][mb][nb][4 * p + q];
              const float sg = fast_sigmoid(av);
              const float silu_a = av * sg;
              dav[q] = dh * vv * sg * (1.0f + av * (1.0f - sg));
              dvv[q] = dh * silu_a;
            }
            *reinterpret_cast<uint2*>((c.shared ? a.da_s : a.da_r) + o) =
                make_uint2(pack_bf16x2(dav[0], dav[1]), pack_bf16x2(dav[2], dav[3]));
            *reinterpret_cast<uint2*>((c.shared ? a.dv_s : a.dv_r) + o) =
                make_uint2(pack_bf16x2(dvv[0], dvv[1]), pack_bf16x2(dvv[2], dvv[3]));
          }
        } else {
          const f32x16& x0 = acc[0][mb][nb];
          if constexpr (MODE == kDx) {
            if (r >= c.rows) continue;
            const int64_t row = c.m0 + r;
            const int64_t col = c.c0 + n;
            if (c.shared)
              *reinterpret_cast<float4*>(a.dx_s + row * a.d + col) =
                  make_float4(x0[4 * p], x0[4 * p + 1], x0[4 * p + 2], x0[4 * p + 3]);
            else
              *reinterpret_cast<uint2*>(a.dx_r + (c.row0 + row) * a.d + col) =
                  make_uint2(pack_bf16x2(x0[4 * p], x0[4 * p + 1]), pack_bf16x2(x0[4 * p + 2], x0[4 * p + 3]));
          } else {
            const int64_t e = c.shared ? c.g - a.n_r : c.g;
            const int64_t M = MODE == kDw13 ? a.F : a.d, N = MODE == kDw13 ? a.d : a.F;
            const int64_t o = e * M * N + static_cast<int64_t>(c.mo + r) * N + c.no + n;
            const uint2 v0 = make_uint2(pack_bf16x2(x0[4 * p], x0[4 * p + 1]), pack_bf16x2(x0[4 * p + 2], x0[4 * p + 3]));
            if constexpr (MODE == kDw13) {
              const f32x16& x1 = acc[1][mb][nb];
              *reinterpret_cast<uint2*>((c.shared ? a.dw1s : a.dw1r) + o) = v0;
              *reinterpret_cast<uint2*>((c.shared ? a.dw3s : a.dw3r) + o) =
                  make_uint2(pack_bf16x2(x1[4 * p], x1[4 * p + 1]), pack_bf16x2(x1[4 * p + 2], x1[4 * p + 3]));
            } else {
              *reinterpret_cast<uint2*>((c.shared ? a.dw2s : a.dw2r) + o) = v0;
            }
          }
        }
      }
}

// xs[r] = u[sorted_token[r]] for the P sorted rows (16 bytes per thread); the first
// block also clears the 256 zero bytes that padded K-rows read.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ u,
                                                          const int32_t* __restrict__ sorted_token,
                                                          uint16_t* __restrict__ xs, uint16_t* __restrict__ zero,
                                                          int64_t P, int d) {
  if (blockIdx.x == 0 && threadIdx.x < 16) reinterpret_cast<uint4*>(zero)[threadIdx.x] = make_uint4(0, 0, 0, 0);
  const int cpr = d / 8;  // 16-byte chunks per row
  const int64_t n = P * cpr;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < n;
       q += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = q / cpr;
    const int ch = static_cast<int>(q % cpr);
    st16(xs + r * d + 8 * ch, ld16(u + static_cast<int64_t>(sorted_token[r]) * d + 8 * ch));
  }
}

// Row tiles of a row-tile launch: routed rows in blocks of TM per expert (at most
// P / TM + n_r blocks), shared rows in blocks of TM per shared group, times the column tiles.
template <int MODE>
int64_t row_tiles(int64_t T, int K, int n_r, int n_s, int d, int F) {
  const int64_t P = T * K, TM = kTM<MODE>;
  const int64_t ntn = (kRowsByFf<MODE> ? F : d) / kTN<MODE>;
  const int64_t nsg = n_s == 0 ? 0 : (kRowsByFf<MODE> ? n_s : 1);
  return ((P + TM - 1) / TM + n_r + nsg * ((T + TM - 1) / TM)) * ntn;
}

template <int MODE>
hipError_t launch_rows(const BwdArgs& a, hipStream_t stream) {
  const unsigned g = grid_of(row_tiles<MODE>(a.T, a.K, a.n_r, a.n_s, a.d, a.F));
  hipLaunchKernelGGL(ffn_bwd_kernel<MODE>, dim3(g), dim3(64 * kWaves<MODE>), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_backward(const BwdArgs& a, hipStream_t stream) {
  const int64_t chunks = a.T * a.K * (a.d / 8);
  const unsigned gg = static_cast<unsigned>(chunks / 256 + 1 < 8192 ? chunks / 256 + 1 : 8192);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(gg), dim3(256), 0, stream, a.u, a.sorted_token, a.xs, a.zero,
                     a.T * a.K, a.d);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if ((err = launch_rows<kAV>(a, stream)) != hipSuccess) return err;
  if ((err = (a.F % kTN<kDh> == 0 ? launch_rows<kDh>(a, stream) : launch_rows<kDh128>(a, stream))) != hipSuccess)
    return err;
  if ((err = launch_rows<kDx>(a, stream)) != hipSuccess) return err;
  const int64_t groups = a.n_r + a.n_s;
  const unsigned g3 = grid_of(groups * (a.F / kTM<kDw13>) * (a.d / kTN<kDw13>));
  hipLaunchKernelGGL(ffn_bwd_kernel<kDw13>, dim3(g3), dim3(64 * kWaves<kDw13>), 0, stream, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const unsigned g4 = grid_of(groups * (a.d / kTM<kDw2>) * (a.F / kTN<kDw2>));
  hipLaunchKernelGGL(ffn_bwd_kernel<kDw2>, dim3(g4), dim3(64 * kWaves<kDw2>), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe

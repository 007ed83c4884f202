// Backward of the grouped SwiGLU experts (bf16 operands, fp32 accumulation, bf16
// gradients: the quantisation section of "DeepSeek モデルアーキテクチャ徹底解説" computes
// the backward's gradients in BF16).
//
// For one expert with rows X (the tokens routed to it, in sorted-row order), output
// gradient dY, a = X W1^T, v = X W3^T, h = SiLU(a) v and y = h W2^T:
//   dh = dY W2,  da = dh v SiLU'(a),  dv = dh SiLU(a),  dX = da W1 + dv W3,
//   dW1 = da^T X,  dW3 = dv^T X,  dW2 = dY^T h.
// a, v and h come from the forward's gate/up GEMM (ffn_bf16.hip), which also stores a and
// v in fp32 when asked to; h is then bit for bit the forward's. Then four launches here,
// each a grid of output tiles (v_mfma_f32_32x32x16_bf16, each wave a grid of 32 x 32
// blocks), K through a ring of LDS stages filled by global_load_lds_dwordx4 (no staging
// registers):
//   kDh:     320 rows x 256 d_ff tiles on 8 waves (128 d_ff when d_ff % 256 != 0), K = d in
//            steps of 64: dh; the epilogue reads a and v and stores da and dv in bf16.
//   kDx:     320 rows x 256 d tiles on 8 waves: dX = [da dv] [W1; W3] as one GEMM whose K
//            runs over da's columns with W1, then dv's with W3 (for the shared group, over
//            all shared experts' columns in each half), in steps of 64.
// In both, a group of r rows is cut into ceil(r / 320) row blocks of equal size, as in the
// forward's GEMMs: a V3 prefill expert of 185..345 rows is then mostly one block, where
// 256-row blocks with a short last one cost two full tiles for most experts (about 40%
// of these launches' MFMA work fell on padding rows, and those experts' weights were read
// twice). The K loop is specialised on the number of 32-row blocks of a wave that hold
// rows, and a wave whose A rows all lie past the tile's rows loads no A.
//   kDw13:   128 d_ff x 128 d tiles per expert on 4 waves, K = the expert's rows: dW1, dW3
//            (two workgroups per CU hide the short K loops' ends better than one of 8 waves).
//   kDw2:    256 d x 128 d_ff tiles per expert on 8 waves, K = the expert's rows: dW2.
// The tile shapes trade FLOP per staged byte, which bounds these loops (the L1 keeps a
// fixed number of line requests in flight), against workgroups per CU, which hide the
// ends of short K loops.
// The routed rows of X are read from a sorted copy of u (gathered once per call), so no
// index lookups sit in the K loops.
// Operands whose K is contiguous in memory (dY in kDh, da, dv in kDx) are staged as
// [rows][BK k] and read with ds_read_b128. Operands
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

enum { kDx = 1, kDw13 = 2, kDw2 = 3, kDh = 5, kDh128 = 6 };
// modes whose row tiles span d_ff columns, one group per shared expert
template <int MODE> constexpr bool kRowsByFf = MODE == kDh || MODE == kDh128;

// Per mode: NA A operands (M side) and NB B operands (N side) -- in the row-tile modes A is
// K-contiguous and B K-major, in the weight-gradient modes every operand is K-major; NACC
// accumulators; a WM x WN grid of waves, each NMB x NNB blocks of 32 x 32, so the
// tile is TM = 32 WM NMB rows by TN = 32 WN NNB columns; kOcc: waves per SIMD the
// register budget is held to; NST: LDS stages in the load ring (NST - 1 K-steps in
// flight); BK: K per step. Operands whose K runs along their rows take whole 128-byte
// lines per row with BK = 64; with BK = 32 each line is requested twice, a step apart.
template <int MODE> struct Cfg;
template <> struct Cfg<kDh> {  // A: dY (K-contiguous); B: W2 (K-major)
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 2, WN = 4, NMB = 5, NNB = 2, kOcc = 2, NST = 2, BK = 64;
};
template <> struct Cfg<kDh128> {  // as kDh, 128 d_ff columns per tile
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 2, WN = 4, NMB = 5, NNB = 1, kOcc = 2, NST = 2, BK = 64;
};
template <> struct Cfg<kDx> {  // A: da, then dv (K-contiguous); B: W1, then W3 (K-major)
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 2, WN = 4, NMB = 5, NNB = 2, kOcc = 2, NST = 2, BK = 64;
};
template <> struct Cfg<kDw13> {  // A: da, dv; B: X (all K-major)
  static constexpr int NA = 2, NB = 1, NACC = 2, WM = 2, WN = 2, NMB = 2, NNB = 2, kOcc = 2, NST = 3, BK = 32;
};
template <> struct Cfg<kDw2> {  // A: dY; B: h (K-major)
  static constexpr int NA = 1, NB = 1, NACC = 1, WM = 4, WN = 2, NMB = 2, NNB = 2, kOcc = 2, NST = 3, BK = 32;
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
// Measured per launch at V3 prefill, it helped the dh (3.70 -> 3.57 ms) and dW2 (4.71 ->
// 4.48) launches (and the a/v launch these kernels had then) and hurt dW1/dW3 (9.06 ->
// 9.49); dX was unchanged. The launches that gain use it.
constexpr int kChunk = 32;
template <int MODE> constexpr bool kChunked = MODE == kDh || MODE == kDh128 || MODE == kDw2;
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
  int c0;         // tile's first output column (kDh: d_ff; kDx: d)
  int mo, no;     // kDw*: tile's first output row / column
  int nk;         // K-steps
};

// Row tiles of kDh / kDx: groups are the routed experts, then the shared groups (kDh:
// each shared expert; kDx: one group for all of them). A group of r rows has
// ceil(r / TM) row blocks of equal size (row_blocks). The offsets are copied to LDS
// (soff, n_r + 1 entries) and one thread walks the groups. Returns false past the last
// tile.
__device__ __forceinline__ int block_rows(int r, int TM) {  // rows per block (0 for r = 0)
  const int mt = (r + TM - 1) / TM;
  return mt > 0 ? (r + mt - 1) / mt : 0;
}
__device__ __forceinline__ int row_blocks(int r, int TM) {
  const int rpb = block_rows(r, TM);
  return rpb > 0 ? (r + rpb - 1) / rpb : 0;
}

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
      const int n = row_blocks(r, TM) * ntn;
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
  const int rpb = block_rows(r, TM);
  c.m0 = static_cast<int64_t>(rb / ntn) * rpb;
  c.c0 = (rb % ntn) * TN;
  c.rows = r - static_cast<int>(c.m0) < rpb ? r - static_cast<int>(c.m0) : rpb;
  return true;
}

// Element offset of (n, k) in one expert's matrix of row length K in the tiled layout of
// pack.hip, [N/R][K/64][R][64]: R = 128 for W1 and W3 (rows n over d_ff), 256 for W2 (rows
// over d). Eight consecutive k from a multiple of 8 stay within one 64-wide block.
template <int R>
__device__ __forceinline__ int64_t tiled_off(int64_t n, int64_t k, int64_t K) {
  return ((n / R) * (K / 64) + k / 64) * (R * 64) + (n % R) * 64 + k % 64;
}

typedef __attribute__((address_space(3))) unsigned char* lds_ptr;

// One global_load_lds_dwordx4: lane i copies the 16 bytes at gptr (its own address) to
// LDS byte lds + 16 i. M0 holds the LDS address (one wait state after writing it). The
// instruction is written out so that the compiler adds no wait of its own before the LDS
// reads; the waits are the explicit ones in ring_wait. M0 is declared clobbered, so the
// compiler keeps no value of its own in M0 across the statement (clang warns that M0 is a
// reserved register; the clobber is what tells its M0-initialisation passes that the
// statement writes it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gptr, const unsigned char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(m0)
               : "memory", "m0");
}

// The same in the SGPR-base form: lane i copies the 16 bytes at sbase + voff (sbase
// wave-uniform, voff the lane's 32-bit byte offset).
__device__ __forceinline__ void dma16s(uint32_t voff, const unsigned char* sbase, const unsigned char* lds) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// A wave-uniform pointer made explicit (both halves from the first lane), for dma16s.
__device__ __forceinline__ const unsigned char* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<const unsigned char*>((hi << 32) | lo);
}

// Loads of the row-tile launches (kDh, kDx): operand A (dY; kDx: da, then dv) is
// K-contiguous, B (W2; kDx: W1, then W3) is K-major. Each operand's tile is split evenly
// over the waves, 64 16-byte slots per instruction (slot = per-wave share * w + 64 i +
// lane), and each lane picks the global chunk whose swizzled LDS position is its slot:
// K-contiguous, slot = (BK / 8) r + (chunk ^ swizzle(r)); K-major, slot = (width / 8) k +
// 4 (unit ^ (k & 3)) + 16-byte piece of the unit (km_slot). Per operand a wave-uniform
// pointer (A at the tile's first row, B at K-row 0 of the expert's matrix) moves with the
// K-step by scalar arithmetic; per lane and instruction a 32-bit byte offset from it is
// made once per tile (A rows past the tile's rows repeat its last row). A wave whose A
// rows all lie past the tile's rows loads no A.
template <int MODE>
struct RowLoads {
  const unsigned char* a[2];  // A at the tile's first row (kDx: da, dv), wave-uniform
  const unsigned char* b[2];  // B of the group at K-row 0 (kDx: W1, W3), wave-uniform
  uint32_t off_a[5], off_b[4];
  bool load_a;
};
template <int MODE> constexpr int row_instrs_a() { return op_bytes<MODE>(0) / 16 / kWaves<MODE> / 64; }
template <int MODE> constexpr int row_instrs_b() { return op_bytes<MODE>(1) / 16 / kWaves<MODE> / 64; }

__device__ __forceinline__ void km_slot(int slot, int width, int& x, int& y);

template <int MODE>
__device__ __forceinline__ void row_setup(const BwdArgs& a, const Ctx& c, int w, int lane, RowLoads<MODE>& L) {
  constexpr int BK = Cfg<MODE>::BK, NW = kWaves<MODE>, TN = kTN<MODE>;
  static_assert(Cfg<MODE>::NA == 1 && Cfg<MODE>::NB == 1 && BK == 64, "row tiles: one A and one B operand");
  static_assert(row_instrs_a<MODE>() <= 5 && row_instrs_b<MODE>() <= 4, "offset arrays");
  const int64_t F = a.F, d = a.d;
  const int e = c.shared ? c.g - a.n_r : c.g;
  int64_t lda, ldk;  // A's row length; B's row length (the K-major stride)
  if constexpr (MODE == kDx) {
    lda = c.shared ? a.n_s * F : F;
    const int64_t first = (c.shared ? 0 : c.row0) + c.m0;
    L.a[0] = uniform_ptr((c.shared ? a.da_s : a.da_r) + first * lda);
    L.a[1] = uniform_ptr((c.shared ? a.dv_s : a.dv_r) + first * lda);
    L.b[0] = uniform_ptr((c.shared ? a.w1s : a.w1r) + static_cast<int64_t>(c.shared ? 0 : e) * F * d);
    L.b[1] = uniform_ptr((c.shared ? a.w3s : a.w3r) + static_cast<int64_t>(c.shared ? 0 : e) * F * d);
    ldk = d;
  } else {
    lda = d;
    L.a[0] = L.a[1] = uniform_ptr((c.shared ? a.dout : a.dy_routed + c.row0 * d) + c.m0 * d);
    L.b[0] = L.b[1] = uniform_ptr((c.shared ? a.w2s : a.w2r) + static_cast<int64_t>(e) * d * F);
    ldk = F;
  }
  constexpr int pa = op_bytes<MODE>(0) / 16 / NW, pb = op_bytes<MODE>(1) / 16 / NW;  // slots per wave
  L.load_a = __builtin_amdgcn_readfirstlane(pa * w / (BK / 8) < c.rows ? 1 : 0) != 0;
#pragma unroll
  for (int i = 0; i < row_instrs_a<MODE>(); ++i) {
    const int slot = pa * w + 64 * i + lane;
    const int x = slot / (BK / 8), y = (slot % (BK / 8)) ^ kc_swz<BK>(x);
    const int xr = x < c.rows ? x : c.rows - 1;
    L.off_a[i] = static_cast<uint32_t>(2 * (xr * lda + 8 * y));
  }
  constexpr int R = MODE == kDx ? 128 : 256;  // the tiled layout's row block of W1/W3, W2
#pragma unroll
  for (int i = 0; i < row_instrs_b<MODE>(); ++i) {
    int x, y;
    km_slot(pb * w + 64 * i + lane, TN, x, y);
    const int64_t col = c.c0 + y;
    const int64_t o = a.tiled ? (col / 64) * (R * 64) + x * 64 + col % 64 : x * ldk + col;
    L.off_b[i] = static_cast<uint32_t>(2 * o);
  }
}

template <int MODE>
__device__ __forceinline__ void row_step(const BwdArgs& a, const Ctx& c, const RowLoads<MODE>& L, int kt,
                                         unsigned char* stage, int w) {
  constexpr int BK = Cfg<MODE>::BK, NW = kWaves<MODE>;
  const int64_t F = a.F, d = a.d;
  const unsigned char *sa, *sb;
  if constexpr (MODE == kDx) {
    // K position: the first half of the steps runs over da (with W1), the second over dv
    // (with W3); each half spans F columns (routed) or n_s F (shared, one expert after
    // another). A step never straddles the halves or the experts (F is a multiple of 128).
    // The shared experts' matrices lie one after another, F rows each, so K-row kk of the
    // half is W row kk of the stacked matrices in either layout (in the tiled one, whose
    // 128-row blocks never straddle two experts, block kk / 128 and row kk % 128 of it).
    const int64_t half = c.shared ? a.n_s * F : F;
    int64_t kk = static_cast<int64_t>(BK) * kt;
    const int second = kk >= half ? 1 : 0;
    kk -= second ? half : 0;
    sa = L.a[second] + 2 * kk;
    const int64_t ob = a.tiled ? (kk >> 7) * (d / 64) * (128 * 64) + (kk & 127) * 64 : kk * d;
    sb = L.b[second] + 2 * ob;
  } else {
    sa = L.a[0] + 2 * static_cast<int64_t>(BK) * kt;
    // W2 [d][d_ff], K-rows BK kt.. (d index); tiled: 256-row blocks of 64-wide K-steps
    const int64_t k0 = static_cast<int64_t>(BK) * kt;
    const int64_t ob = a.tiled ? (k0 / 256) * (F / 64) * (256 * 64) + (k0 % 256) * 64 : k0 * F;
    sb = L.b[0] + 2 * ob;
  }
  constexpr int pa = op_bytes<MODE>(0) / 16 / NW, pb = op_bytes<MODE>(1) / 16 / NW;
  if (L.load_a) {
#pragma unroll
    for (int i = 0; i < row_instrs_a<MODE>(); ++i) dma16s(L.off_a[i], sa, stage + (pa * w + 64 * i) * 16);
  }
#pragma unroll
  for (int i = 0; i < row_instrs_b<MODE>(); ++i)
    dma16s(L.off_b[i], sb, stage + op_offset<MODE>(1) + (pb * w + 64 * i) * 16);
}

// Loads of the weight-gradient launches (every operand K-major, K = the group's rows).
// Per operand: a wave-uniform pointer to K-row 0 of the tile's columns and the bytes from
// one K-row to the next; per lane and instruction: the 32-bit byte offset of its 16 bytes
// (K-row x, column y of the step, chosen as in row_setup). A step moves the pointers by BK
// K-rows with scalar arithmetic, so the K loop spends no VALU work on addresses. Only a
// step that runs past the group's rows (its last) checks rows, lane by lane, and sends
// the lanes past them to the zeroed 16 bytes at a.zero.
template <int MODE>
constexpr int dw_instrs(int op) {
  return op_bytes<MODE>(op) / 16 / kWaves<MODE> / 64;
}
template <int MODE>
struct DwLoads {
  static constexpr int NOP = Cfg<MODE>::NA + Cfg<MODE>::NB;
  const unsigned char* base[NOP];  // wave-uniform
  int64_t row_bytes[NOP];
  uint32_t off[NOP][4];
};

// (x, y) of slot `slot` of a K-major operand `width` columns wide.
__device__ __forceinline__ void km_slot(int slot, int width, int& x, int& y) {
  const int spr = width / 8;
  x = slot / spr;
  const int ws = slot % spr;
  y = (((ws / 4) ^ (x & 3)) * 32) + (ws % 4) * 8;
}

template <int MODE>
__device__ __forceinline__ void dw_setup(const BwdArgs& a, const Ctx& c, int w, int lane, DwLoads<MODE>& L) {
  constexpr int NA = Cfg<MODE>::NA, NOP = DwLoads<MODE>::NOP, NW = kWaves<MODE>;
  const int64_t F = a.F, d = a.d, sF = static_cast<int64_t>(a.n_s) * a.F;
  const int64_t s = c.shared ? c.g - a.n_r : 0;
#pragma unroll
  for (int op = 0; op < NOP; ++op) {
    const uint16_t* p;
    int64_t ld;
    if constexpr (MODE == kDw13) {
      if (op < NA) {  // da / dv, columns mo.. (d_ff)
        ld = c.shared ? sF : F;
        p = c.shared ? (op == 0 ? a.da_s : a.dv_s) + s * F + c.mo : (op == 0 ? a.da_r : a.dv_r) + c.row0 * F + c.mo;
      } else {  // X, columns no.. (d)
        ld = d;
        p = c.shared ? a.u + c.no : a.xs + c.row0 * d + c.no;
      }
    } else {
      if (op < NA) {  // dY, columns mo.. (d)
        ld = d;
        p = c.shared ? a.dout + c.mo : a.dy_routed + c.row0 * d + c.mo;
      } else {  // h, columns no.. (d_ff)
        ld = c.shared ? sF : F;
        p = c.shared ? a.h_s + s * F + c.no : a.h_r + c.row0 * F + c.no;
      }
    }
    L.base[op] = uniform_ptr(p);
    L.row_bytes[op] = 2 * ld;
    const int width = op < NA ? kTM<MODE> : kTN<MODE>;
    const int per_wave = op_bytes<MODE>(op) / 16 / NW;
#pragma unroll
    for (int i = 0; i < dw_instrs<MODE>(op); ++i) {
      int x, y;
      km_slot(per_wave * w + 64 * i + lane, width, x, y);
      L.off[op][i] = static_cast<uint32_t>(x * 2 * ld + 2 * y);
    }
  }
}

// K-step kt's loads of the weight-gradient modes into a stage of the ring. sb[op]: the
// operands' wave-uniform pointers at K-row BK kt. A step wholly within the group's rows
// takes the SGPR-base form; the one that runs past them sends those lanes to the zeroed
// 16 bytes at a.zero. The choice is made once per step (it is wave-uniform).
template <int MODE>
__device__ __forceinline__ void dw_issue(const BwdArgs& a, const Ctx& c, const DwLoads<MODE>& L,
                                         const unsigned char* const (&sb)[DwLoads<MODE>::NOP], int kt,
                                         unsigned char* stage, int w, int lane) {
  constexpr int NA = Cfg<MODE>::NA, NOP = DwLoads<MODE>::NOP, BK = Cfg<MODE>::BK, NW = kWaves<MODE>;
  if ((kt + 1) * BK <= c.rows) {
#pragma unroll
    for (int op = 0; op < NOP; ++op) {
      const int per_wave = op_bytes<MODE>(op) / 16 / NW;
#pragma unroll
      for (int i = 0; i < dw_instrs<MODE>(op); ++i)
        dma16s(L.off[op][i], sb[op], stage + op_offset<MODE>(op) + (per_wave * w + 64 * i) * 16);
    }
  } else {
#pragma unroll
    for (int op = 0; op < NOP; ++op) {
      const int width = op < NA ? kTM<MODE> : kTN<MODE>;
      const int per_wave = op_bytes<MODE>(op) / 16 / NW;
#pragma unroll
      for (int i = 0; i < dw_instrs<MODE>(op); ++i) {
        int x, y;
        km_slot(per_wave * w + 64 * i + lane, width, x, y);
        dma16(kt * BK + x < c.rows ? static_cast<const void*>(sb[op] + L.off[op][i]) : static_cast<const void*>(a.zero),
              stage + op_offset<MODE>(op) + (per_wave * w + 64 * i) * 16);
      }
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

// One K-step's MFMAs of the row-tile modes for the first NL of the wave's NMB 32-row blocks
// (the others hold no rows of the tile).
template <int MODE, int NL>
__device__ __forceinline__ void compute(const unsigned char* base,
                                        f32x16 (&acc)[Cfg<MODE>::NACC][Cfg<MODE>::NMB][Cfg<MODE>::NNB], int wm,
                                        int wn, int lane) {
  static_assert(Cfg<MODE>::NA == 1 && Cfg<MODE>::NB == 1 && Cfg<MODE>::NACC == 1, "the row-tile modes");
  constexpr int BK = Cfg<MODE>::BK;
  constexpr int NMB = NL, NNB = Cfg<MODE>::NNB;
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>;
  const int r0 = (TM / Cfg<MODE>::WM) * wm, n0 = (TN / Cfg<MODE>::WN) * wn;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    bf16x8 fa[NMB > 0 ? NMB : 1], fb[NNB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) fa[mb] = frag_kc<BK>(base + op_offset<MODE>(0), r0 + 32 * mb, s, lane);
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) fb[nb] = frag_km<2 * TN>(base + op_offset<MODE>(1), n0 + 32 * nb, s, lane);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
        // the n-side fragment goes first, so each lane's accumulator holds 4 consecutive
        // output columns of one output row (see the epilogue)
        acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[mb], acc[0][mb][nb], 0, 0, 0);
  }
}

// This lane's fragment addresses (LDS bytes, stage 0) in the weight-gradient modes, one
// per operand and 32-block: with k = 16 s + k0 and k0 = 8 (lane/16 / 2) + lane%16 / 4, the
// swizzle term k & 3 does not depend on s, so a fragment of sub-step s lies at the base
// plus the stage's offset, plus 16 s RB (and its upper half 4 RB further), which are
// immediate offsets of the transposing read.
template <int MODE>
struct DwFrag {
  uint32_t a[Cfg<MODE>::NA][Cfg<MODE>::NMB];
  uint32_t b[Cfg<MODE>::NNB];
};

template <int MODE>
__device__ __forceinline__ void dw_frag_setup(const unsigned char* lds, int wm, int wn, int lane, DwFrag<MODE>& f) {
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>, NA = Cfg<MODE>::NA;
  const uint32_t l0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)(lds)));
  const int g = lane / 16, j = lane % 16;
  const int k0 = 8 * (g / 2) + j / 4, cl = 16 * (g % 2) + 4 * (j % 4);
  const int r0 = (TM / Cfg<MODE>::WM) * wm, n0 = (TN / Cfg<MODE>::WN) * wn;
#pragma unroll
  for (int op = 0; op < NA; ++op)
#pragma unroll
    for (int mb = 0; mb < Cfg<MODE>::NMB; ++mb)
      f.a[op][mb] = l0 + op_offset<MODE>(op) + km_off<2 * TM>(k0, 2 * (r0 + 32 * mb + cl));
#pragma unroll
  for (int nb = 0; nb < Cfg<MODE>::NNB; ++nb)
    f.b[nb] = l0 + op_offset<MODE>(NA) + km_off<2 * TN>(k0, 2 * (n0 + 32 * nb + cl));
}

// The 8 consecutive k of a fragment: two transposing reads 4 K-rows apart.
template <int RB>
__device__ __forceinline__ bf16x8 frag_at(uint32_t base, int off) {
  typedef __attribute__((address_space(3))) v4s lds_v4s;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(base + off + 4 * RB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One K-step's MFMAs of the weight-gradient modes from stage ST.
template <int MODE>
__device__ __forceinline__ void compute_dw(const DwFrag<MODE>& f, uint32_t stage_off,
                                           f32x16 (&acc)[Cfg<MODE>::NACC][Cfg<MODE>::NMB][Cfg<MODE>::NNB]) {
  constexpr int NA = Cfg<MODE>::NA, NMB = Cfg<MODE>::NMB, NNB = Cfg<MODE>::NNB, BK = Cfg<MODE>::BK;
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>;
  static_assert(16 * (BK / 16 - 1) * 2 * (TM > TN ? TM : TN) + 4 * 2 * (TM > TN ? TM : TN) < 65536,
                "the fragment offsets fit the read's 16-bit immediate");
  uint32_t ba[NA][NMB], bb[NNB];  // this step's fragment bases
#pragma unroll
  for (int op = 0; op < NA; ++op)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) ba[op][mb] = f.a[op][mb] + stage_off;
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) bb[nb] = f.b[nb] + stage_off;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    bf16x8 fa[NA][NMB], fb[NNB];
#pragma unroll
    for (int op = 0; op < NA; ++op)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) fa[op][mb] = frag_at<2 * TM>(ba[op][mb], 16 * s * 2 * TM);
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) fb[nb] = frag_at<2 * TN>(bb[nb], 16 * s * 2 * TN);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        // the n-side fragment first, as in compute
        acc[0][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[0][mb], acc[0][mb][nb], 0, 0, 0);
        if constexpr (MODE == kDw13)
          acc[1][mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[nb], fa[1][mb], acc[1][mb][nb], 0, 0, 0);
      }
  }
}

// The weight-gradient K loop, a ring of three stages: steps 0 and 1 first; at step kt, once
// it has landed (step kt + 1's loads may stay in flight), step kt + 2 goes into the stage
// step kt - 1 was read from (every wave is past that read: it came before the barrier),
// then the MFMAs. The stages' offsets rotate in scalar registers and each operand's
// pointer moves by one scalar add per step, so the loop spends its vector instructions on
// the transposing reads and the MFMAs. On exit every wave is past its last read of the ring.
template <int MODE>
__device__ __forceinline__ void k_loop_dw(const BwdArgs& a, const Ctx& c, const DwLoads<MODE>& dl,
                                          unsigned char* lds,
                                          f32x16 (&acc)[Cfg<MODE>::NACC][Cfg<MODE>::NMB][Cfg<MODE>::NNB], int w,
                                          int wm, int wn, int lane) {
  static_assert(Cfg<MODE>::NST == 3, "a ring of three stages");
  constexpr int NOP = DwLoads<MODE>::NOP, BK = Cfg<MODE>::BK, kStage = kStageBytes<MODE>;
  constexpr int ND = loads_per_step<MODE>();  // loads per wave per K-step
  const unsigned char* sb[NOP];
  int64_t adv[NOP];
#pragma unroll
  for (int op = 0; op < NOP; ++op) {
    sb[op] = dl.base[op];
    adv[op] = BK * dl.row_bytes[op];
  }
  DwFrag<MODE> f;
  dw_frag_setup<MODE>(lds, wm, wn, lane, f);
  auto issue = [&](int kt, uint32_t off) {
    dw_issue<MODE>(a, c, dl, sb, kt, lds + off, w, lane);
#pragma unroll
    for (int op = 0; op < NOP; ++op) sb[op] += adv[op];
  };
  issue(0, 0);
  if (1 < c.nk) issue(1, kStage);
  uint32_t rd = 0, wr = 2 * kStage;  // the stage read at step kt, the stage step kt + 2 goes into
  for (int kt = 0; kt < c.nk; ++kt) {
    if (kt + 1 < c.nk)
      ring_wait<ND>();
    else
      ring_wait<0>();
    if (kt + 2 < c.nk) issue(kt + 2, wr);
    compute_dw<MODE>(f, rd, acc);
    rd = rd == 2 * kStage ? 0 : rd + kStage;
    wr = wr == 2 * kStage ? 0 : wr + kStage;
  }
}

// The load ring and MFMAs of one tile, for NL live row blocks per wave. The row-tile modes
// run a ring of two stages: step 0 first; at step kt, once step kt has landed, step kt + 1
// goes into the stage step kt - 1 was read from (every wave is past that read: it came
// before the barrier). The weight-gradient modes run k_loop_dw. On exit every wave is past
// its last read of the ring.
template <int MODE, int NL>
__device__ __forceinline__ void k_loop(const BwdArgs& a, const Ctx& c, const DwLoads<MODE>& dl,
                                       const RowLoads<MODE>& rl, unsigned char* lds,
                                       f32x16 (&acc)[Cfg<MODE>::NACC][Cfg<MODE>::NMB][Cfg<MODE>::NNB], int w,
                                       int wm, int wn, int lane) {
  constexpr int NST = Cfg<MODE>::NST;
  constexpr int kStage = kStageBytes<MODE>;
  if constexpr (MODE == kDw13 || MODE == kDw2) {
    k_loop_dw<MODE>(a, c, dl, lds, acc, w, wm, wn, lane);
  } else {
    static_assert(NST == 2, "the row-tile modes run a ring of two stages");
    row_step<MODE>(a, c, rl, 0, lds, w);
    for (int kt = 0; kt < c.nk; ++kt) {
      ring_wait<0>();
      if (kt + 1 < c.nk) row_step<MODE>(a, c, rl, kt + 1, lds + ((kt + 1) % 2) * kStage, w);
      compute<MODE, NL>(lds + (kt % 2) * kStage, acc, wm, wn, lane);
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(64 * kWaves<MODE>, Cfg<MODE>::kOcc) void ffn_bwd_kernel(BwdArgs a) {
  constexpr int NACC = Cfg<MODE>::NACC, NMB = Cfg<MODE>::NMB, NNB = Cfg<MODE>::NNB;
  constexpr int NST = Cfg<MODE>::NST, BK = Cfg<MODE>::BK;
  constexpr int TM = kTM<MODE>, TN = kTN<MODE>;
  constexpr int kStage = kStageBytes<MODE>;
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
      c.nk = 2 * (c.shared ? a.n_s * a.F : a.F) / BK;
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

  constexpr bool kDw = MODE == kDw13 || MODE == kDw2;
  DwLoads<MODE> dl;
  RowLoads<MODE> rl;
  if constexpr (kDw)
    dw_setup<MODE>(a, c, w, lane, dl);
  else
    row_setup<MODE>(a, c, w, lane, rl);
  // live 32-row blocks of this wave (wave-uniform; all of them in the weight-gradient modes)
  int live = NMB;
  if constexpr (!kDw) {
    live = (c.rows - (TM / Cfg<MODE>::WM) * wm + 31) / 32;
    live = live < 0 ? 0 : (live > NMB ? NMB : live);
    live = __builtin_amdgcn_readfirstlane(live);
  }
  static_assert(NMB <= 5, "the K loop is specialised for 0..5 live row blocks");
  switch (live) {  // every wave runs the same loads and barriers; only the MFMA count differs
    case 5:
      if constexpr (NMB >= 5) k_loop<MODE, (NMB >= 5 ? 5 : 0)>(a, c, dl, rl, lds, acc, w, wm, wn, lane);
      break;
    case 4:
      if constexpr (NMB >= 4) k_loop<MODE, (NMB >= 4 ? 4 : 0)>(a, c, dl, rl, lds, acc, w, wm, wn, lane);
      break;
    case 3:
      if constexpr (NMB >= 3) k_loop<MODE, (NMB >= 3 ? 3 : 0)>(a, c, dl, rl, lds, acc, w, wm, wn, lane);
      break;
    case 2:
      if constexpr (NMB >= 2) k_loop<MODE, (NMB >= 2 ? 2 : 0)>(a, c, dl, rl, lds, acc, w, wm, wn, lane);
      break;
    case 1: k_loop<MODE, 1>(a, c, dl, rl, lds, acc, w, wm, wn, lane); break;
    default: k_loop<MODE, 0>(a, c, dl, rl, lds, acc, w, wm, wn, lane); break;
  }

  // epilogue. The MFMA's first operand indexes the output rows of its 32x32 result and the
  // second the columns: with the n-side fragment first, lane l holds output row m =
  // l % 32 of its 32-row block and columns n = 8 (v / 4) + 4 (l / 32) + v % 4 of its
  // 32-column block, i.e. 4 consecutive columns per group of 4 v: one 8-byte store each.
  const int m_in = lane % 32;
  if constexpr (MODE == kDw13 || MODE == kDw2) {
    // Weight gradients leave through LDS: a direct 8-byte store per lane would put each
    // instruction's 32 row pieces in 32 different rows (16 bytes each), and those write
    // requests, not the bytes, bounded these launches (skipping the stores took dW1/dW3
    // from 9.1 to 5.4 ms and dW2 from 4.5 to 2.5 ms at V3 prefill). The bf16 tiles of the
    // NACC outputs go into the free ring, rows padded by 16 bytes (row m's banks shift by
    // 4 per row, so a write's 32 rows meet at most in pairs), then whole rows go out with
    // 16-byte stores, TN / 8 lanes per row. The stores are non-temporal: nothing in this
    // launch reads the gradients back (6.8 and 3.4 ms instead of 7.0 and 3.5).
    constexpr int kPitch = 2 * TN + 16;
    static_assert(NACC * TM * kPitch <= NST * kStage, "the output tiles fit in the ring");
    __syncthreads();  // every wave is past its last read of the ring
#pragma unroll
    for (int x = 0; x < NACC; ++x)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int r = (TM / Cfg<MODE>::WM) * wm + 32 * mb + m_in;
            const int n = (TN / Cfg<MODE>::WN) * wn + 32 * nb + 8 * p + 4 * (lane / 32);
            const f32x16& v = acc[x][mb][nb];
            *reinterpret_cast<uint2*>(lds + (x * TM + r) * kPitch + 2 * n) =
                make_uint2(pack_bf16x2(v[4 * p], v[4 * p + 1]), pack_bf16x2(v[4 * p + 2], v[4 * p + 3]));
          }
    __syncthreads();
    const int64_t e = c.shared ? c.g - a.n_r : c.g;
    const int64_t M = MODE == kDw13 ? a.F : a.d, N = MODE == kDw13 ? a.d : a.F;
#pragma unroll
    for (int x = 0; x < NACC; ++x) {
      uint16_t* out;
      if constexpr (MODE == kDw13)
        out = x == 0 ? (c.shared ? a.dw1s : a.dw1r) : (c.shared ? a.dw3s : a.dw3r);
      else
        out = c.shared ? a.dw2s : a.dw2r;
      out += e * M * N;
      for (int idx = threadIdx.x; idx < TM * (TN / 8); idx += 64 * kWaves<MODE>) {
        const int r = idx / (TN / 8), ch = idx % (TN / 8);
        // the gradient in the weights' layout: row mo + r, columns no + 8 ch ..
        const int64_t m = c.mo + r, n = c.no + 8 * ch;
        const int64_t o = a.tiled ? (MODE == kDw13 ? tiled_off<128>(m, n, N) : tiled_off<256>(m, n, N)) : m * N + n;
        __builtin_nontemporal_store(*reinterpret_cast<const i32x4*>(lds + (x * TM + r) * kPitch + 16 * ch),
                                    reinterpret_cast<i32x4*>(out + o));
      }
    }
    return;
  }
  if constexpr (kRowsByFf<MODE>) {
    // da = dh v SiLU'(a), dv = dh SiLU(a), with a and v (fp32) from the gate/up launch. Per
    // 32 x 32 block, all of its loads of a and v are issued before any result is stored, so
    // a tile waits one load latency per block instead of one per 4 columns (the loads used
    // to wait behind the previous columns' stores: 0.5 of this launch's 3.7 ms at V3
    // prefill). Rows past the tile's read its last row and store nothing.
    const int64_t ldr = c.shared ? a.n_s * static_cast<int64_t>(a.F) : a.F;
    const int64_t col0 = (c.shared ? static_cast<int64_t>(c.g - a.n_r) * a.F : 0) + c.c0;
    const int64_t row0 = c.shared ? 0 : c.row0;
    const float* pa = c.shared ? a.a_s : a.a_r;
    const float* pv = c.shared ? a.v_s : a.v_r;
    uint16_t* pda = c.shared ? a.da_s : a.da_r;
    uint16_t* pdv = c.shared ? a.dv_s : a.dv_r;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if ((TM / Cfg<MODE>::WM) * wm + 32 * mb >= c.rows) continue;  // no row of this block (wave-uniform)
      const int r = (TM / Cfg<MODE>::WM) * wm + 32 * mb + m_in;
      const bool live = r < c.rows;
      const int64_t o = (row0 + c.m0 + (live ? r : c.rows - 1)) * ldr + col0;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        float4 a4[4], v4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int n = (TN / Cfg<MODE>::WN) * wn + 32 * nb + 8 * p + 4 * (lane / 32);
          a4[p] = *reinterpret_cast<const float4*>(pa + o + n);
          v4[p] = *reinterpret_cast<const float4*>(pv + o + n);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int n = (TN / Cfg<MODE>::WN) * wn + 32 * nb + 8 * p + 4 * (lane / 32);
          const float aa[4] = {a4[p].x, a4[p].y, a4[p].z, a4[p].w};
          const float vv[4] = {v4[p].x, v4[p].y, v4[p].z, v4[p].w};
          float dav[4], dvv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float dh = acc[0][mb][nb][4 * p + q];
            const float sg = fast_sigmoid(aa[q]);
            dav[q] = dh * vv[q] * sg * (1.0f + aa[q] * (1.0f - sg));
            dvv[q] = dh * (aa[q] * sg);
          }
          if (live) {
            *reinterpret_cast<uint2*>(pda + o + n) = make_uint2(pack_bf16x2(dav[0], dav[1]), pack_bf16x2(dav[2], dav[3]));
            *reinterpret_cast<uint2*>(pdv + o + n) = make_uint2(pack_bf16x2(dvv[0], dvv[1]), pack_bf16x2(dvv[2], dvv[3]));
          }
        }
      }
    }
  } else if constexpr (MODE == kDx) {
    // dX: bf16 for the routed rows, the fp32 sum over the shared experts for the shared group
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = (TM / Cfg<MODE>::WM) * wm + 32 * mb + m_in;
          const int n = (TN / Cfg<MODE>::WN) * wn + 32 * nb + 8 * p + 4 * (lane / 32);
          if (r >= c.rows) continue;
          const f32x16& x0 = acc[0][mb][nb];
          const int64_t row = c.m0 + r;
          const int64_t col = c.c0 + n;
          if (c.shared)
            *reinterpret_cast<float4*>(a.dx_s + row * a.d + col) =
                make_float4(x0[4 * p], x0[4 * p + 1], x0[4 * p + 2], x0[4 * p + 3]);
          else
            *reinterpret_cast<uint2*>(a.dx_r + (c.row0 + row) * a.d + col) =
                make_uint2(pack_bf16x2(x0[4 * p], x0[4 * p + 1]), pack_bf16x2(x0[4 * p + 2], x0[4 * p + 3]));
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

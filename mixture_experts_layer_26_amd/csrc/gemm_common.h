// Scheduling pieces shared by the grouped expert GEMMs (bf16 and FP8).
//
// A launch covers a list of groups: routed expert g < n_r owns the sorted rows
// [offset[g], offset[g+1]); groups n_r.. are the shared experts (all T tokens). Each
// group is cut into row blocks of at most RB rows (the kernel's tile height) -- a group
// of r rows into ceil(r/RB) blocks of equal size, so the blocks of one expert take the
// same time -- and each block into output-column tiles. The tile list is built on the device
// from expert_offset, so no host synchronisation is needed, and it is walked by gangs of
// workgroups that run neighbouring tiles at the same time (see for_each_tile).
#pragma once

#include "device.h"
#include "launch.h"

namespace moe {
namespace gemm {

constexpr int kThreads = 512;  // 8 waves: two groups of 4, one wave of each group per SIMD
constexpr int BM = kTileRows;  // rows per tile (at most) of the FP8 kernel and the bf16 down-projection
constexpr int BNB = 256;       // B rows (weight rows) per tile
constexpr int kRowBytes = 128; // bytes per tile row per K-step (64 bf16 or 128 fp8)
constexpr int kMaxGroups = 256 + 8;

struct Tile {
  int group;  // routed expert, or n_r + shared index
  int m0;     // first row of the tile within the group
  int n0;     // first output column
  int rows;   // valid rows in this tile
};

// Tile list, by position: first the shared groups, then the routed experts with an even
// number of row blocks, then those with an odd number, so that with 16 column tiles per
// block and 32-tile gang items an expert of two blocks fills exactly one item. The shared
// groups' tiles are all of full height and come first; the routed tiles, whose heights
// vary, fill the tail of the launch, where short tiles even out the finish. In the gate/up
// launch (SORT) the experts of each routed pass go by row count, most rows first (ties:
// lower expert id first). A gang item then holds experts of about the same height, so its
// members' tiles take about the same time and no member of the gang lags behind the
// others, and the shortest tiles come last. A CPU model of the launch (tile times from
// the measured per-step cost, the gang protocol run as written, the V3-prefill expert
// loads) gave 94% of the ideal finish with the experts in id order and 97% in this
// order. The down-projection keeps id order: its items straddle experts (28 column tiles
// per block at d = 7168), and in id order the experts that run side by side are
// neighbours in H and in y_routed; sorted, its launch measured 2% slower.
// Routed groups list their tiles column-major (the row blocks of one column tile are
// neighbours: they read the same weights). A shared group is a dense GEMM over all tokens
// (many row blocks), so its tiles go in blocks of kSharedBR row blocks x kSharedBC column
// tiles (one 32-tile gang item): within a gang's item each weight tile is read by 4 CUs and
// each row block by 8, through the XCD's L2, where a row-major order re-read the shared
// expert's weights once per row block. Built per workgroup in LDS.
constexpr int kSharedBR = 4, kSharedBC = 8;  // shared groups: tiles in blocks of 4 row blocks x 8 columns

struct TileMap {
  int cum[kMaxGroups + 1];  // first tile index of the group at each position
  int grp[kMaxGroups];      // group at each position
  int mt[kMaxGroups];       // row blocks of each group
  int rpb[kMaxGroups];      // rows per block of each group
  int rows[kMaxGroups];     // rows of each routed expert (the sort key)
  int ord[kMaxGroups];      // routed experts in list order (SORT: most rows first, ties: lower id first)
  int ng;                   // positions (groups with rows)
  int total;
};

template <int RB = BM, bool SORT = true>  // rows per block at most; routed experts by row count
__device__ inline void build_tile_map(TileMap& tm, const int32_t* offset, int n_r, int n_groups_shared,
                                      int64_t T, int ntn) {
  const int ng = n_r + n_groups_shared;
  for (int g = threadIdx.x; g < ng; g += kThreads) {
    const int64_t rows = g < n_r ? (offset[g + 1] - offset[g]) : T;
    const int64_t mt0 = (rows + RB - 1) / RB;
    const int64_t rpb = mt0 > 0 ? (rows + mt0 - 1) / mt0 : 0;  // <= RB
    tm.rpb[g] = static_cast<int>(rpb);
    tm.mt[g] = rpb > 0 ? static_cast<int>((rows + rpb - 1) / rpb) : 0;  // no empty last block
    if (g < n_r) tm.rows[g] = static_cast<int>(rows);  // int32 offsets: fits
  }
  __syncthreads();
  // position of each routed expert in the order: the experts before it have more rows, or
  // as many and a lower id (a total order, so the positions are a permutation); without
  // SORT, id order
  for (int g = threadIdx.x; g < n_r; g += kThreads) {
    int pos = g;
    if constexpr (SORT) {
      const int rg = tm.rows[g];
      pos = 0;
      for (int h = 0; h < n_r; ++h) {
        const int rh = tm.rows[h];
        pos += (rh > rg || (rh == rg && h < g)) ? 1 : 0;
      }
    }
    tm.ord[pos] = g;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0, pos = 0;
    for (int pass = 0; pass < 3; ++pass) {
      const int lo = pass == 0 ? n_r : 0, hi = pass == 0 ? ng : n_r;
      for (int i = lo; i < hi; ++i) {
        const int g = pass == 0 ? i : tm.ord[i];
        const int mt = tm.mt[g];
        if (mt == 0 || (pass > 0 && (mt & 1) != pass - 1)) continue;
        tm.grp[pos] = g;
        tm.cum[pos] = acc;
        acc += mt * ntn;
        ++pos;
      }
    }
    tm.cum[pos] = acc;
    tm.ng = pos;
    tm.total = acc;
  }
  __syncthreads();
}

// Tile L of the list. rows_of(g) gives the rows of group g.
template <class RowsOf>
__device__ __forceinline__ Tile tile_at(const TileMap& tm, int L, int n_r, int bn_out, int ntn,
                                        RowsOf&& rows_of) {
  int lo = 0, hi = tm.ng - 1;  // last position with cum[pos] <= L
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (tm.cum[mid] <= L) lo = mid; else hi = mid - 1;
  }
  Tile t;
  t.group = tm.grp[lo];
  const int local = L - tm.cum[lo];
  int m, n;
  if (t.group < n_r) {
    const int mt = tm.mt[t.group];
    n = local / mt;
    m = local - n * mt;
  } else {
    // row groups of kSharedBR row blocks (the last may be shorter); within one, column
    // groups of kSharedBC tiles (the last may be narrower); row-major inside a block
    const int mt = tm.mt[t.group];
    const int rg = local / (kSharedBR * ntn);
    const int rem = local - rg * kSharedBR * ntn;
    const int br = mt - rg * kSharedBR < kSharedBR ? mt - rg * kSharedBR : kSharedBR;
    const int cg = rem / (br * kSharedBC);
    const int rem2 = rem - cg * br * kSharedBC;
    const int bc = ntn - cg * kSharedBC < kSharedBC ? ntn - cg * kSharedBC : kSharedBC;
    m = rg * kSharedBR + rem2 / bc;
    n = cg * kSharedBC + rem2 % bc;
  }
  const int rpb = tm.rpb[t.group];
  t.n0 = n * bn_out;
  t.m0 = m * rpb;
  const int64_t left = rows_of(t.group) - t.m0;
  t.rows = static_cast<int>(left < rpb ? left : rpb);
  return t;
}

// The reciprocal b_offset takes for segments of kseg_steps K-steps.
__host__ __device__ inline uint32_t kseg_recip(int kseg_steps) {
  return static_cast<uint32_t>(((1ull << 31) + kseg_steps - 1) / kseg_steps);
}

// Tile claiming by gangs. Workgroup b is member b / 8 of gang b % 8; workgroups are
// dispatched round-robin over the 8 XCDs, so a gang's members share one XCD and its L2.
// A gang takes items of G = gridDim.x / 8 consecutive tiles and member i computes tile i
// of the item, so the column tiles of a row block (same rows) and the row blocks of a
// column tile (same weights) run side by side and their common operand comes from HBM
// once. Items are handed out dynamically from one counter. The k-th item of a gang is
// published in slot k of the gang's row of slots: the first member to reach step k
// claims it (slot 0 -> -1 -> item + 1), the others read the slot. A member only waits
// for one that has passed the compare-and-swap and is two atomics from publishing, so
// every wait ends. The claims decide which workgroup computes a tile, never what it
// computes.
// sched: [0] the item counter, then kGangs rows of slot_stride slots, all zeroed before
// the launch; slot_stride > ceil(total / G).
template <class F>
__device__ __forceinline__ void for_each_tile(int total, int* sched, int slot_stride, F&& body) {
  __shared__ int claim;
  const int G = static_cast<int>(gridDim.x) / kGangs;
  const int gang = static_cast<int>(blockIdx.x) % kGangs, rank = static_cast<int>(blockIdx.x) / kGangs;
  if (rank >= G) return;  // a grid that is not a multiple of 8 leaves its last workgroups idle
  const int n_items = (total + G - 1) / G;
  int* slot = sched + 1 + static_cast<int64_t>(gang) * slot_stride;
  for (int k = 0; k < slot_stride; ++k) {
    if (threadIdx.x == 0) {
      int v = 0;
      if (__hip_atomic_compare_exchange_strong(slot + k, &v, -1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        v = atomicAdd(sched, 1) + 1;
        __hip_atomic_store(slot + k, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        while (v == -1) {
          __builtin_amdgcn_s_sleep(2);
          v = __hip_atomic_load(slot + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      claim = v - 1;
    }
    __syncthreads();
    const int item = claim;
    __syncthreads();
    if (item >= n_items) break;
    const int L = item * G + rank;
    if (L < total) body(L);
  }
}

// LDS byte offset of 16-byte chunk c (0..7) of row r in a [rows][128 B] stage. The
// chunk index is XORed with (r/2)%8, which spreads the 16 rows a ds_read_b128 serves at
// once over all 64 banks (no conflicts, checked with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4); }

// Element offset of K-step kt within a B row. For the shared down-projection the K
// range runs over the shared experts' segments (seg selects the expert, seg_stride is
// its distance); elsewhere kseg_steps == nk, so seg is 0. The quotient is
// floor(2 kt * kseg_inv / 2^32) with the precomputed kseg_inv = ceil(2^31 / kseg_steps)
// (kseg_recip), exact while kt * kseg_steps < 2^31, and defined for kseg_steps = 1.
__device__ __forceinline__ int64_t b_offset(int kt, int kseg_steps, uint32_t kseg_inv, int64_t seg_stride,
                                            int step_elems) {
  const int seg = static_cast<int>(__umulhi(2u * static_cast<uint32_t>(kt), kseg_inv));
  return static_cast<int64_t>(seg) * seg_stride + static_cast<int64_t>(kt - seg * kseg_steps) * step_elems;
}

}  // namespace gemm
}  // namespace moe

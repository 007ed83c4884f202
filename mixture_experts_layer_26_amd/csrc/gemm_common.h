// Scheduling pieces shared by the grouped expert GEMMs (bf16 and FP8).
//
// A launch covers a list of groups: routed expert g < n_r owns the sorted rows
// [offset[g], offset[g+1]); groups n_r.. are the shared experts (all T tokens). Each
// group is cut into tiles of BM rows x one output-column block; the tile list is built
// on the device from expert_offset, so no host synchronisation is needed, and tiles
// are claimed per XCD (see for_each_tile).
#pragma once

#include "device.h"

namespace moe {
namespace gemm {

constexpr int kThreads = 512;  // 8 waves: two groups of 4, one wave of each group per SIMD
constexpr int BM = 256;        // rows per tile
constexpr int BNB = 256;       // B rows (weight rows) per tile
constexpr int kRowBytes = 128; // bytes per tile row per K-step (64 bf16 or 128 fp8)
constexpr int kStageBytes = BM * kRowBytes;  // one operand's LDS stage (32 KB)
constexpr int kMaxGroups = 256 + 8;

struct Tile {
  int group;  // routed expert, or n_r + shared index
  int m0;     // first row of the tile within the group
  int n0;     // first output column
  int rows;   // valid rows in this tile
};

// Tile list: routed groups first (expert-major, then output-column tile, then row
// tile), then the shared groups. Built per workgroup in LDS.
struct TileMap {
  int cum[kMaxGroups + 1];  // first tile index of each group
  int mt[kMaxGroups];       // row tiles per group
  int total;
};

__device__ inline void build_tile_map(TileMap& tm, const int32_t* offset, int n_r, int n_groups_shared,
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

__device__ __forceinline__ Tile tile_at(const TileMap& tm, int L, int ng, const int32_t* offset, int n_r,
                                        int64_t T, int bn_out) {
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

// Tile claiming. The tile list is cut into 8 contiguous chunks, one per XCD. A
// workgroup claims tiles of its own XCD's chunk (XCD id read from HW_REG_XCC_ID) from
// that chunk's counter, so the tiles in flight on an XCD are neighbours in the list (one
// expert's column and row tiles), whose gathered rows and weights its L2 then serves
// to several CUs. When its chunk runs out it helps the other chunks. The counters only
// decide which CU computes a tile, never what a tile computes. counter: 8 zeroed ints.
template <class F>
__device__ __forceinline__ void for_each_tile(int total, int* counter, F&& body) {
  __shared__ int claim;
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  xcc &= 7;
  const int chunk = (total + 7) / 8;
  int o = 0;
  while (o < 8) {
    const int x = (static_cast<int>(xcc) + o) & 7;
    if (threadIdx.x == 0) claim = atomicAdd(counter + x, 1);
    __syncthreads();
    const int local = claim;
    __syncthreads();
    const int L = x * chunk + local;
    if (local >= chunk || L >= total) {
      ++o;
      continue;
    }
    body(L);
  }
}

// LDS byte offset of 16-byte chunk c (0..7) of row r in a [rows][128 B] stage. The
// chunk index is XORed with (r/2)%8, which spreads the 16 rows a ds_read_b128 serves at
// once over all 64 banks (no conflicts, checked with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int swz(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4); }

// Element offset of K-step kt within a B row. For the shared down-projection the K
// range runs over the shared experts' segments (seg selects the expert, seg_stride is
// its distance); elsewhere kseg_steps == nk, so seg is 0. The quotient uses a
// precomputed reciprocal kseg_inv = ceil(2^32 / kseg_steps), exact below 2^16.
__device__ __forceinline__ int64_t b_offset(int kt, int kseg_steps, uint32_t kseg_inv, int64_t seg_stride,
                                            int step_elems) {
  const int seg = static_cast<int>(__umulhi(static_cast<uint32_t>(kt), kseg_inv));
  return static_cast<int64_t>(seg) * seg_stride + static_cast<int64_t>(kt - seg * kseg_steps) * step_elems;
}

}  // namespace gemm
}  // namespace moe

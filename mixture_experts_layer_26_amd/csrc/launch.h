// Internal launchers of the gfx950 kernels (host side). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Arguments of one grouped GEMM launch (phase 1 = gated gate/up, phase 2 = down).
// Group g < n_r is routed expert g with rows [offset[g], offset[g+1]); groups n_r.. are
// shared (phase 1: one per shared expert, rows = all T tokens; phase 2: one group whose
// K runs over all shared experts' H columns, k_segments = n_shared).
struct GemmArgs {
  const uint16_t* a_routed;  // phase 1: u [T, d]; phase 2: H routed [P, d_ff] (FP8: byte codes)
  const uint16_t* a_shared;  // phase 1: u; phase 2: H shared [T, n_s * d_ff]
  int64_t lda_routed, lda_shared;
  const int32_t* gather;     // phase 1: sorted_token; phase 2: nullptr
  const uint16_t* b1_routed; // phase 1: W1 [n_r, d_ff, d]; phase 2: W2 [n_r, d, d_ff]
  const uint16_t* b3_routed; // phase 1: W3; phase 2: unused
  const uint16_t* b1_shared;
  const uint16_t* b3_shared;
  int64_t b_expert_stride;   // elements per expert in the weight arrays
  int64_t ldb;               // row length of B (the K extent of one expert)
  int b_tiled;               // weights in the tiled layout (see moe_pack_weights)
  void* out_routed;          // phase 1: H routed (bf16); phase 2: y_routed (bf16)
  void* out_shared;          // phase 1: H shared (bf16); phase 2: y_shared (fp32)
  int64_t ldo_routed, ldo_shared;
  const int32_t* offset;     // expert_offset [n_r + 1]
  int n_r;
  int n_shared_groups;       // phase 1: n_s; phase 2: 1 if n_s > 0 else 0
  int64_t T;
  int N;                     // output columns per group
  int K;                     // K of one expert
  int k_segments;            // phase 2 shared: n_s
  int* sched;                // zeroed gang-scheduling state: 1 + kGangs * slot_stride ints
  int slot_stride;           // slots per gang (> tiles / (grid / kGangs))
  // bf16 phase 1 only, optional (nullptr: not stored): the pre-activations a = x W1^T and
  // v = x W3^T in fp32, laid out as H (routed [P][ldo_routed], shared [T][ldo_shared] at
  // column s * N); the backward reads them
  float* pre_gate_routed;
  float* pre_up_routed;
  float* pre_gate_shared;
  float* pre_up_shared;
};

// Tile scheduling of the grouped GEMMs: workgroup b belongs to gang b % kGangs (one
// gang per XCD). Ints of scheduling state one launch of at most max_tiles tiles needs on
// a grid of `grid` workgroups, and the slot stride that goes with it.
constexpr int kGangs = 8;
constexpr int kTileRows = 256;  // row-block size of the tile-count bound (no kernel has more blocks)
inline int64_t sched_slot_stride(int64_t max_tiles, int grid) {
  const int64_t G = grid / kGangs > 0 ? grid / kGangs : 1;
  return (max_tiles + G - 1) / G + 2;
}
inline int64_t sched_ints(int64_t max_tiles, int grid) { return 1 + kGangs * sched_slot_stride(max_tiles, grid); }

hipError_t launch_zero_i32(int* p, int n, hipStream_t stream);

// The fixed scratch of moe_grouped_ffn_noalloc (scratch.hip): its size, and its device
// address on the current device (looked up once per device, then cached).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// FP8 grouped GEMM: the codes travel in the GemmArgs pointers (as bytes), the fp32
// scales here. A-row scales: one per row per 128-wide K block, stored K-block-major
// (the scale of row r in K block kb at [kb * ld + r]) so that one K-step's scales of a
// tile's rows are contiguous; routed rows are indexed by sorted row, shared rows by
// token. B scales: one per 128 x 128 block of a weight matrix [E, N/128, K/128].
struct Fp8Args {
  GemmArgs g;
  const float* sa_routed;   // [K/128][ldsa_routed] by sorted row
  const float* sa_shared;   // [K/128][ldsa_shared] by token
  int64_t ldsa_routed, ldsa_shared;
  const float* sb1_routed;  // phase 1: s1; phase 2: s2
  const float* sb3_routed;  // phase 1: s3
  const float* sb1_shared;
  const float* sb3_shared;
  int64_t sb_expert_stride; // scales per expert: (N/128) * (K/128)
  int kblocks;              // K/128 of one expert (scale row length)
  float* os_routed;         // phase 1: H scales, K-block-major [d_ff/128][ldos_routed] by sorted row
  float* os_shared;         // phase 1: H scales, K-block-major [n_s * d_ff/128][ldos_shared] by token
  int64_t ldos_routed, ldos_shared;
};

size_t ffn_fp8_lds_bytes();
hipError_t launch_grouped_gemm_fp8(const Fp8Args& args, bool gated, int grid, hipStream_t stream);

// Router (bf16): the K range is split into chunks of whole 64-wide steps; the partial
// logits of every chunk, [chunks][T][n_r] fp32, live in the caller's workspace.
struct RouteChunks {
  int chunks;
  int steps_per_chunk;
};
RouteChunks route_chunks(int64_t T, int d);
size_t route_workspace_bytes(int64_t T, int d, int n_r);
// score: 0 sigmoid with bias, 1 softmax over the top-K logits (bias unused, may be null)
hipError_t launch_route(int act, int score, const void* u, const void* e, const float* bias, int64_t T,
                        int d, int n_r, int K, int32_t* idx, float* gate, float* part, hipStream_t stream);

int dispatch_blocks(int64_t T);
hipError_t launch_dispatch(const int32_t* idx, int64_t T, int K, int n_r, int32_t* hist,
                           int32_t* count, int32_t* offset, int32_t* sorted_token,
                           int32_t* pair_row, hipStream_t stream);

// bf16 grouped GEMM. Batches of at most kSmallBatchRows tokens (every group then fits one
// row block of that height) run on 128-row tiles with a three-stage ring, larger ones on
// 320-row tiles with two stages.
constexpr int kSmallBatchRows = 128;
size_t ffn_bf16_lds_bytes();
hipError_t launch_grouped_gemm_bf16(const GemmArgs& args, bool gated, int grid, hipStream_t stream);

hipError_t launch_ffn_f32(const float* u, const int32_t* offset, const int32_t* sorted_token,
                          const float* w1r, const float* w3r, const float* w2r, const float* w1s,
                          const float* w3s, const float* w2s, int64_t T, int d, int d_ff, int n_r,
                          int K, int n_s, float* h, float* y_routed, float* y_shared,
                          hipStream_t stream);

hipError_t launch_combine(int act, const void* u, const void* y_routed, const float* y_shared,
                          const int32_t* pair_row, const float* gate, void* out, int64_t T, int d,
                          int K, hipStream_t stream);

hipError_t launch_bias_update(const int32_t* count, int64_t T, int n_r, int K, float gamma,
                              float* bias, hipStream_t stream);

// Tiled weight layout: [E, N, K] row-major -> [E][N/R][K/KS][R][KS], KS elements = 128
// bytes (64 bf16, 128 fp8), R = 128 (gate/up) or 256 (down).
hipError_t launch_pack_weights(const void* src, void* dst, int esz, int64_t E, int64_t N, int64_t K, int R,
                               hipStream_t stream);

// K-block-major A-row scales of the FP8 phase 1 from the 1x128 tile scales s [T][nkb] of
// u: out[kb * (P + T) + j] is the scale of sorted row j (token sorted_token[j]) for
// j < P and of token j - P for P <= j < P + T.
hipError_t launch_scale_columns(const float* s, int nkb, const int32_t* sorted_token, int64_t P, int64_t T,
                                float* out, hipStream_t stream);
hipError_t launch_quantize_fp8(const void* x, int xt, int64_t rows, int64_t cols, int tile_r,
                               int tile_c, uint8_t* q, float* scale, hipStream_t stream);

// ---------------------------------------------------------------------------- backward
// Grouped SwiGLU backward (bf16, row-major or tiled weights; d a multiple of 256, d_ff of 128).
struct BwdArgs {
  const uint16_t* u;             // [T, d]
  const uint16_t* dout;          // [T, d]: the shared experts' output gradient
  const uint16_t* dy_routed;     // [P, d]: the routed rows' output gradient (sorted rows)
  const int32_t* offset;         // expert_offset [n_r + 1]
  const int32_t* sorted_token;   // [P]
  const uint16_t *w1r, *w3r, *w2r;  // routed weights [n_r, d_ff, d], [n_r, d, d_ff]
  const uint16_t *w1s, *w3s, *w2s;  // shared weights (n_s experts)
  uint16_t *h_r, *da_r, *dv_r;   // workspace [P, d_ff]: h, da, dv of the routed rows
  uint16_t *h_s, *da_s, *dv_s;   // workspace [T, n_s * d_ff]
  float *a_r, *v_r;              // workspace [P, d_ff]: a = X W1^T, v = X W3^T (fp32)
  float *a_s, *v_s;              // workspace [T, n_s * d_ff]
  uint16_t* xs;                  // workspace [P, d]: u of the sorted rows
  uint16_t* zero;                // workspace, 256 bytes cleared by the call
  uint16_t* dx_r;                // out [P, d] bf16
  float* dx_s;                   // out [T, d] fp32, sum over the shared experts
  uint16_t *dw1r, *dw3r, *dw2r;  // out, routed weight gradients (bf16, weight layouts)
  uint16_t *dw1s, *dw3s, *dw2s;  // out, shared
  int64_t T;
  int K, d, F, n_r, n_s;
  int tiled;                     // weights and weight gradients in the tiled layout (else row-major)
};
hipError_t launch_ffn_backward(const BwdArgs& args, hipStream_t stream);

hipError_t launch_combine_backward(const void* dout, const void* y_routed, const int32_t* pair_row,
                                   const float* gate, void* dy_routed, float* dgate, int64_t T, int d, int K,
                                   hipStream_t stream);
// score: 0 sigmoid, 1 softmax. dz_sorted: workspace [P] fp32.
hipError_t launch_route_backward(int score, const void* u, const void* e, const int32_t* idx, const float* gate,
                                 const float* dgate, const int32_t* offset, const int32_t* sorted_token,
                                 const int32_t* pair_row, const void* dout, const void* dx_routed,
                                 const float* dx_shared, void* du, void* de, float* dz, float* dz_sorted,
                                 int64_t T, int d, int n_r, int K, hipStream_t stream);

// ---------------------------------------------------------------------------- MOE_DEBUG
// One check: every p[i] of n entries in [lo, hi), or (offsets) p[0] == 0, p[n] == hi and
// p non-decreasing over n + 1 entries.
struct IndexCheck {
  const int32_t* p;
  int64_t n;
  int32_t lo, hi;
  bool offsets;
};
// Runs the checks on `stream`, waits for them, and sets *bad if any failed.
hipError_t debug_check_indices(const IndexCheck* checks, int count, hipStream_t stream, bool* bad);

}  // namespace moe

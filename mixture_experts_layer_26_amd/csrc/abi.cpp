// C ABI of the MoE layer (include/moe.h): host-side validation, workspace sizing and
// kernel launches. Validation runs before any HIP call, so a rejected call touches
// neither the device nor the caller's memory.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>

#include "launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool valid_shape(const moe_shape* s) {
  if (!s) return false;
  if (s->T < 0 || s->T > (1LL << 26)) return false;
  if (s->n_routed < 1 || s->n_routed > 256) return false;
  if (s->top_k < 1 || s->top_k > 16 || s->top_k > s->n_routed) return false;
  if (s->n_shared < 0 || s->n_shared > 8) return false;
  if (s->d < 64 || s->d % 64 != 0 || s->d_ff < 64 || s->d_ff % 64 != 0) return false;
  if (s->T * s->top_k >= (1LL << 31)) return false;
  const bool f32 = s->act == MOE_F32 && s->ffn == MOE_F32;
  const bool bf16 = s->act == MOE_BF16 && s->ffn == MOE_BF16;
  const bool fp8 = s->act == MOE_BF16 && s->ffn == MOE_FP8_E4M3;
  if (s->score != MOE_SCORE_SIGMOID && s->score != MOE_SCORE_SOFTMAX) return false;
  return f32 || bf16 || fp8;
}

// Arrays whose size scales with T may be NULL for an empty batch (T = 0).
bool ok_t(const moe_shape* s, const void* p) { return p != nullptr || s->T == 0; }

// Clears `bytes` (a multiple of 4) with a fill kernel, in pieces of at most 2^30 words.
hipError_t zero_bytes(void* p, size_t bytes, hipStream_t stream) {
  int32_t* q = static_cast<int32_t*>(p);
  size_t words = bytes / 4;
  while (words > 0) {
    const size_t n = words < (size_t(1) << 30) ? words : (size_t(1) << 30);
    const hipError_t e = moe::launch_zero_i32(q, static_cast<int>(n), stream);
    if (e != hipSuccess) return e;
    q += n;
    words -= n;
  }
  return hipSuccess;
}

// shapes the MFMA kernels tile exactly: output columns of the gated phase in 128s, of
// the down phase in 256s
bool tiled_shape(const moe_shape* s) {
  if (s->ffn == MOE_F32) return true;
  return s->d % 256 == 0 && s->d_ff % 128 == 0;
}

// The bf16 and FP8 grouped GEMMs address each loaded row with a wave-uniform 64-bit base
// and a 32-bit byte offset. The gathered rows of u (bf16: u itself; FP8: its 1x128 codes)
// are offsets from the operand's start, so it must hold fewer than 2^32 bytes (bf16: T*d
// below 2^31; FP8: below 2^32); every other offset stays within one tile's rows (at most
// 320 rows of d, d_ff or N_s * d_ff elements, or 256 weight rows), which row lengths below
// 2^22 elements keep under 2^32 bytes.
bool gemm_offsets_fit(const moe_shape* s) {
  const int64_t row_lim = 1LL << 22;
  const int64_t elem = s->ffn == MOE_FP8_E4M3 ? 1 : 2;
  return s->T * s->d * elem < (1LL << 32) && s->d < row_lim && s->d_ff < row_lim &&
         static_cast<int64_t>(s->n_shared) * s->d_ff < row_lim;
}

size_t act_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }

hipStream_t as_stream(void* p) { return static_cast<hipStream_t>(p); }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// MOE_DEBUG=1 (read at every call): index arrays from earlier calls are checked on the
// device before use; a bad one gives MOE_ERR_INVALID_ARG and nothing else is launched.
bool debug_on() {
  const char* e = std::getenv("MOE_DEBUG");
  return e != nullptr && e[0] == '1';
}

moe_status debug_check(std::initializer_list<moe::IndexCheck> checks, void* stream) {
  if (!debug_on()) return MOE_OK;
  bool bad = false;
  const hipError_t e = moe::debug_check_indices(checks.begin(), static_cast<int>(checks.size()),
                                                as_stream(stream), &bad);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return bad ? MOE_ERR_INVALID_ARG : MOE_OK;
}

moe::IndexCheck range(const int32_t* p, int64_t n, int32_t lo, int32_t hi) { return {p, n, lo, hi, false}; }
moe::IndexCheck offsets(const int32_t* p, int n, int32_t total) { return {p, n, 0, total, true}; }

int grid_for_device() {
  // one persistent workgroup per CU; cached per device
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 256;
    cus[dev] = n / 8 * 8;
  }
  return cus[dev];
}

// Upper bound on the tiles of a grouped GEMM launch (phase 1: gate/up, 128 output
// columns per tile; phase 2: down, 256): an expert of r rows has ceil(r / 256) row
// blocks, at most r / 256 + 1, and each shared group ceil(T / 256). Kernels with taller
// tiles (the 320-row tiles of the bf16 GEMMs and of the FP8 one) have no more blocks than
// that, and the bf16 GEMMs' 128-row tiles are used only for batches of at most 128 tokens,
// where every group is a single block.
int64_t ffn_max_tiles(const moe_shape* s, int phase) {
  const int64_t bm = moe::kTileRows;
  const int64_t P = s->T * s->top_k;
  const int64_t routed_blocks = P / bm + s->n_routed + 1;
  const int64_t tb = (s->T + bm - 1) / bm;
  if (phase == 1) return (routed_blocks + s->n_shared * tb) * (s->d_ff / 128);
  return (routed_blocks + (s->n_shared > 0 ? tb : 0)) * (s->d / 256);
}

// Persistent grid of the grouped GEMMs: one workgroup per CU, at least 64 (8 per gang),
// which the scheduling state in the workspace is sized for.
constexpr int kMinGemmGrid = 64;
int gemm_grid() {
  const int g = grid_for_device();
  return g < kMinGemmGrid ? kMinGemmGrid : g;
}

struct SchedState {  // the two launches' regions of the scheduling state
  int32_t* s1;
  int32_t* s2;
  int stride1, stride2;
};

struct FfnWorkspace {
  size_t sched, h_routed, h_shared, q_u, s_u, s_cols, s_h_routed, s_h_shared, total;
};

FfnWorkspace ffn_workspace(const moe_shape* s) {
  FfnWorkspace w{};
  const int64_t P = s->T * s->top_k;
  const int64_t Hs = s->T * static_cast<int64_t>(s->n_shared) * s->d_ff;
  size_t off = 0;
  w.sched = off;  // gang-scheduling state of the two GEMM launches, sized for the smallest grid
  off = align_up(off + (moe::sched_ints(ffn_max_tiles(s, 1), kMinGemmGrid) +
                        moe::sched_ints(ffn_max_tiles(s, 2), kMinGemmGrid)) * sizeof(int32_t));
  if (s->ffn == MOE_FP8_E4M3) {
    w.q_u = off;
    off = align_up(off + static_cast<size_t>(s->T) * s->d);
    w.s_u = off;
    off = align_up(off + static_cast<size_t>(s->T) * (s->d / 128) * 4);
    w.s_cols = off;  // the same scales K-block-major, routed rows in sorted order then the tokens
    off = align_up(off + static_cast<size_t>(P + s->T) * (s->d / 128) * 4);
    w.h_routed = off;
    off = align_up(off + static_cast<size_t>(P) * s->d_ff);
    w.s_h_routed = off;
    off = align_up(off + static_cast<size_t>(P) * (s->d_ff / 128) * 4);
    w.h_shared = off;
    off = align_up(off + static_cast<size_t>(Hs));
    w.s_h_shared = off;
    off = align_up(off + static_cast<size_t>(Hs / 128) * 4);
  } else {
    const size_t e = act_bytes(s->ffn);
    w.h_routed = off;
    off = align_up(off + static_cast<size_t>(P) * s->d_ff * e);
    w.h_shared = off;
    off = align_up(off + static_cast<size_t>(Hs) * e);
  }
  w.total = off;
  return w;
}

// Backward: shapes it runs (bf16, either weight layout, d % 256 == 0, d_ff % 128 == 0) and its
// workspaces.
bool backward_shape(const moe_shape* s) {
  return s->act == MOE_BF16 && s->ffn == MOE_BF16 && s->d % 256 == 0 && s->d_ff % 128 == 0 && s->top_k <= 16;
}

struct BwdWorkspace {
  size_t sched, zero, xs, h_r, da_r, dv_r, h_s, da_s, dv_s, a_r, v_r, a_s, v_s, total;
};

BwdWorkspace bwd_workspace(const moe_shape* s) {
  BwdWorkspace w{};
  const size_t pr = static_cast<size_t>(s->T) * s->top_k * s->d_ff * 2;
  const size_t ps = static_cast<size_t>(s->T) * s->n_shared * s->d_ff * 2;
  size_t off = 0;
  w.sched = off;  // gang-scheduling state of the gate/up launch, sized for the smallest grid
  off = align_up(off + moe::sched_ints(ffn_max_tiles(s, 1), kMinGemmGrid) * sizeof(int32_t));
  w.zero = off;
  off = align_up(off + 256);
  w.xs = off;
  off = align_up(off + static_cast<size_t>(s->T) * s->top_k * s->d * 2);
  w.h_r = off;
  off = align_up(off + pr);
  w.da_r = off;
  off = align_up(off + pr);
  w.dv_r = off;
  off = align_up(off + pr);
  w.h_s = off;
  off = align_up(off + ps);
  w.da_s = off;
  off = align_up(off + ps);
  w.dv_s = off;
  off = align_up(off + ps);
  // a and v in fp32 (twice the bf16 sizes), from the gate/up launch to the dh launch
  w.a_r = off;
  off = align_up(off + 2 * pr);
  w.v_r = off;
  off = align_up(off + 2 * pr);
  w.a_s = off;
  off = align_up(off + 2 * ps);
  w.v_s = off;
  off = align_up(off + 2 * ps);
  w.total = off;
  return w;
}


// The FP8 expert FFN: u quantised per 1x128 tile into the workspace, then the two
// FP8 grouped GEMMs (phase 1 also quantises H per 1x128).
moe_status grouped_ffn_fp8(const moe_shape* s, const void* u, const int32_t* expert_offset,
                           const int32_t* sorted_token, const moe_expert_set* routed,
                           const moe_expert_set* shared, void* y_routed, float* y_shared,
                           unsigned char* wsb, const FfnWorkspace& w, const SchedState& sc, int grid,
                           int b_tiled, hipStream_t st) {
  uint8_t* q_u = wsb + w.q_u;
  float* s_u = reinterpret_cast<float*>(wsb + w.s_u);
  float* s_cols = reinterpret_cast<float*>(wsb + w.s_cols);
  uint8_t* h_r = wsb + w.h_routed;
  uint8_t* h_s = wsb + w.h_shared;
  float* sh_r = reinterpret_cast<float*>(wsb + w.s_h_routed);
  float* sh_s = reinterpret_cast<float*>(wsb + w.s_h_shared);
  const int d = s->d, I = s->d_ff, ns = s->n_shared;
  const int64_t P = s->T * s->top_k;
  if (moe::launch_quantize_fp8(u, MOE_BF16, s->T, d, 1, 128, q_u, s_u, st) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_scale_columns(s_u, d / 128, sorted_token, P, s->T, s_cols, st) != hipSuccess) return MOE_ERR_HIP;
  auto b = [](const void* p) { return static_cast<const uint16_t*>(p); };

  moe::Fp8Args f1{};
  f1.g.a_routed = f1.g.a_shared = reinterpret_cast<const uint16_t*>(q_u);
  f1.g.lda_routed = f1.g.lda_shared = d;
  f1.g.gather = sorted_token;
  f1.g.b1_routed = b(routed->w1);
  f1.g.b3_routed = b(routed->w3);
  f1.g.b1_shared = ns > 0 ? b(shared->w1) : nullptr;
  f1.g.b3_shared = ns > 0 ? b(shared->w3) : nullptr;
  f1.g.b_expert_stride = static_cast<int64_t>(I) * d;
  f1.g.ldb = d;
  f1.g.out_routed = h_r;
  f1.g.out_shared = h_s;
  f1.g.ldo_routed = I;
  f1.g.ldo_shared = static_cast<int64_t>(ns) * I;
  f1.g.offset = expert_offset;
  f1.g.n_r = s->n_routed;
  f1.g.n_shared_groups = ns;
  f1.g.T = s->T;
  f1.g.N = I;
  f1.g.K = d;
  f1.g.k_segments = 1;
  f1.g.sched = sc.s1;
  f1.g.b_tiled = b_tiled;
  f1.g.slot_stride = sc.stride1;
  f1.sa_routed = s_cols;
  f1.sa_shared = s_cols + P;
  f1.ldsa_routed = f1.ldsa_shared = P + s->T;
  f1.sb1_routed = routed->s1;
  f1.sb3_routed = routed->s3;
  f1.sb1_shared = ns > 0 ? shared->s1 : nullptr;
  f1.sb3_shared = ns > 0 ? shared->s3 : nullptr;
  f1.sb_expert_stride = static_cast<int64_t>(I / 128) * (d / 128);
  f1.kblocks = d / 128;
  f1.os_routed = sh_r;
  f1.os_shared = sh_s;
  f1.ldos_routed = P;
  f1.ldos_shared = s->T;
  if (moe::launch_grouped_gemm_fp8(f1, true, grid, st) != hipSuccess) return MOE_ERR_HIP;

  moe::Fp8Args f2{};
  f2.g.a_routed = reinterpret_cast<const uint16_t*>(h_r);
  f2.g.a_shared = reinterpret_cast<const uint16_t*>(h_s);
  f2.g.lda_routed = I;
  f2.g.lda_shared = static_cast<int64_t>(ns) * I;
  f2.g.gather = nullptr;
  f2.g.b1_routed = b(routed->w2);
  f2.g.b1_shared = ns > 0 ? b(shared->w2) : nullptr;
  f2.g.b_expert_stride = static_cast<int64_t>(d) * I;
  f2.g.ldb = I;
  f2.g.out_routed = y_routed;
  f2.g.out_shared = y_shared;
  f2.g.ldo_routed = d;
  f2.g.ldo_shared = d;
  f2.g.offset = expert_offset;
  f2.g.n_r = s->n_routed;
  f2.g.n_shared_groups = ns > 0 ? 1 : 0;
  f2.g.T = s->T;
  f2.g.N = d;
  f2.g.K = I;
  f2.g.k_segments = ns;
  f2.g.sched = sc.s2;
  f2.g.b_tiled = b_tiled;
  f2.g.slot_stride = sc.stride2;
  f2.sa_routed = sh_r;
  f2.ldsa_routed = P;
  f2.sa_shared = sh_s;
  f2.ldsa_shared = s->T;
  f2.sb1_routed = routed->s2;
  f2.sb1_shared = ns > 0 ? shared->s2 : nullptr;
  f2.sb_expert_stride = static_cast<int64_t>(d / 128) * (I / 128);
  f2.kblocks = I / 128;
  return from_hip(moe::launch_grouped_gemm_fp8(f2, false, grid, st));
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH_LIMIT:
      return "shape needs more scratch than moe_grouped_ffn_noalloc's fixed buffer holds "
             "(MOE_NOALLOC_SCRATCH_BYTES; use moe_grouped_ffn with a workspace)";
  }
  return "unknown status";
}

size_t moe_workspace_bytes(const moe_shape* s, int32_t call) {
  if (!valid_shape(s) || s->T == 0) return 0;  // an empty batch needs no workspace
  if (call == MOE_CALL_DISPATCH)
    return align_up(static_cast<size_t>(moe::dispatch_blocks(s->T)) * s->n_routed * sizeof(int32_t));
  if (call == MOE_CALL_GROUPED_FFN) return ffn_workspace(s).total;
  if (call == MOE_CALL_GROUPED_FFN_BACKWARD) return backward_shape(s) ? bwd_workspace(s).total : 0;
  if (call == MOE_CALL_ROUTE_BACKWARD)
    return backward_shape(s) ? align_up(static_cast<size_t>(s->T) * s->top_k * sizeof(float)) : 0;
  if (call == MOE_CALL_ROUTE)
    return s->act == MOE_BF16 ? align_up(moe::route_workspace_bytes(s->T, s->d, s->n_routed)) : 0;
  return 0;
}

moe_status moe_route(const moe_shape* s, const void* u, const void* centroids, const float* bias,
                     int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_shape(s) || !ok_t(s, u) || !centroids || !ok_t(s, topk_idx) || !ok_t(s, topk_gate))
    return MOE_ERR_INVALID_ARG;
  const bool softmax = s->score == MOE_SCORE_SOFTMAX;
  if (!bias && !softmax) return MOE_ERR_INVALID_ARG;
  if (s->T == 0) return MOE_OK;
  const size_t need = moe_workspace_bytes(s, MOE_CALL_ROUTE);
  if (need > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return from_hip(moe::launch_route(s->act == MOE_BF16 ? 1 : 0, softmax ? 1 : 0, u, centroids,
                                    softmax ? nullptr : bias, s->T, s->d, s->n_routed, s->top_k, topk_idx,
                                    topk_gate, static_cast<float*>(ws), as_stream(stream)));
}

moe_status moe_dispatch(const moe_shape* s, const int32_t* topk_idx, int32_t* expert_count,
                        int32_t* expert_offset, int32_t* sorted_token, int32_t* pair_row, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!valid_shape(s) || !ok_t(s, topk_idx) || !expert_count || !expert_offset || !ok_t(s, sorted_token) ||
      !ok_t(s, pair_row))
    return MOE_ERR_INVALID_ARG;
  if (s->T == 0) {  // no pairs: every count and offset is zero
    hipError_t e = zero_bytes(expert_count, sizeof(int32_t) * s->n_routed, as_stream(stream));
    if (e == hipSuccess) e = zero_bytes(expert_offset, sizeof(int32_t) * (s->n_routed + 1), as_stream(stream));
    return from_hip(e);
  }
  if (!ws || ws_bytes < moe_workspace_bytes(s, MOE_CALL_DISPATCH)) return MOE_ERR_WORKSPACE;
  const int64_t P = s->T * s->top_k;
  if (moe_status d = debug_check({range(topk_idx, P, 0, s->n_routed)}, stream)) return d;
  return from_hip(moe::launch_dispatch(topk_idx, s->T, s->top_k, s->n_routed,
                                       static_cast<int32_t*>(ws), expert_count, expert_offset,
                                       sorted_token, pair_row, as_stream(stream)));
}

}  // extern "C"

namespace {

// Host-side checks of moe_grouped_ffn's arguments other than the workspace.
moe_status grouped_ffn_check(const moe_shape* s, const void* u, const int32_t* expert_offset,
                             const int32_t* sorted_token, const moe_expert_set* routed,
                             const moe_expert_set* shared, const void* y_routed, const float* y_shared) {
  if (!valid_shape(s) || !ok_t(s, u) || !expert_offset || !ok_t(s, sorted_token) || !routed || !ok_t(s, y_routed))
    return MOE_ERR_INVALID_ARG;
  if (!routed->w1 || !routed->w3 || !routed->w2) return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0 && (!shared || !shared->w1 || !shared->w3 || !shared->w2 || !ok_t(s, y_shared)))
    return MOE_ERR_INVALID_ARG;
  const bool fp8 = s->ffn == MOE_FP8_E4M3;
  if (fp8 && (!routed->s1 || !routed->s3 || !routed->s2 ||
              (s->n_shared > 0 && (!shared->s1 || !shared->s3 || !shared->s2))))
    return MOE_ERR_INVALID_ARG;
  if (routed->layout != MOE_LAYOUT_ROWS && routed->layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0 && shared->layout != routed->layout) return MOE_ERR_INVALID_ARG;
  const int b_tiled = routed->layout == MOE_LAYOUT_TILED ? 1 : 0;
  if (b_tiled && s->ffn == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (!tiled_shape(s)) return MOE_ERR_UNSUPPORTED;
  if (s->ffn != MOE_F32 && !gemm_offsets_fit(s)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Arguments of the bf16 gate/up GEMM (phase 1): x gathered from u through sorted_token,
// H into h_r (routed rows, sorted order) and h_s (tokens, N_s * d_ff columns).
moe::GemmArgs gate_up_args(const moe_shape* s, const void* u, const int32_t* expert_offset,
                           const int32_t* sorted_token, const moe_expert_set* routed,
                           const moe_expert_set* shared, uint16_t* h_r, uint16_t* h_s, int b_tiled,
                           int32_t* sched, int slot_stride) {
  moe::GemmArgs g{};
  const uint16_t* ub = static_cast<const uint16_t*>(u);
  g.a_routed = ub;
  g.a_shared = ub;
  g.lda_routed = g.lda_shared = s->d;
  g.gather = sorted_token;
  g.b1_routed = static_cast<const uint16_t*>(routed->w1);
  g.b3_routed = static_cast<const uint16_t*>(routed->w3);
  g.b1_shared = s->n_shared > 0 ? static_cast<const uint16_t*>(shared->w1) : nullptr;
  g.b3_shared = s->n_shared > 0 ? static_cast<const uint16_t*>(shared->w3) : nullptr;
  g.b_expert_stride = static_cast<int64_t>(s->d_ff) * s->d;
  g.ldb = s->d;
  g.out_routed = h_r;
  g.out_shared = h_s;
  g.ldo_routed = s->d_ff;
  g.ldo_shared = static_cast<int64_t>(s->n_shared) * s->d_ff;
  g.offset = expert_offset;
  g.n_r = s->n_routed;
  g.n_shared_groups = s->n_shared;
  g.T = s->T;
  g.N = s->d_ff;
  g.K = s->d;
  g.k_segments = 1;
  g.sched = sched;
  g.b_tiled = b_tiled;
  g.slot_stride = slot_stride;
  return g;
}

// The grouped FFN on a checked shape with T > 0 and a workspace of at least
// ffn_workspace(s).total bytes.
moe_status grouped_ffn_run(const moe_shape* s, const void* u, const int32_t* expert_offset,
                           const int32_t* sorted_token, const moe_expert_set* routed,
                           const moe_expert_set* shared, void* y_routed, float* y_shared, void* ws,
                           void* stream) {
  const FfnWorkspace w = ffn_workspace(s);
  const bool fp8 = s->ffn == MOE_FP8_E4M3;
  const int b_tiled = routed->layout == MOE_LAYOUT_TILED ? 1 : 0;
  hipStream_t st = as_stream(stream);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  const int64_t P = s->T * s->top_k;
  if (moe_status d = debug_check({offsets(expert_offset, s->n_routed, static_cast<int32_t>(P)),
                                  range(sorted_token, P, 0, static_cast<int32_t>(s->T))},
                                 stream))
    return d;

  if (s->ffn == MOE_F32) {
    const moe_expert_set empty{};
    const moe_expert_set* sh = s->n_shared > 0 ? shared : &empty;
    return from_hip(moe::launch_ffn_f32(
        static_cast<const float*>(u), expert_offset, sorted_token,
        static_cast<const float*>(routed->w1), static_cast<const float*>(routed->w3),
        static_cast<const float*>(routed->w2), static_cast<const float*>(sh->w1),
        static_cast<const float*>(sh->w3), static_cast<const float*>(sh->w2), s->T, s->d, s->d_ff,
        s->n_routed, s->top_k, s->n_shared, reinterpret_cast<float*>(wsb + w.h_routed),
        static_cast<float*>(y_routed), y_shared, st));
  }
  const int grid = gemm_grid();
  const int64_t t1 = ffn_max_tiles(s, 1), t2 = ffn_max_tiles(s, 2);
  if (t1 > INT32_MAX / 2 || t2 > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  SchedState sc;
  sc.s1 = reinterpret_cast<int32_t*>(wsb + w.sched);
  sc.s2 = sc.s1 + moe::sched_ints(t1, grid);
  sc.stride1 = static_cast<int>(moe::sched_slot_stride(t1, grid));
  sc.stride2 = static_cast<int>(moe::sched_slot_stride(t2, grid));
  const int64_t n_sched = moe::sched_ints(t1, grid) + moe::sched_ints(t2, grid);
  if (moe::launch_zero_i32(sc.s1, static_cast<int>(n_sched), st) != hipSuccess) return MOE_ERR_HIP;
  if (fp8) return grouped_ffn_fp8(s, u, expert_offset, sorted_token, routed, shared, y_routed, y_shared,
                                  wsb, w, sc, grid, b_tiled, st);
  uint16_t* h_r = reinterpret_cast<uint16_t*>(wsb + w.h_routed);
  uint16_t* h_s = reinterpret_cast<uint16_t*>(wsb + w.h_shared);
  const moe::GemmArgs g1 =
      gate_up_args(s, u, expert_offset, sorted_token, routed, shared, h_r, h_s, b_tiled, sc.s1, sc.stride1);
  hipError_t err = moe::launch_grouped_gemm_bf16(g1, true, grid, st);
  if (err != hipSuccess) return MOE_ERR_HIP;

  moe::GemmArgs g2{};
  g2.a_routed = h_r;
  g2.a_shared = h_s;
  g2.lda_routed = s->d_ff;
  g2.lda_shared = static_cast<int64_t>(s->n_shared) * s->d_ff;
  g2.gather = nullptr;
  g2.b1_routed = static_cast<const uint16_t*>(routed->w2);
  g2.b1_shared = s->n_shared > 0 ? static_cast<const uint16_t*>(shared->w2) : nullptr;
  g2.b_expert_stride = static_cast<int64_t>(s->d) * s->d_ff;
  g2.ldb = s->d_ff;
  g2.out_routed = y_routed;
  g2.out_shared = y_shared;
  g2.ldo_routed = s->d;
  g2.ldo_shared = s->d;
  g2.offset = expert_offset;
  g2.n_r = s->n_routed;
  g2.n_shared_groups = s->n_shared > 0 ? 1 : 0;
  g2.T = s->T;
  g2.N = s->d;
  g2.K = s->d_ff;
  g2.k_segments = s->n_shared;
  g2.sched = sc.s2;
  g2.b_tiled = b_tiled;
  g2.slot_stride = sc.stride2;
  (void)P;
  return from_hip(moe::launch_grouped_gemm_bf16(g2, false, grid, st));
}

}  // namespace

extern "C" {

moe_status moe_grouped_ffn(const moe_shape* s, const void* u, const int32_t* expert_offset,
                           const int32_t* sorted_token, const moe_expert_set* routed,
                           const moe_expert_set* shared, void* y_routed, float* y_shared, void* ws,
                           size_t ws_bytes, void* stream) {
  if (moe_status c = grouped_ffn_check(s, u, expert_offset, sorted_token, routed, shared, y_routed, y_shared))
    return c;
  if (s->T == 0) return MOE_OK;
  if (!ws || ws_bytes < ffn_workspace(s).total) return MOE_ERR_WORKSPACE;
  return grouped_ffn_run(s, u, expert_offset, sorted_token, routed, shared, y_routed, y_shared, ws, stream);
}

moe_status moe_grouped_ffn_noalloc(const moe_shape* s, const void* u, const int32_t* expert_offset,
                                   const int32_t* sorted_token, const moe_expert_set* routed,
                                   const moe_expert_set* shared, void* y_routed, float* y_shared, void* stream) {
  if (moe_status c = grouped_ffn_check(s, u, expert_offset, sorted_token, routed, shared, y_routed, y_shared))
    return c;
  if (s->T == 0) return MOE_OK;
  if (ffn_workspace(s).total > moe::kNoAllocScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  void* scratch = nullptr;  // this device's copy of the library's fixed scratch array
  if (moe::noalloc_scratch(&scratch) != hipSuccess) return MOE_ERR_HIP;
  return grouped_ffn_run(s, u, expert_offset, sorted_token, routed, shared, y_routed, y_shared, scratch, stream);
}

moe_status moe_combine(const moe_shape* s, const void* u, const void* y_routed,
                       const float* y_shared, const int32_t* pair_row, const float* topk_gate,
                       void* out, void* stream) {
  if (!valid_shape(s) || !ok_t(s, u) || !ok_t(s, y_routed) || !ok_t(s, pair_row) || !ok_t(s, topk_gate) ||
      !ok_t(s, out))
    return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0 && !ok_t(s, y_shared)) return MOE_ERR_INVALID_ARG;
  if (s->T == 0) return MOE_OK;
  if (out == u) return MOE_ERR_INVALID_ARG;
  if (moe_status d = debug_check({range(pair_row, s->T * s->top_k, 0, static_cast<int32_t>(s->T * s->top_k))},
                                 stream))
    return d;
  return from_hip(moe::launch_combine(s->act == MOE_BF16 ? 1 : 0, u, y_routed,
                                      s->n_shared > 0 ? y_shared : nullptr, pair_row, topk_gate,
                                      out, s->T, s->d, s->top_k, as_stream(stream)));
}

moe_status moe_bias_update(const moe_shape* s, const int32_t* expert_count, float gamma,
                           float* bias, void* stream) {
  if (!valid_shape(s) || !expert_count || !bias) return MOE_ERR_INVALID_ARG;
  if (!(gamma >= 0.0f) || gamma > 1.0f) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_bias_update(expert_count, s->T, s->n_routed, s->top_k, gamma, bias,
                                          as_stream(stream)));
}

moe_status moe_pack_weights(const moe_shape* s, int32_t matrix, int64_t n_experts, const void* src, void* dst,
                            void* stream) {
  if (!valid_shape(s) || !src || !dst || n_experts < 1) return MOE_ERR_INVALID_ARG;
  if (matrix != MOE_W1 && matrix != MOE_W3 && matrix != MOE_W2) return MOE_ERR_INVALID_ARG;
  if (s->ffn == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (!tiled_shape(s)) return MOE_ERR_UNSUPPORTED;
  const int esz = s->ffn == MOE_FP8_E4M3 ? 1 : 2;
  const int64_t N = matrix == MOE_W2 ? s->d : s->d_ff;
  const int64_t K = matrix == MOE_W2 ? s->d_ff : s->d;
  const int R = matrix == MOE_W2 ? 256 : 128;
  const int64_t bytes = n_experts * N * K * esz;
  if (n_experts > (1LL << 40) / (N * K)) return MOE_ERR_INVALID_ARG;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlap
  return from_hip(moe::launch_pack_weights(src, dst, esz, n_experts, N, K, R, as_stream(stream)));
}

moe_status moe_quantize_fp8(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t tile_r,
                            int32_t tile_c, uint8_t* q, float* scale, void* stream) {
  if (!x || !q || !scale) return MOE_ERR_INVALID_ARG;
  if (xt != MOE_F32 && xt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!((tile_r == 1 && tile_c == 128) || (tile_r == 128 && tile_c == 128)))
    return MOE_ERR_UNSUPPORTED;
  if (rows < 1 || cols < 1 || rows % tile_r != 0 || cols % tile_c != 0) return MOE_ERR_INVALID_ARG;
  if (rows * cols >= (1LL << 40)) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_quantize_fp8(x, xt, rows, cols, tile_r, tile_c, q, scale,
                                           as_stream(stream)));
}

moe_status moe_combine_backward(const moe_shape* s, const void* dout, const void* y_routed,
                                const int32_t* pair_row, const float* topk_gate, void* dy_routed, float* dgate,
                                void* stream) {
  if (!valid_shape(s) || !ok_t(s, dout) || !ok_t(s, y_routed) || !ok_t(s, pair_row) || !ok_t(s, topk_gate) ||
      !ok_t(s, dy_routed) || !ok_t(s, dgate))
    return MOE_ERR_INVALID_ARG;
  if (!backward_shape(s)) return MOE_ERR_UNSUPPORTED;
  if (s->T == 0) return MOE_OK;
  if (moe_status d = debug_check({range(pair_row, s->T * s->top_k, 0, static_cast<int32_t>(s->T * s->top_k))},
                                 stream))
    return d;
  return from_hip(moe::launch_combine_backward(dout, y_routed, pair_row, topk_gate, dy_routed, dgate, s->T, s->d,
                                               s->top_k, as_stream(stream)));
}

moe_status moe_grouped_ffn_backward(const moe_shape* s, const void* u, const void* dout,
                                    const int32_t* expert_offset, const int32_t* sorted_token,
                                    const moe_expert_set* routed, const moe_expert_set* shared,
                                    const void* dy_routed, void* dx_routed, float* dx_shared,
                                    const moe_expert_grads* d_routed, const moe_expert_grads* d_shared, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!valid_shape(s) || !ok_t(s, u) || !ok_t(s, dout) || !expert_offset || !ok_t(s, sorted_token) || !routed ||
      !ok_t(s, dy_routed) || !ok_t(s, dx_routed) || !d_routed)
    return MOE_ERR_INVALID_ARG;
  if (!routed->w1 || !routed->w3 || !routed->w2 || !d_routed->dw1 || !d_routed->dw3 || !d_routed->dw2)
    return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0) {
    if (!shared || !shared->w1 || !shared->w3 || !shared->w2 || !ok_t(s, dx_shared) || !d_shared ||
        !d_shared->dw1 || !d_shared->dw3 || !d_shared->dw2)
      return MOE_ERR_INVALID_ARG;
  }
  if (!backward_shape(s) || !gemm_offsets_fit(s)) return MOE_ERR_UNSUPPORTED;
  if (routed->layout != MOE_LAYOUT_ROWS && routed->layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0 && shared->layout != routed->layout) return MOE_ERR_INVALID_ARG;
  const int tiled = routed->layout == MOE_LAYOUT_TILED ? 1 : 0;
  if (s->T == 0) {  // no rows: every weight gradient is zero (in either layout)
    const size_t m = sizeof(uint16_t) * s->d * s->d_ff;  // one weight matrix
    hipStream_t st = as_stream(stream);
    hipError_t e = hipSuccess;
    for (void* p : {d_routed->dw1, d_routed->dw3, d_routed->dw2})
      if (e == hipSuccess) e = zero_bytes(p, m * s->n_routed, st);
    if (s->n_shared > 0)
      for (void* p : {d_shared->dw1, d_shared->dw3, d_shared->dw2})
        if (e == hipSuccess) e = zero_bytes(p, m * s->n_shared, st);
    return from_hip(e);
  }
  const BwdWorkspace w = bwd_workspace(s);
  if (!ws || ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  {
    const int64_t P = s->T * s->top_k;
    if (moe_status d = debug_check({offsets(expert_offset, s->n_routed, static_cast<int32_t>(P)),
                                    range(sorted_token, P, 0, static_cast<int32_t>(s->T))},
                                   stream))
      return d;
  }
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  moe::BwdArgs a{};
  a.u = static_cast<const uint16_t*>(u);
  a.dout = static_cast<const uint16_t*>(dout);
  a.dy_routed = static_cast<const uint16_t*>(dy_routed);
  a.offset = expert_offset;
  a.sorted_token = sorted_token;
  a.w1r = static_cast<const uint16_t*>(routed->w1);
  a.w3r = static_cast<const uint16_t*>(routed->w3);
  a.w2r = static_cast<const uint16_t*>(routed->w2);
  const bool has_s = s->n_shared > 0;
  a.w1s = has_s ? static_cast<const uint16_t*>(shared->w1) : nullptr;
  a.w3s = has_s ? static_cast<const uint16_t*>(shared->w3) : nullptr;
  a.w2s = has_s ? static_cast<const uint16_t*>(shared->w2) : nullptr;
  a.zero = reinterpret_cast<uint16_t*>(wsb + w.zero);
  a.xs = reinterpret_cast<uint16_t*>(wsb + w.xs);
  a.h_r = reinterpret_cast<uint16_t*>(wsb + w.h_r);
  a.da_r = reinterpret_cast<uint16_t*>(wsb + w.da_r);
  a.dv_r = reinterpret_cast<uint16_t*>(wsb + w.dv_r);
  a.h_s = reinterpret_cast<uint16_t*>(wsb + w.h_s);
  a.da_s = reinterpret_cast<uint16_t*>(wsb + w.da_s);
  a.dv_s = reinterpret_cast<uint16_t*>(wsb + w.dv_s);
  a.a_r = reinterpret_cast<float*>(wsb + w.a_r);
  a.v_r = reinterpret_cast<float*>(wsb + w.v_r);
  a.a_s = reinterpret_cast<float*>(wsb + w.a_s);
  a.v_s = reinterpret_cast<float*>(wsb + w.v_s);
  a.dx_r = static_cast<uint16_t*>(dx_routed);
  a.dx_s = has_s ? dx_shared : nullptr;
  a.dw1r = static_cast<uint16_t*>(d_routed->dw1);
  a.dw3r = static_cast<uint16_t*>(d_routed->dw3);
  a.dw2r = static_cast<uint16_t*>(d_routed->dw2);
  a.dw1s = has_s ? static_cast<uint16_t*>(d_shared->dw1) : nullptr;
  a.dw3s = has_s ? static_cast<uint16_t*>(d_shared->dw3) : nullptr;
  a.dw2s = has_s ? static_cast<uint16_t*>(d_shared->dw2) : nullptr;
  a.T = s->T;
  a.K = s->top_k;
  a.d = s->d;
  a.F = s->d_ff;
  a.n_r = s->n_routed;
  a.n_s = s->n_shared;
  a.tiled = tiled;
  // a, v (fp32) and h (bf16) from the forward's gate/up GEMM, then the rest of the backward
  hipStream_t st = as_stream(stream);
  const int grid = gemm_grid();
  const int64_t t1 = ffn_max_tiles(s, 1);
  if (t1 > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  int32_t* sched = reinterpret_cast<int32_t*>(wsb + w.sched);
  if (moe::launch_zero_i32(sched, static_cast<int>(moe::sched_ints(t1, grid)), st) != hipSuccess) return MOE_ERR_HIP;
  moe::GemmArgs g1 = gate_up_args(s, u, expert_offset, sorted_token, routed, shared, a.h_r, a.h_s, tiled, sched,
                                  static_cast<int>(moe::sched_slot_stride(t1, grid)));
  g1.pre_gate_routed = a.a_r;
  g1.pre_up_routed = a.v_r;
  g1.pre_gate_shared = a.a_s;
  g1.pre_up_shared = a.v_s;
  if (moe::launch_grouped_gemm_bf16(g1, true, grid, st) != hipSuccess) return MOE_ERR_HIP;
  return from_hip(moe::launch_ffn_backward(a, st));
}

moe_status moe_route_backward(const moe_shape* s, const void* u, const void* centroids, const int32_t* topk_idx,
                              const float* topk_gate, const float* dgate, const int32_t* expert_offset,
                              const int32_t* sorted_token, const int32_t* pair_row, const void* dout,
                              const void* dx_routed, const float* dx_shared, void* du, void* dcentroids, float* dz,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!valid_shape(s) || !ok_t(s, u) || !centroids || !ok_t(s, topk_idx) || !ok_t(s, topk_gate) ||
      !ok_t(s, dgate) || !expert_offset || !ok_t(s, sorted_token) || !ok_t(s, pair_row) || !ok_t(s, dout) ||
      !ok_t(s, dx_routed) || !ok_t(s, du) || !dcentroids || !ok_t(s, dz))
    return MOE_ERR_INVALID_ARG;
  if (s->n_shared > 0 && !ok_t(s, dx_shared)) return MOE_ERR_INVALID_ARG;
  if (!backward_shape(s)) return MOE_ERR_UNSUPPORTED;
  if (s->T == 0)  // no tokens: the centroid gradient is zero
    return from_hip(zero_bytes(dcentroids, sizeof(uint16_t) * s->n_routed * s->d, as_stream(stream)));
  if (!ws || ws_bytes < moe_workspace_bytes(s, MOE_CALL_ROUTE_BACKWARD)) return MOE_ERR_WORKSPACE;
  {
    const int64_t P = s->T * s->top_k;
    if (moe_status d = debug_check({range(topk_idx, P, 0, s->n_routed), range(pair_row, P, 0, static_cast<int32_t>(P)),
                                    offsets(expert_offset, s->n_routed, static_cast<int32_t>(P)),
                                    range(sorted_token, P, 0, static_cast<int32_t>(s->T))},
                                   stream))
      return d;
  }
  return from_hip(moe::launch_route_backward(s->score == MOE_SCORE_SOFTMAX ? 1 : 0, u, centroids, topk_idx,
                                             topk_gate, dgate, expert_offset, sorted_token, pair_row, dout,
                                             dx_routed, s->n_shared > 0 ? dx_shared : nullptr, du, dcentroids, dz,
                                             static_cast<float*>(ws), s->T, s->d, s->n_routed, s->top_k,
                                             as_stream(stream)));
}

}  // extern "C"

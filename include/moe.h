/*
 * moe.h - C ABI of the DeepSeekMoE layer (forward, bias update, backward) on AMD MI355X
 * (gfx950).
 *
 * The layer (DeepSeek-V3 explainer, "DeepSeek-V3 テクニカルレポート 論文解説",
 * xyznot.com, method section 2 "DeepSeekMoE with auxiliary-loss-free balancing"):
 *
 *   h'_t = u_t + sum_{j<N_s} FFN^(s)_j(u_t) + sum_{i<N_r} g_{i,t} FFN^(r)_i(u_t)
 *   s_{i,t} = Sigmoid(u_t . e_i)
 *   g'_{i,t} = s_{i,t} if s_{i,t} + b_i is among the K largest of {s_{j,t} + b_j}, else 0
 *   g_{i,t}  = g'_{i,t} normalised over the selected experts
 *   end of step: b_i -= gamma if expert i is overloaded, += gamma if underloaded
 *
 * FFN_i is the gated SiLU form W2 (SiLU(W1 x) * (W3 x)) with no bias terms. The
 * optional FP8 path follows the same page's key ideas (E4M3 everywhere, 1x128
 * activation tiles, 128x128 weight blocks, FP32 accumulation every 128 products)
 * and the quantisation pseudo-code of "DeepSeek モデルアーキテクチャ徹底解説"
 * (deepseekmodel.com): scale = amax / 448.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers, allocated and owned by the caller.
 *    The library allocates no device memory and keeps no per-call state; the one
 *    exception, moe_grouped_ffn_noalloc, uses a fixed array that is part of the
 *    library's device code (each GPU's copy keeps the last call's scratch contents).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every call
 *    only enqueues work and returns; calls on one stream run in order. There is no
 *    device-to-host copy or synchronisation inside any call (MOE_DEBUG aside, below),
 *    no allocation and no memset: the forward calls can be recorded into a HIP graph by
 *    stream capture and replayed (after one uncaptured call has loaded the kernels).
 *  - Arguments are validated on the host before anything is enqueued; a bad
 *    argument returns MOE_ERR_INVALID_ARG (or MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE)
 *    and touches no memory. Kernels trust the index arrays produced by earlier calls,
 *    unless the environment variable MOE_DEBUG is 1: then every call that takes
 *    topk_idx, expert_offset, sorted_token or pair_row first checks them on the device
 *    (in range; offsets from 0 to T*K, non-decreasing), waits for the check (the one
 *    synchronisation in the library), and returns MOE_ERR_INVALID_ARG without launching
 *    anything else if one fails.
 *  - Results are deterministic: the same inputs give bit-identical outputs, counts,
 *    permutations and biases on every run (no atomics on any result).
 *  - Row-major layouts throughout; "[A, B]" means A rows of B contiguous elements.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad shape or bad dtype combination   */
  MOE_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement    */
  MOE_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required     */
  MOE_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed          */
  MOE_ERR_SCRATCH_LIMIT = 5 /* moe_grouped_ffn_noalloc: the shape needs more scratch
                               than its fixed buffer (MOE_NOALLOC_SCRATCH_BYTES) holds */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Router scoring.
 *   SIGMOID  the explainer's method section 2: s = Sigmoid(z), top-K of s + b, gates s
 *            normalised over the selection (the default, 0).
 *   SOFTMAX  the deepseekmodel.com DeepSeekMoE forward listing: top-K of the logits z
 *            themselves, no bias, gates = softmax of the K selected logits. */
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score;

/* Layer shape.
 *   T        tokens in the batch (>= 0). An empty batch (T = 0) is valid: arrays whose
 *            size scales with T may then be NULL, and each call only defines its outputs
 *            that do not: moe_dispatch zeroes expert_count and expert_offset,
 *            moe_bias_update leaves the bias unchanged (every count equals the mean, 0),
 *            moe_grouped_ffn_backward zeroes the weight gradients and moe_route_backward
 *            the centroid gradient; the other calls return MOE_OK and do nothing.
 *   d        hidden size (multiple of 64, at least 64)
 *   n_routed routed experts N_r (1..256)
 *   top_k    experts per token K (1..min(N_r, 16))
 *   n_shared shared experts N_s (0..8)
 *   d_ff     SwiGLU intermediate size per expert (multiple of 64, at least 64)
 *            The bf16 and FP8 expert GEMMs need d % 256 == 0 and d_ff % 128 == 0
 *            (moe_grouped_ffn returns MOE_ERR_UNSUPPORTED otherwise); fp32 takes any valid
 *            shape.
 *   act      dtype of u, the centroids and the output: MOE_F32 or MOE_BF16
 *   ffn      dtype of the expert GEMM operands: MOE_F32 (with act F32), MOE_BF16 or
 *            MOE_FP8_E4M3 (both with act BF16)
 *   score    moe_score of the router (only moe_route reads it) */
typedef struct {
  int64_t T;
  int32_t d, n_routed, top_k, n_shared, d_ff;
  int32_t act, ffn; /* moe_dtype */
  int32_t score;    /* moe_score */
} moe_shape;

/* Weight layouts. ROWS: [E, N, K] row-major as listed below. TILED: the same values
 * reordered by moe_pack_weights so that each GEMM tile's K-step is contiguous in HBM
 * (bf16 and FP8 only). */
typedef enum { MOE_LAYOUT_ROWS = 0, MOE_LAYOUT_TILED = 1 } moe_weight_layout;

/* Expert weights of one kind (routed: E = n_routed; shared: E = n_shared).
 *   w1, w3: [E, d_ff, d]  gate and up projections (row j of expert i = output j)
 *   w2:     [E, d, d_ff]  down projection
 * Element type: fp32 (ffn F32), bf16 (ffn BF16) or E4M3 codes, one byte each (FP8).
 * For FP8 the 128x128 block scales (fp32) are
 *   s1, s3: [E, d_ff/128, d/128]    s2: [E, d/128, d_ff/128]
 * and NULL otherwise (scales are never tiled). Weights are quantised once with
 * moe_quantize_fp8(.., 128, 128), on the row-major layout.
 * layout: moe_weight_layout of w1, w3 and w2. */
typedef struct {
  const void *w1, *w3, *w2;
  const float *s1, *s3, *s2;
  int32_t layout;
} moe_expert_set;

/* ---------------------------------------------------------------------------
 * moe_route: router of method section 2 (sigmoid affinity, biased top-K, gates), or
 * with shape->score == MOE_SCORE_SOFTMAX the forward listing's softmax router.
 *   u         [T, d]      act dtype
 *   centroids [N_r, d]    act dtype (the e_i; a bias-free linear gate)
 *   bias      [N_r]       fp32, the b_i (read only here; may be NULL for SOFTMAX, which
 *                         does not read it)
 *   topk_idx  [T, K]      int32 out: selected expert ids, ascending within a token
 *   topk_gate [T, K]      fp32 out: g_{i,t} aligned with topk_idx; sums to 1 per token
 *   ws            workspace of moe_workspace_bytes(shape, MOE_CALL_ROUTE) bytes (the
 *                 partial logits of the K chunks; 0 bytes, ws may be NULL, for fp32 act)
 * Logits accumulate in fp32 (bf16: per K chunk, the chunks added in order); ties in
 * the selection key (s + b, or z) go to the lower expert index. SOFTMAX gates are
 * expf(z_k - max z) over the selection divided by their sum in ascending expert order. */
moe_status moe_route(const moe_shape* shape, const void* u, const void* centroids,
                     const float* bias, int32_t* topk_idx, float* topk_gate, void* ws,
                     size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_dispatch: the per-expert grouping behind the sums of h'_t (the explainer's
 * equation; the per-expert token masks of the deepseekmodel.com forward listing):
 * a stable counting sort of the T*K (token, slot) pairs by expert.
 *   topk_idx      [T, K]     int32 in (from moe_route)
 *   expert_count  [N_r]      int32 out: pairs per expert (the expert's load)
 *   expert_offset [N_r + 1]  int32 out: exclusive prefix sum of expert_count
 *   sorted_token  [T*K]      int32 out: source token of each sorted row; rows of
 *                            expert i are [offset[i], offset[i+1]), tokens ascending
 *   pair_row      [T, K]     int32 out: sorted row of pair (t, k)
 *   ws            workspace of moe_workspace_bytes(shape, MOE_CALL_DISPATCH) bytes */
moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* expert_count,
                        int32_t* expert_offset, int32_t* sorted_token, int32_t* pair_row,
                        void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_ffn: every routed expert's SwiGLU FFN on its sorted rows, and every
 * shared expert's on all tokens (the FFN terms of h'_t).
 *   u             [T, d]       act dtype
 *   expert_offset [N_r + 1]    from moe_dispatch (read on the device only)
 *   sorted_token  [T*K]        from moe_dispatch
 *   routed        N_r experts; shared: N_s experts (may be NULL when N_s == 0)
 *   y_routed      [T*K, d]     out, act dtype: FFN_i(u_t) for sorted row r of (t, i)
 *   y_shared      [T, d]       out, fp32: sum over the shared experts (not used, and may
 *                              be NULL, when N_s = 0)
 *   ws            workspace of moe_workspace_bytes(shape, MOE_CALL_GROUPED_FFN) bytes;
 *                 holds H (and, for FP8, the 1x128-quantised u and H with their scales)
 *                 and the GEMMs' tile-scheduling state
 * H is rounded to the GEMM operand type (fp32, bf16; FP8: fp32 then 1x128 E4M3).
 * routed and shared must have the same layout; TILED needs ffn BF16 or FP8 (else
 * MOE_ERR_UNSUPPORTED). Both layouts give bit-identical results. With ffn BF16 or FP8, u
 * must take fewer than 2^32 bytes in the GEMM operand type (bf16: T*d below 2^31, at
 * d = 7168 up to 299,593 tokens; FP8: T*d below 2^32) and d, d_ff and N_s*d_ff must each
 * be below 2^22, else MOE_ERR_UNSUPPORTED. */
moe_status moe_grouped_ffn(const moe_shape* shape, const void* u, const int32_t* expert_offset,
                           const int32_t* sorted_token, const moe_expert_set* routed,
                           const moe_expert_set* shared, void* y_routed, float* y_shared,
                           void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * moe_grouped_ffn_noalloc: moe_grouped_ffn without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops, harnesses
 * that forbid hipMalloc). It calls no allocating routine: the scratch the kernels need
 * (tile-scheduling state and H, the bytes moe_workspace_bytes(shape, MOE_CALL_GROUPED_FFN)
 * gives) lives in a fixed device array inside the library, MOE_NOALLOC_SCRATCH_BYTES long,
 * of which each GPU holds its own copy until the process ends (its address is looked up
 * once per device, on that device's first call). Arguments, outputs and results are those
 * of moe_grouped_ffn, bit for bit.
 *  - A shape whose workspace exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 *    MOE_ERR_SCRATCH_LIMIT and enqueues nothing (at the V3 shape, d = 7168 and d_ff = 2048
 *    with 8 + 1 experts per token, bf16 fits up to 1,818 tokens).
 *  - Every call on one GPU shares that GPU's array, and the array keeps the last call's
 *    contents (the call clears the state it needs zeroed itself, with a fill kernel). So
 *    calls that overlap on one GPU (on different streams, or from several threads without
 *    ordering) race and give wrong results: order them on one stream. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_grouped_ffn_noalloc(const moe_shape* shape, const void* u, const int32_t* expert_offset,
                                   const int32_t* sorted_token, const moe_expert_set* routed,
                                   const moe_expert_set* shared, void* y_routed, float* y_shared,
                                   void* stream);

/* ---------------------------------------------------------------------------
 * moe_combine: h'_t = u_t + shared sum + sum_k g_{k,t} * y_routed[pair_row[t,k]], in
 * fp32 in that order (experts ascending), rounded once to the act dtype.
 *   out [T, d] act dtype (may not alias u) */
moe_status moe_combine(const moe_shape* shape, const void* u, const void* y_routed,
                       const float* y_shared, const int32_t* pair_row, const float* topk_gate,
                       void* out, void* stream);

/* ---------------------------------------------------------------------------
 * moe_bias_update: end-of-step rule of method section 2. With the mean load
 * T*K/N_r: count_i > mean -> b_i = fl32(b_i - gamma); count_i < mean -> fl32(b_i + gamma);
 * count_i == mean -> unchanged (the comparison is exact, in integers).
 *   bias [N_r] fp32, updated in place. Feeds the next step's moe_route. */
moe_status moe_bias_update(const moe_shape* shape, const int32_t* expert_count, float gamma,
                           float* bias, void* stream);

/* ---------------------------------------------------------------------------
 * moe_quantize_fp8: E4M3 tile quantisation (deepseekmodel.com pseudo-code; tile
 * shapes from the explainer's key ideas). Per tile_r x tile_c tile:
 *   amax = max|x| (fp32), s = fl32(amax / 448), q = E4M3_RNE(fl32(x / s)) saturating
 *   at +-448 (OCP E4M3FN codes); s == 0 gives q = 0.
 *   x [rows, cols] of dtype xt (MOE_F32 or MOE_BF16); rows % tile_r == 0,
 *   cols % tile_c == 0; (tile_r, tile_c) = (1, 128) or (128, 128).
 *   q [rows, cols] uint8 out; scale [rows/tile_r, cols/tile_c] fp32 out. */
moe_status moe_quantize_fp8(const void* x, int32_t xt, int64_t rows, int64_t cols, int32_t tile_r,
                            int32_t tile_c, uint8_t* q, float* scale, void* stream);

/* ---------------------------------------------------------------------------
 * moe_pack_weights: reorders one weight array of an expert set from the ROWS layout
 * into the TILED layout read by moe_grouped_ffn. Not a step of the layer: a one-time
 * preparation, like the FP8 quantisation of the weights. With KS = 128 bytes of K
 * (64 bf16 or 128 FP8 codes) and R = 128 for W1/W3 (N = d_ff, K = d) or 256 for W2
 * (N = d, K = d_ff), [E, N, K] becomes [E][N/R][K/KS][R][KS].
 *   matrix      MOE_W1, MOE_W3 or MOE_W2
 *   n_experts   E (>= 1)
 *   src, dst    device arrays of E*N*K elements of the ffn dtype (bf16 or E4M3 codes);
 *               they must not overlap
 * Needs a shape the MFMA kernels tile (d % 256 == 0, d_ff % 128 == 0); ffn F32 gives
 * MOE_ERR_UNSUPPORTED. */
enum { MOE_W1 = 0, MOE_W3 = 1, MOE_W2 = 2 };
moe_status moe_pack_weights(const moe_shape* shape, int32_t matrix, int64_t n_experts, const void* src,
                            void* dst, void* stream);

/* ===========================================================================
 * Backward (gradients of L = sum dout . h' with the routing held fixed; the selection is
 * piecewise constant, and the bias only selects, so it has no gradient). Gradients are
 * bf16 ("gradients in BF16", quantisation section of deepseekmodel.com): GEMM operands
 * bf16, fp32 accumulation, each gradient rounded once. Needs act = ffn = MOE_BF16,
 * d % 256 == 0 and d_ff % 128 == 0, and the size limits of the bf16 moe_grouped_ffn (its
 * gate/up GEMM recomputes a, v and h here), else MOE_ERR_UNSUPPORTED. The weights may be in
 * either layout (the same for routed and shared, else MOE_ERR_INVALID_ARG); the weight
 * gradients are written in the weights' layout, so an elementwise optimiser step applies to
 * TILED weights as it is. Both layouts give bit-identical results.
 * The order of the three calls: moe_combine_backward, moe_grouped_ffn_backward,
 * moe_route_backward. */

/* Weight gradients of one expert kind, bf16, in the layout of the weights they belong to
 * (ROWS: dw1, dw3 [E, d_ff, d], dw2 [E, d, d_ff]; TILED: as moe_pack_weights makes them). */
typedef struct {
  void *dw1, *dw3, *dw2;
} moe_expert_grads;

/* moe_combine_backward: adjoint of moe_combine.
 *   dout      [T, d]   bf16: gradient of the layer output
 *   y_routed  [T*K, d] bf16 from moe_grouped_ffn; pair_row, topk_gate [T, K] from the step
 *   dy_routed [T*K, d] bf16 out: g_{k,t} dout_t at sorted row pair_row[t, k]
 *   dgate     [T, K]   fp32 out: dout_t . y_routed[pair_row[t, k]] (fp32 sum) */
moe_status moe_combine_backward(const moe_shape* shape, const void* dout, const void* y_routed,
                                const int32_t* pair_row, const float* topk_gate, void* dy_routed,
                                float* dgate, void* stream);

/* moe_grouped_ffn_backward: backward of every expert's SwiGLU FFN on its rows. With
 * a = X W1^T, v = X W3^T, h = SiLU(a) v, y = h W2^T per expert:
 *   dh = dY W2, da = dh v SiLU'(a), dv = dh SiLU(a) (h, da, dv rounded to bf16),
 *   dX = da W1 + dv W3, dW1 = da^T X, dW3 = dv^T X, dW2 = dY^T h.
 *   u, expert_offset, sorted_token, routed, shared: as in moe_grouped_ffn
 *   dout      [T, d] bf16: the shared experts' dY
 *   dy_routed [T*K, d] bf16 from moe_combine_backward: the routed rows' dY
 *   dx_routed [T*K, d] bf16 out, sorted rows
 *   dx_shared [T, d] fp32 out: sum over the shared experts (NULL when N_s == 0)
 *   d_routed  weight gradients of the N_r routed experts (out; zeros for experts with no
 *             rows); d_shared: of the N_s shared experts (NULL when N_s == 0)
 *   ws        moe_workspace_bytes(shape, MOE_CALL_GROUPED_FFN_BACKWARD) bytes (h, da, dv) */
moe_status moe_grouped_ffn_backward(const moe_shape* shape, const void* u, const void* dout,
                                    const int32_t* expert_offset, const int32_t* sorted_token,
                                    const moe_expert_set* routed, const moe_expert_set* shared,
                                    const void* dy_routed, void* dx_routed, float* dx_shared,
                                    const moe_expert_grads* d_routed, const moe_expert_grads* d_shared,
                                    void* ws, size_t ws_bytes, void* stream);

/* moe_route_backward: the router's logit gradients, the input gradient and the centroid
 * gradient (the explainer's method section 2 for sigmoid gates, the forward listing for
 * softmax gates; shape->score picks).
 *   sigmoid: s_k = Sigmoid(z_k) of the picks (z recomputed in fp32), S = sum s_k,
 *            dz_k = (dg_k - sum_j g_j dg_j) / S * s_k (1 - s_k) with g_j = s_j / S;
 *   softmax: dz_k = g_k (dg_k - sum_j g_j dg_j) with the forward's gates.
 *   u, centroids, topk_idx, topk_gate, expert_offset, sorted_token, pair_row: the step's
 *   dgate [T, K] from moe_combine_backward; dout [T, d] bf16
 *   dx_routed, dx_shared from moe_grouped_ffn_backward (dx_shared NULL when N_s == 0)
 *   du   [T, d] bf16 out: dout + dx_shared + sum_k dx_routed[pair_row] + sum_k dz_k e_{i_k},
 *        added in fp32 in that order (experts ascending) and rounded once
 *   dcentroids [N_r, d] bf16 out: sum over expert i's sorted rows of dz u_t
 *   dz   [T, K] fp32 out
 *   ws   moe_workspace_bytes(shape, MOE_CALL_ROUTE_BACKWARD) bytes */
moe_status moe_route_backward(const moe_shape* shape, const void* u, const void* centroids,
                              const int32_t* topk_idx, const float* topk_gate, const float* dgate,
                              const int32_t* expert_offset, const int32_t* sorted_token,
                              const int32_t* pair_row, const void* dout, const void* dx_routed,
                              const float* dx_shared, void* du, void* dcentroids, float* dz, void* ws,
                              size_t ws_bytes, void* stream);

/* workspace sizing: call = MOE_CALL_ROUTE, MOE_CALL_DISPATCH, MOE_CALL_GROUPED_FFN,
 * MOE_CALL_GROUPED_FFN_BACKWARD or MOE_CALL_ROUTE_BACKWARD; 0 for others, for invalid
 * shapes and for an empty batch (T = 0: no call needs a workspace, ws may be NULL) */
enum { MOE_CALL_ROUTE = 0, MOE_CALL_DISPATCH = 1, MOE_CALL_GROUPED_FFN = 2,
       MOE_CALL_COMBINE = 3, MOE_CALL_BIAS_UPDATE = 4, MOE_CALL_GROUPED_FFN_BACKWARD = 5,
       MOE_CALL_ROUTE_BACKWARD = 6 };
size_t moe_workspace_bytes(const moe_shape* shape, int32_t call);

const char* moe_status_string(moe_status status);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */

/*
 * CPU oracle for the DeepSeekMoE layer forward pass and its bias update.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * constant generator with the HIP path.
 *
 * Sources ("pages"):
 *  [V3] "DeepSeek-V3 テクニカルレポート 論文解説" (xyznot.com explainer of the
 *       DeepSeek-V3 technical report): key ideas (1 shared + 256 routed experts,
 *       8 active; FP8 E4M3 with 1x128 activation tiles, 128x128 weight blocks,
 *       FP32 accumulation every N_c = 128); method section 2 "DeepSeekMoE with
 *       auxiliary-loss-free balancing" (the equation for h'_t, the sigmoid
 *       affinity, the equation for g'_{i,t}, the end-of-step +-gamma bias rule).
 *  [ARCH] "DeepSeek モデルアーキテクチャ徹底解説" (deepseekmodel.com): the block
 *       quantisation pseudo-code (scale = amax / 448, the E4M3 maximum) and the
 *       DeepSeekMoE forward listing (gate without bias, per-expert masks).
 *
 * Arithmetic: every sum is in double, in the order stated at each function.
 * The only rounding points are the ones named (H at the FFN's rounding point,
 * and the FP8 codes). The oracle is parallel over tokens or rows, never inside
 * a sum, so its results do not depend on the thread count.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8 = 2 };
enum { ORC_SIGMOID = 0, ORC_SOFTMAX = 1 }; /* router scoring */

/* ---- scalar conversions --------------------------------------------------- */
double orc_bf16_value(uint16_t bits);          /* exact widening                     */
uint16_t orc_bf16_from_double(double x);       /* round to nearest even              */
double orc_e4m3_value(uint8_t code);           /* OCP E4M3FN decode (NaN for 0x7F/0xFF) */
uint8_t orc_e4m3_from_float(float x);          /* round to nearest even, saturating at +-448 */

/* array forms of the two roundings */
void orc_bf16_from_double_array(const double* x, int64_t n, uint16_t* out);
void orc_e4m3_from_float_array(const float* x, int64_t n, uint8_t* out);

/* ---- FP8 tile quantisation ([V3] key ideas; [ARCH] quantisation pseudo-code)
 * x: [rows, cols] row-major of dtype xdt (ORC_F32 or ORC_BF16); tiles of tr x tc
 * (rows % tr == 0, cols % tc == 0). Per tile: amax = max |x| (fp32), s = fl32(amax/448),
 * q = E4M3_RNE(fl32(x / s)); s == 0 gives q = 0. s: [rows/tr, cols/tc]. */
void orc_quantize_tiles(const void* x, int xdt, int64_t rows, int64_t cols, int tr, int tc,
                        uint8_t* q, float* s);

/* ---- routing
 * score ORC_SIGMOID ([V3] method section 2: sigmoid affinity, biased top-K, g'
 * normalised) or ORC_SOFTMAX ([ARCH] DeepSeekMoE forward listing: top-K of the logits,
 * no bias, softmax over the selected logits).
 * u: [n, d] rows (act dtype), e: [n_r, d] (act dtype), b: [n_r] fp32 (sigmoid only).
 * Out: idx [n, K] ascending expert ids; gate [n, K] (double) aligned with idx;
 * gap [n] = v_(K) - v_(K+1) (+inf when K == n_r); v [n, n_r] selection keys, s + b or
 * z (optional). */
void orc_route(int64_t n, int d, int n_r, int K, int act, int score, const void* u, const void* e,
               const float* b, int32_t* idx, double* gate, double* gap, double* v);

/* ---- dispatch: counts, exclusive offsets [n_r+1], rows sorted by (expert, token) */
void orc_dispatch(int64_t T, int n_r, int K, const int32_t* idx, int32_t* count,
                  int32_t* offset, int32_t* sorted_token, int32_t* pair_row);

/* ---- end-of-step bias update ([V3] method section 2): overloaded -gamma, underloaded +gamma */
void orc_bias_update(int64_t T, int n_r, int K, const int32_t* count, float gamma, float* b);

/* ---- one expert's SwiGLU FFN on n rows
 * ffn = ORC_F32: x, w fp32; H rounded to fp32.
 * ffn = ORC_BF16: x, w bf16; H rounded to bf16.
 * ffn = ORC_FP8: x bf16 (quantised here per 1x128), w1/w3/w2 E4M3 codes with block
 *   scales s1/s3 [d_ff/128, d/128] and s2 [d/128, d_ff/128]; H rounded to fp32 then
 *   quantised per 1x128.
 * w1, w3: [d_ff, d]; w2: [d, d_ff]. Out: y [n, d] in double; h [n, d_ff] the H values
 * at the rounding point (optional). */
void orc_expert_rows(int d, int d_ff, int ffn, const void* x, int64_t n, const void* w1,
                     const void* w3, const void* w2, const float* s1, const float* s3,
                     const float* s2, double* h, double* y);

/* ---- the layer for n tokens ([V3] method section 2, equation for h'_t)
 * u: [n, d] rows of the tokens (act dtype). Routed expert i's weights are wr1[i],
 * wr3[i], wr2[i] (and scales sr1[i], sr3[i], sr2[i] for FP8); an expert no token of
 * the list selects may be NULL. Shared experts likewise (ws*, ss*), n_s of them.
 * Out: out [n, d] = u + sum_shared + sum_routed(g * y), in double; routing by
 * orc_route with the given score; optional idx/gate/gap as in orc_route; optional shared_sum/routed_sum [n, d].
 * Returns 0, or -1 if a routed expert that is needed has a NULL weight pointer. */
int orc_layer(int64_t n, int d, int n_r, int K, int n_s, int d_ff, int act, int ffn, int score,
              const void* u, const void* e, const float* b,
              const void* const* wr1, const void* const* wr3, const void* const* wr2,
              const float* const* sr1, const float* const* sr3, const float* const* sr2,
              const void* const* ws1, const void* const* ws3, const void* const* ws2,
              const float* const* ss1, const float* const* ss3, const float* const* ss2,
              double* out, int32_t* idx, double* gate, double* gap,
              double* shared_sum, double* routed_sum);

/* ---- backward of the layer (gradients of L = sum dout . h', routing held fixed)
 * Forward as orc_layer with bf16 or fp32 experts (FP8 returns -1). Row chain rule:
 *   a = W1 x, v = W3 x, h = SiLU(a) v, y = W2 h; dh = W2^T dy, da = dh v SiLU'(a),
 *   dv = dh SiLU(a), dx = W1^T da + W3^T dv; row terms of dW1, dW3, dW2: da x^T,
 *   dv x^T, dy h^T. Rounded to the operand type: h, da, dv, and a routed row's dy =
 *   g dout_t ([ARCH] quantisation section: gradients in BF16); shared rows take dy = dout_t.
 * Router ([V3] method section 2: the bias only selects): with the selection fixed,
 *   sigmoid: dz_k = (dg_k - sum_j g_j dg_j) / S * s_k (1 - s_k), S = sum of picked s;
 *   softmax: dz_k = g_k (dg_k - sum_j g_j dg_j); dg_k = dout_t . y_k.
 * Outputs (each may be NULL; so may entries of dwr* and dws*):
 *   du [n, d] = dout_t + shared dx + routed dx (ascending) + sum_k dz_k e_{i_k}
 *   de [n_r, d] = sum over tokens choosing i (ascending) of dz u_t
 *   dwr1[i], dwr3[i] [d_ff, d], dwr2[i] [d, d_ff]; dws* for the shared experts,
 *     each a sum over the expert's rows in token order
 *   idx, gate, dgate, dz [n, K]
 * Returns 0, -1 (FP8) or -2 (a needed expert has no weights). */
int orc_layer_backward(int64_t n, int d, int n_r, int K, int n_s, int d_ff, int act, int ffn,
                       int score, const void* u, const void* e, const float* b,
                       const void* const* wr1, const void* const* wr3, const void* const* wr2,
                       const void* const* ws1, const void* const* ws3, const void* const* ws2,
                       const void* dout, double* du, double* de, double* const* dwr1,
                       double* const* dwr3, double* const* dwr2, double* const* dws1,
                       double* const* dws3, double* const* dws2, int32_t* idx_out,
                       double* gate_out, double* dgate_out, double* dz_out);

/* ---- combine of precomputed expert outputs ([V3] method section 2, equation for h'_t)
 * u [n, d] and y [rows, d] in act dtype; ysh [n, d] fp32 (sum over shared experts, may be
 * NULL); pair_row [n, K]; gate [n, K] fp32. out [n, d] double. */
void orc_combine(int64_t n, int d, int K, int act, const void* u, const float* ysh,
                 const void* y, const int32_t* pair_row, const float* gate, double* out);

#ifdef __cplusplus
}
#endif
#endif

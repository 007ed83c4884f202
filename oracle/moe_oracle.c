/*
 * CPU oracle for the DeepSeekMoE layer forward pass and its bias update.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product path never does. It shares
 * no code with the HIP path. Page citations and the rounding points are listed
 * in moe_oracle.h; each function below names the passage it follows.
 *
 * Plainness over speed: every sum is an ordinary loop in double, in ascending
 * index order. The only liberty taken is computing four independent sums side by
 * side (four rows of a weight matrix at once); each sum keeps its own order.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- conversions */

double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits, 8 exponent bits), ties to
 * even, straight from double (a single rounding). */
uint16_t orc_bf16_from_double(double x) {
  if (isnan(x)) return 0x7FC0;
  double ax = fabs(x), q;
  if (ax < 0x1p-126) {
    q = rint(ax * 0x1p133) * 0x1p-133; /* subnormal grid: 2^-133 */
  } else {
    int ex;
    double m = frexp(ax, &ex); /* ax = m * 2^ex, m in [0.5, 1) */
    q = ldexp(rint(ldexp(m, 8)), ex - 8);
  }
  float f = (float)(signbit(x) ? -q : q); /* exact, or +-inf past the bf16 range */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* OCP 8-bit floating point, E4M3 ("FN") variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds subnormals m * 2^-9; the all-ones
 * pattern S.1111.111 is NaN; no infinities; largest finite value S.1111.110 = 448,
 * the maximum the [ARCH] quantisation pseudo-code divides by. */
double orc_e4m3_value(uint8_t code) {
  int sign = code >> 7, ex = (code >> 3) & 15, man = code & 7;
  double v;
  if (ex == 15 && man == 7) return NAN;
  if (ex == 0)
    v = ldexp((double)man, -9);
  else
    v = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

/* Nearest E4M3 value, ties to the even code; magnitudes past 448 saturate to 448. */
uint8_t orc_e4m3_from_float(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double ax = fabs((double)x);
  int code;
  if (ax >= 448.0) {
    code = 0x7E;
  } else if (ax < 0x1p-6) {
    code = (int)rint(ax * 0x1p9); /* subnormal step 2^-9; 8 lands on the first normal */
  } else {
    int ex;
    frexp(ax, &ex);       /* ax in [2^(ex-1), 2^ex) */
    int e = ex - 1;       /* unbiased exponent, -6..8 */
    int n = (int)rint(ldexp(ax, 3 - e)); /* 8..16 steps of 2^(e-3) */
    code = ((e + 7) << 3) + (n - 8);     /* n == 16 carries into the next exponent */
    if (code > 0x7E) code = 0x7E;
  }
  return (uint8_t)(sign | code);
}

static inline double load_val(const void* p, int dt, int64_t i) {
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  return orc_bf16_value(((const uint16_t*)p)[i]);
}

static inline float load_f32(const void* p, int dt, int64_t i) {
  if (dt == ORC_F32) return ((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ------------------------------------------------------------ FP8 quantisation */

/* [ARCH] block quantisation pseudo-code, with the tile shapes of [V3] key ideas
 * (1x128 activation tiles, 128x128 weight blocks): scale = amax / 448; quantise
 * x / scale onto the E4M3 grid. The division and the rounding onto the grid are
 * two separate correctly rounded steps. */
static void quantize_tile(const void* x, int xdt, int64_t cols, int tr, int tc, int64_t br,
                          int64_t bc, uint8_t* q, float* s_out) {
  float amax = 0.0f;
  for (int64_t r = br * tr; r < (br + 1) * tr; ++r)
    for (int64_t c = bc * tc; c < (bc + 1) * tc; ++c) {
      float a = fabsf(load_f32(x, xdt, r * cols + c));
      if (a > amax) amax = a;
    }
  const float sc = amax / 448.0f;
  *s_out = sc;
  for (int64_t r = br * tr; r < (br + 1) * tr; ++r)
    for (int64_t c = bc * tc; c < (bc + 1) * tc; ++c)
      q[r * cols + c] = (sc == 0.0f) ? 0 : orc_e4m3_from_float(load_f32(x, xdt, r * cols + c) / sc);
}

void orc_quantize_tiles(const void* x, int xdt, int64_t rows, int64_t cols, int tr, int tc,
                        uint8_t* q, float* s) {
  const int64_t nbr = rows / tr, nbc = cols / tc;
#pragma omp parallel for schedule(static)
  for (int64_t tb = 0; tb < nbr * nbc; ++tb)
    quantize_tile(x, xdt, cols, tr, tc, tb / nbc, tb % nbc, q, s + tb);
}

/* one row of 1x128 tiles, serial (called inside the per-row parallel loops) */
static void quantize_row(const void* x, int xdt, int64_t cols, uint8_t* q, float* s) {
  for (int64_t bc = 0; bc < cols / 128; ++bc) quantize_tile(x, xdt, cols, 1, 128, 0, bc, q, s + bc);
}

/* -------------------------------------------------------------------- routing */

/* score == ORC_SIGMOID, [V3] method section 2: s_{i,t} = Sigmoid(u_t . e_i); expert i
 * is selected when s_{i,t} + b_i is among the K largest biased scores, and then
 * g'_{i,t} = s_{i,t}; g_{i,t} is g' normalised over the selected experts (the bias
 * only steers the choice, it is not part of the gate).
 * score == ORC_SOFTMAX, the [ARCH] DeepSeekMoE forward listing: the K largest logits
 * z_{i,t} = u_t . e_i are selected (no bias; b is not read), and the gates are the
 * softmax of the selected logits, exp(z_i - z_max) / sum over the selection of
 * exp(z_j - z_max), the sum taken in ascending expert order.
 * Either way equal keys go to the lower index, v holds the selection keys (s + b or
 * z), and the K ids are returned in ascending order. */
static void route_one(int d, int n_r, int K, int act, int score, const void* u_row, const void* e,
                      const float* b, double* ud, double* s, double* v, char* taken, int32_t* idx,
                      double* gate, double* gap) {
  for (int c = 0; c < d; ++c) ud[c] = load_val(u_row, act, c);
  for (int i0 = 0; i0 < n_r; i0 += 4) {
    const int ni = (n_r - i0) < 4 ? (n_r - i0) : 4;
    double z[4] = {0, 0, 0, 0};
    for (int c = 0; c < d; ++c)
      for (int q = 0; q < ni; ++q) z[q] += ud[c] * load_val(e, act, (int64_t)(i0 + q) * d + c);
    for (int q = 0; q < ni; ++q) {
      if (score == ORC_SOFTMAX) {
        s[i0 + q] = z[q];
        v[i0 + q] = z[q];
      } else {
        s[i0 + q] = sigmoid(z[q]);
        v[i0 + q] = s[i0 + q] + (double)b[i0 + q];
      }
      taken[i0 + q] = 0;
    }
  }
  double vK = 0.0;
  for (int k = 0; k < K; ++k) { /* K passes of arg-max; strict '>' keeps the lower index */
    int best = -1;
    for (int i = 0; i < n_r; ++i)
      if (!taken[i] && (best < 0 || v[i] > v[best])) best = i;
    taken[best] = 1;
    vK = v[best];
  }
  if (K < n_r) {
    int nxt = -1;
    for (int i = 0; i < n_r; ++i)
      if (!taken[i] && (nxt < 0 || v[i] > v[nxt])) nxt = i;
    *gap = vK - v[nxt];
  } else {
    *gap = INFINITY;
  }
  int k = 0;
  for (int i = 0; i < n_r; ++i)
    if (taken[i]) idx[k++] = i;
  if (score == ORC_SOFTMAX) { /* g'_k = exp(z_k - max z), then normalised like s */
    double zmax = -INFINITY;
    for (k = 0; k < K; ++k) zmax = s[idx[k]] > zmax ? s[idx[k]] : zmax;
    for (k = 0; k < K; ++k) s[idx[k]] = exp(s[idx[k]] - zmax);
  }
  double denom = 0.0;
  for (k = 0; k < K; ++k) denom += s[idx[k]];
  for (k = 0; k < K; ++k) gate[k] = s[idx[k]] / denom;
}

void orc_route(int64_t n, int d, int n_r, int K, int act, int score, const void* u, const void* e,
               const float* b, int32_t* idx, double* gate, double* gap, double* v) {
  const size_t esz = (act == ORC_F32) ? 4 : 2;
#pragma omp parallel
  {
    double* ud = (double*)malloc(sizeof(double) * d);
    double* s = (double*)malloc(sizeof(double) * n_r);
    double* vv = (double*)malloc(sizeof(double) * n_r);
    char* taken = (char*)malloc(n_r);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
      double g;
      route_one(d, n_r, K, act, score, (const char*)u + (size_t)t * d * esz, e, b, ud, s, vv, taken,
                idx + t * K, gate + t * K, &g);
      if (gap) gap[t] = g;
      if (v) memcpy(v + t * n_r, vv, sizeof(double) * n_r);
    }
    free(ud);
    free(s);
    free(vv);
    free(taken);
  }
}

/* ------------------------------------------------------------------- dispatch */

/* The sums over experts in [V3]'s equation for h'_t, grouped per expert as the
 * [ARCH] listing's per-expert token masks do: a stable counting sort of the
 * (token, slot) pairs by expert, tokens ascending within an expert. */
void orc_dispatch(int64_t T, int n_r, int K, const int32_t* idx, int32_t* count,
                  int32_t* offset, int32_t* sorted_token, int32_t* pair_row) {
  for (int i = 0; i < n_r; ++i) count[i] = 0;
  for (int64_t p = 0; p < T * K; ++p) count[idx[p]]++;
  offset[0] = 0;
  for (int i = 0; i < n_r; ++i) offset[i + 1] = offset[i] + count[i];
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * n_r);
  for (int i = 0; i < n_r; ++i) next[i] = offset[i];
  for (int64_t t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      int32_t row = next[idx[t * K + k]]++;
      sorted_token[row] = (int32_t)t;
      pair_row[t * K + k] = row;
    }
  free(next);
}

/* [V3] method section 2, end of step: an overloaded expert's bias drops by gamma,
 * an underloaded one's rises by gamma. Load is the expert's count in this step,
 * compared with the mean load T*K/n_r (as integers: count*n_r vs T*K); an expert
 * exactly at the mean is neither and keeps its bias. The add is one fp32 add. */
void orc_bias_update(int64_t T, int n_r, int K, const int32_t* count, float gamma, float* b) {
  const int64_t total = T * (int64_t)K;
  for (int i = 0; i < n_r; ++i) {
    const int64_t load = (int64_t)count[i] * n_r;
    if (load > total)
      b[i] = b[i] - gamma;
    else if (load < total)
      b[i] = b[i] + gamma;
  }
}

/* ------------------------------------------------------------------ expert FFN */

/* y = W2 (SiLU(W1 x) * (W3 x)) with SiLU(a) = a * sigmoid(a), for one row whose
 * values are xd[0..d) (already decoded to double). FFN_i of [V3]'s equation for
 * h'_t, in the gated (SwiGLU) form; no bias terms. */
static void ffn_row_dense(int d, int d_ff, int wdt, const double* xd, const void* w1,
                          const void* w3, const void* w2, int hround, double* h, double* y) {
  for (int j0 = 0; j0 < d_ff; j0 += 4) {
    double a[4] = {0, 0, 0, 0}, g[4] = {0, 0, 0, 0};
    const int nj = (d_ff - j0) < 4 ? (d_ff - j0) : 4;
    for (int c = 0; c < d; ++c)
      for (int q = 0; q < nj; ++q) {
        a[q] += xd[c] * load_val(w1, wdt, (int64_t)(j0 + q) * d + c);
        g[q] += xd[c] * load_val(w3, wdt, (int64_t)(j0 + q) * d + c);
      }
    for (int q = 0; q < nj; ++q) {
      double hv = a[q] * sigmoid(a[q]) * g[q];
      /* rounding point of H: the storage type of the second GEMM's operand */
      h[j0 + q] = hround == ORC_F32 ? (double)(float)hv : orc_bf16_value(orc_bf16_from_double(hv));
    }
  }
  for (int n0 = 0; n0 < d; n0 += 4) {
    double acc[4] = {0, 0, 0, 0};
    const int nn = (d - n0) < 4 ? (d - n0) : 4;
    for (int j = 0; j < d_ff; ++j)
      for (int q = 0; q < nn; ++q) acc[q] += h[j] * load_val(w2, wdt, (int64_t)(n0 + q) * d_ff + j);
    for (int q = 0; q < nn; ++q) y[n0 + q] = acc[q];
  }
}

/* FP8 form ([V3] key ideas; [ARCH] pseudo-code): out[r] = sum over 128-wide blocks kb
 * of s_x[kb] * s_w[rb][kb] * B_kb, B_kb = sum over the block of dec(q_x) * dec(q_w).
 * Every E4M3 value is a multiple of 2^-9 below 2^9 in magnitude, so B_kb is exact in
 * double; the dequantisation by the product of the two scales follows per block
 * (the N_c = 128 accumulation interval). */
static double fp8_dot(int len, const uint8_t* qx, const float* sx, const uint8_t* qw,
                      const float* sw_row, const double* lut) {
  double acc = 0.0;
  for (int kb = 0; kb < len / 128; ++kb) {
    double blk = 0.0;
    for (int c = kb * 128; c < kb * 128 + 128; ++c) blk += lut[qx[c]] * lut[qw[c]];
    acc += ((double)sx[kb] * (double)sw_row[kb]) * blk;
  }
  return acc;
}

static void ffn_row_fp8(int d, int d_ff, const void* x_row, const uint8_t* w1, const uint8_t* w3,
                        const uint8_t* w2, const float* s1, const float* s3, const float* s2,
                        const double* lut, uint8_t* qx, float* sx, float* hf, uint8_t* qh,
                        float* sh, double* h, double* y) {
  quantize_row(x_row, ORC_BF16, d, qx, sx);
  const int dkb = d / 128, fkb = d_ff / 128;
  for (int j = 0; j < d_ff; ++j) {
    double a = fp8_dot(d, qx, sx, w1 + (int64_t)j * d, s1 + (int64_t)(j / 128) * dkb, lut);
    double g = fp8_dot(d, qx, sx, w3 + (int64_t)j * d, s3 + (int64_t)(j / 128) * dkb, lut);
    hf[j] = (float)(a * sigmoid(a) * g); /* rounding point: fp32, then 1x128 quantisation */
    if (h) h[j] = (double)hf[j];
  }
  quantize_row(hf, ORC_F32, d_ff, qh, sh);
  for (int n = 0; n < d; ++n)
    y[n] = fp8_dot(d_ff, qh, sh, w2 + (int64_t)n * d_ff, s2 + (int64_t)(n / 128) * fkb, lut);
}

typedef struct {
  double* xd;
  double* h;
  uint8_t* qx;
  float* sx;
  float* hf;
  uint8_t* qh;
  float* sh;
} row_scratch;

static void scratch_alloc(row_scratch* s, int d, int d_ff) {
  s->xd = (double*)malloc(sizeof(double) * d);
  s->h = (double*)malloc(sizeof(double) * d_ff);
  s->qx = (uint8_t*)malloc(d);
  s->sx = (float*)malloc(sizeof(float) * (d / 128 + 1));
  s->hf = (float*)malloc(sizeof(float) * d_ff);
  s->qh = (uint8_t*)malloc(d_ff);
  s->sh = (float*)malloc(sizeof(float) * (d_ff / 128 + 1));
}

static void scratch_free(row_scratch* s) {
  free(s->xd); free(s->h); free(s->qx); free(s->sx); free(s->hf); free(s->qh); free(s->sh);
}

static void e4m3_table(double lut[256]) {
  for (int i = 0; i < 256; ++i) lut[i] = orc_e4m3_value((uint8_t)i);
}

/* one row through one expert; h_out (optional) gets H at its rounding point */
static void expert_row(int d, int d_ff, int ffn, const void* x_row, const void* w1, const void* w3,
                       const void* w2, const float* s1, const float* s3, const float* s2,
                       const double* lut, row_scratch* sc, double* h_out, double* y) {
  if (ffn == ORC_FP8) {
    ffn_row_fp8(d, d_ff, x_row, (const uint8_t*)w1, (const uint8_t*)w3, (const uint8_t*)w2, s1, s3,
                s2, lut, sc->qx, sc->sx, sc->hf, sc->qh, sc->sh, h_out, y);
    return;
  }
  for (int c = 0; c < d; ++c) sc->xd[c] = load_val(x_row, ffn, c);
  ffn_row_dense(d, d_ff, ffn, sc->xd, w1, w3, w2, ffn, sc->h, y);
  if (h_out) memcpy(h_out, sc->h, sizeof(double) * d_ff);
}

void orc_expert_rows(int d, int d_ff, int ffn, const void* x, int64_t n, const void* w1,
                     const void* w3, const void* w2, const float* s1, const float* s3,
                     const float* s2, double* h, double* y) {
  const size_t xsz = (ffn == ORC_F32) ? 4 : 2;
  double lut[256];
  e4m3_table(lut);
#pragma omp parallel
  {
    row_scratch sc;
    scratch_alloc(&sc, d, d_ff);
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; ++r)
      expert_row(d, d_ff, ffn, (const char*)x + (size_t)r * d * xsz, w1, w3, w2, s1, s3, s2, lut,
                 &sc, h ? h + r * d_ff : NULL, y + r * d);
    scratch_free(&sc);
  }
}

/* ----------------------------------------------------------------------- layer */

/* [V3] method section 2, equation for h'_t, token by token:
 *   h'_t = u_t + sum_{j<N_s} FFN^(s)_j(u_t) + sum_{i selected} g_{i,t} FFN^(r)_i(u_t),
 * added in that order (residual, shared experts ascending, routed experts ascending),
 * in double. Shared experts carry no gate. */
int orc_layer(int64_t n, int d, int n_r, int K, int n_s, int d_ff, int act, int ffn, int score,
              const void* u, const void* e, const float* b,
              const void* const* wr1, const void* const* wr3, const void* const* wr2,
              const float* const* sr1, const float* const* sr3, const float* const* sr2,
              const void* const* ws1, const void* const* ws3, const void* const* ws2,
              const float* const* ss1, const float* const* ss3, const float* const* ss2,
              double* out, int32_t* idx, double* gate, double* gap,
              double* shared_sum, double* routed_sum) {
  const size_t usz = (act == ORC_F32) ? 4 : 2;
  int32_t* my_idx = (int32_t*)malloc(sizeof(int32_t) * n * K);
  double* my_gate = (double*)malloc(sizeof(double) * n * K);
  double* my_gap = (double*)malloc(sizeof(double) * n);
  orc_route(n, d, n_r, K, act, score, u, e, b, my_idx, my_gate, my_gap, NULL);
  int status = 0;
  for (int64_t p = 0; p < n * K; ++p)
    if (!wr1[my_idx[p]] || !wr3[my_idx[p]] || !wr2[my_idx[p]]) status = -1;
  if (status == 0) {
    double lut[256];
    e4m3_table(lut);
#pragma omp parallel
    {
      row_scratch sc;
      scratch_alloc(&sc, d, d_ff);
      double* y = (double*)malloc(sizeof(double) * d);
      double* ssum = (double*)malloc(sizeof(double) * d);
      double* rsum = (double*)malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < n; ++t) {
        const void* xrow = (const char*)u + (size_t)t * d * usz;
        double* o = out + t * d;
        for (int c = 0; c < d; ++c) {
          o[c] = load_val(xrow, act, c);
          ssum[c] = 0.0;
          rsum[c] = 0.0;
        }
        for (int j = 0; j < n_s; ++j) {
          expert_row(d, d_ff, ffn, xrow, ws1[j], ws3[j], ws2[j], ss1 ? ss1[j] : NULL,
                     ss3 ? ss3[j] : NULL, ss2 ? ss2[j] : NULL, lut, &sc, NULL, y);
          for (int c = 0; c < d; ++c) {
            o[c] += y[c];
            ssum[c] += y[c];
          }
        }
        for (int k = 0; k < K; ++k) {
          const int i = my_idx[t * K + k];
          const double g = my_gate[t * K + k];
          expert_row(d, d_ff, ffn, xrow, wr1[i], wr3[i], wr2[i], sr1 ? sr1[i] : NULL,
                     sr3 ? sr3[i] : NULL, sr2 ? sr2[i] : NULL, lut, &sc, NULL, y);
          for (int c = 0; c < d; ++c) {
            o[c] += g * y[c];
            rsum[c] += g * y[c];
          }
        }
        if (shared_sum) memcpy(shared_sum + t * d, ssum, sizeof(double) * d);
        if (routed_sum) memcpy(routed_sum + t * d, rsum, sizeof(double) * d);
      }
      free(y);
      free(ssum);
      free(rsum);
      scratch_free(&sc);
    }
  }
  if (idx) memcpy(idx, my_idx, sizeof(int32_t) * n * K);
  if (gate) memcpy(gate, my_gate, sizeof(double) * n * K);
  if (gap) memcpy(gap, my_gap, sizeof(double) * n);
  free(my_idx);
  free(my_gate);
  free(my_gap);
  return status;
}

/* ------------------------------------------------------------ array helpers */

void orc_bf16_from_double_array(const double* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(x[i]);
}

void orc_e4m3_from_float_array(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_from_float(x[i]);
}

/* [V3] method section 2, equation for h'_t, as a combine of precomputed expert
 * outputs: out_t = u_t + ysh_t + sum_k g_{t,k} y[pair_row[t,k]], in double, in that
 * order (k ascending = experts ascending). ysh may be NULL (no shared experts). */
void orc_combine(int64_t n, int d, int K, int act, const void* u, const float* ysh,
                 const void* y, const int32_t* pair_row, const float* gate, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n; ++t)
    for (int c = 0; c < d; ++c) {
      double o = load_val(u, act, t * d + c);
      if (ysh) o += (double)ysh[t * d + c];
      for (int k = 0; k < K; ++k)
        o += (double)gate[t * K + k] * load_val(y, act, (int64_t)pair_row[t * K + k] * d + c);
      out[t * d + c] = o;
    }
}

/* -------------------------------------------------------------------- backward */

/* rounding to the GEMM operand type (ORC_F32 or ORC_BF16) */
static double op_round(int dt, double x) {
  return dt == ORC_F32 ? (double)(float)x : orc_bf16_value(orc_bf16_from_double(x));
}

/* Backward of one row through one SwiGLU expert, the chain rule on
 *   a = W1 x,  v = W3 x,  h = SiLU(a) v,  y = W2 h,
 * for the row's output gradient dy:
 *   dh = W2^T dy,  da = dh v SiLU'(a),  dv = dh SiLU(a),  dx = W1^T da + W3^T dv,
 * with SiLU(a) = a sigmoid(a) and SiLU'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))).
 * The row's weight-gradient terms are da x^T (W1), dv x^T (W3) and dy h^T (W2).
 * Rounding points: h as in the forward; da and dv at the operand type, since the
 * products that take them run in that type ([ARCH] quantisation section: gradients
 * in BF16). xd and dyd are the row's x and dy in double, dy already rounded.
 * Out: h, da, dv [d_ff]; y [d] (optional); dx [d] (optional). */
static void ffn_row_backward(int d, int d_ff, int wdt, const double* xd, const double* dyd,
                             const void* w1, const void* w3, const void* w2, double* h, double* da,
                             double* dv, double* y, double* dx) {
  for (int j = 0; j < d_ff; ++j) {
    double a = 0.0, v = 0.0, dh = 0.0;
    for (int c = 0; c < d; ++c) {
      a += xd[c] * load_val(w1, wdt, (int64_t)j * d + c);
      v += xd[c] * load_val(w3, wdt, (int64_t)j * d + c);
      dh += dyd[c] * load_val(w2, wdt, (int64_t)c * d_ff + j);
    }
    const double sg = sigmoid(a);
    h[j] = op_round(wdt, a * sg * v);
    da[j] = op_round(wdt, dh * v * sg * (1.0 + a * (1.0 - sg)));
    dv[j] = op_round(wdt, dh * a * sg);
  }
  if (y)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < d_ff; ++j) acc += h[j] * load_val(w2, wdt, (int64_t)c * d_ff + j);
      y[c] = acc;
    }
  if (dx)
    for (int c = 0; c < d; ++c) {
      double s1 = 0.0, s3 = 0.0;
      for (int j = 0; j < d_ff; ++j) {
        s1 += da[j] * load_val(w1, wdt, (int64_t)j * d + c);
        s3 += dv[j] * load_val(w3, wdt, (int64_t)j * d + c);
      }
      dx[c] = s1 + s3;
    }
}

/* Gradient of the router's gates with respect to the selected logits z_k.
 * Sigmoid ([V3] method section 2): g_k = s_k / S, s_k = sigmoid(z_k), S = sum of the
 * selected s; the bias only chooses the set, so it carries no gradient and the set is
 * held fixed: dL/ds_k = (dg_k - sum_j g_j dg_j) / S, dz_k = dL/ds_k s_k (1 - s_k).
 * Softmax ([ARCH] forward listing): dz_k = g_k (dg_k - sum_j g_j dg_j).
 * sel[k]: s_k (sigmoid) or z_k (softmax) of the K picks; g: their gates. */
static void router_backward(int K, int score, const double* sel, const double* g, const double* dg,
                            double* dz) {
  double gbar = 0.0;
  for (int k = 0; k < K; ++k) gbar += g[k] * dg[k];
  if (score == ORC_SOFTMAX) {
    for (int k = 0; k < K; ++k) dz[k] = g[k] * (dg[k] - gbar);
    return;
  }
  double S = 0.0;
  for (int k = 0; k < K; ++k) S += sel[k];
  for (int k = 0; k < K; ++k) dz[k] = (dg[k] - gbar) / S * sel[k] * (1.0 - sel[k]);
}

typedef struct {
  double *h, *da, *dv, *dy;
} row_grads;

/* Backward of the layer for n tokens with output gradient dout [n, d] (act dtype),
 * i.e. the gradients of L = sum dout . h' with the routing held fixed (selection is
 * piecewise constant in u, e and b). Forward as orc_layer (bf16 or fp32 experts).
 *   du [n, d]: dout (residual) + shared experts' dx + routed dx + sum_k dz_k e_{i_k}
 *   de [n_r, d]: sum over the tokens that chose expert i of dz u_t
 *   dwr1/dwr3 [d_ff, d], dwr2 [d, d_ff] per routed expert; dws* per shared expert:
 *     sums over the expert's rows in token order of the row terms of ffn_row_backward.
 * A routed row's dy is g_k dout_t rounded to the operand type; a shared row's is dout_t.
 * dgate [n, K] = dout_t . y_{k,t}; dz [n, K] as router_backward. Every output pointer
 * may be NULL (an entry of dwr* / dws* too: that expert's gradient is not formed);
 * only the rows that the requested outputs need are evaluated.
 * Returns 0; -1 for FP8 experts; -2 if a needed expert has no weights. */
int orc_layer_backward(int64_t n, int d, int n_r, int K, int n_s, int d_ff, int act, int ffn,
                       int score, const void* u, const void* e, const float* b,
                       const void* const* wr1, const void* const* wr3, const void* const* wr2,
                       const void* const* ws1, const void* const* ws3, const void* const* ws2,
                       const void* dout, double* du, double* de, double* const* dwr1,
                       double* const* dwr3, double* const* dwr2, double* const* dws1,
                       double* const* dws3, double* const* dws2, int32_t* idx_out,
                       double* gate_out, double* dgate_out, double* dz_out) {
  if (ffn == ORC_FP8) return -1;
  const size_t usz = (act == ORC_F32) ? 4 : 2;
  const int full = du || de || dgate_out || dz_out;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * n * K);
  double* gate = (double*)malloc(sizeof(double) * n * K);
  double* sel = (double*)malloc(sizeof(double) * n * K);
  double* dg = (double*)calloc((size_t)(n * K), sizeof(double));
  double* dz = (double*)calloc((size_t)(n * K), sizeof(double));
  /* routing, as the forward */
#pragma omp parallel
  {
    double* ud = (double*)malloc(sizeof(double) * d);
    double* s = (double*)malloc(sizeof(double) * n_r);
    double* vv = (double*)malloc(sizeof(double) * n_r);
    char* taken = (char*)malloc(n_r);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
      double gap;
      route_one(d, n_r, K, act, score, (const char*)u + (size_t)t * d * usz, e, b, ud, s, vv, taken,
                idx + t * K, gate + t * K, &gap);
      for (int k = 0; k < K; ++k) sel[t * K + k] = s[idx[t * K + k]];
    }
    free(ud); free(s); free(vv); free(taken);
  }
  int status = 0;
  /* which rows are evaluated, and where the kept row terms go */
  const int wants_r = dwr1 || dwr3 || dwr2;
  int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * n * K);
  int64_t n_keep = 0;
  for (int64_t p = 0; p < n * K; ++p) {
    const int i = idx[p];
    const int keep = wants_r && ((dwr1 && dwr1[i]) || (dwr3 && dwr3[i]) || (dwr2 && dwr2[i]));
    slot[p] = keep ? n_keep++ : -1;
    if ((full || keep) && (!wr1[i] || !wr3[i] || !wr2[i])) status = -2;
  }
  int shared_keep = 0;
  for (int j = 0; j < n_s; ++j)
    if ((dws1 && dws1[j]) || (dws3 && dws3[j]) || (dws2 && dws2[j])) shared_keep = 1;
  if (status != 0) {
    free(idx); free(gate); free(sel); free(dg); free(dz); free(slot);
    return status;
  }
  const size_t rowlen = (size_t)3 * d_ff + d;
  double* kept = (double*)malloc(sizeof(double) * rowlen * (size_t)(n_keep > 0 ? n_keep : 1));
  double* kept_s = shared_keep ? (double*)malloc(sizeof(double) * rowlen * (size_t)n * n_s) : NULL;
#pragma omp parallel
  {
    double* xd = (double*)malloc(sizeof(double) * d);
    double* dyd = (double*)malloc(sizeof(double) * d);
    double* y = (double*)malloc(sizeof(double) * d);
    double* dx = (double*)malloc(sizeof(double) * d);
    double* acc = (double*)malloc(sizeof(double) * d);
    double* tmp = (double*)malloc(sizeof(double) * rowlen);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < n; ++t) {
      const void* xrow = (const char*)u + (size_t)t * d * usz;
      int any = full || shared_keep;
      for (int k = 0; k < K; ++k) any |= slot[t * K + k] >= 0;
      if (!any) continue;
      for (int c = 0; c < d; ++c) {
        xd[c] = load_val(xrow, act, c);
        acc[c] = load_val(dout, act, t * d + c); /* residual */
      }
      /* shared experts: dy = dout_t */
      if (full || shared_keep)
        for (int j = 0; j < n_s; ++j) {
          double* r = kept_s ? kept_s + rowlen * (size_t)(t * n_s + j) : tmp;
          for (int c = 0; c < d; ++c) r[3 * d_ff + c] = load_val(dout, act, t * d + c);
          ffn_row_backward(d, d_ff, ffn, xd, r + 3 * d_ff, ws1[j], ws3[j], ws2[j], r, r + d_ff,
                           r + 2 * d_ff, NULL, full ? dx : NULL);
          if (full)
            for (int c = 0; c < d; ++c) acc[c] += dx[c];
        }
      /* routed experts, ascending: dy = g dout_t at the operand type */
      for (int k = 0; k < K; ++k) {
        const int64_t p = t * K + k;
        if (!full && slot[p] < 0) continue;
        const int i = idx[p];
        double* r = slot[p] >= 0 ? kept + rowlen * (size_t)slot[p] : tmp;
        for (int c = 0; c < d; ++c) r[3 * d_ff + c] = op_round(ffn, gate[p] * load_val(dout, act, t * d + c));
        ffn_row_backward(d, d_ff, ffn, xd, r + 3 * d_ff, wr1[i], wr3[i], wr2[i], r, r + d_ff,
                         r + 2 * d_ff, full ? y : NULL, full ? dx : NULL);
        if (full) {
          double s = 0.0;
          for (int c = 0; c < d; ++c) {
            acc[c] += dx[c];
            s += load_val(dout, act, t * d + c) * y[c];
          }
          dg[p] = s;
        }
      }
      if (full) {
        router_backward(K, score, sel + t * K, gate + t * K, dg + t * K, dz + t * K);
        for (int k = 0; k < K; ++k) {
          const int i = idx[t * K + k];
          for (int c = 0; c < d; ++c) acc[c] += dz[t * K + k] * load_val(e, act, (int64_t)i * d + c);
        }
        if (du) memcpy(du + t * d, acc, sizeof(double) * d);
      }
    }
    free(xd); free(dyd); free(y); free(dx); free(acc); free(tmp);
  }
  /* per-expert sums over rows in token order */
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_r + n_s; ++i) {
    const int shared = i >= n_r;
    const int j = shared ? i - n_r : i;
    double* g1 = shared ? (dws1 ? dws1[j] : NULL) : (dwr1 ? dwr1[j] : NULL);
    double* g3 = shared ? (dws3 ? dws3[j] : NULL) : (dwr3 ? dwr3[j] : NULL);
    double* g2 = shared ? (dws2 ? dws2[j] : NULL) : (dwr2 ? dwr2[j] : NULL);
    double* gde = (!shared && de) ? de + (int64_t)j * d : NULL;
    if (!g1 && !g3 && !g2 && !gde) continue;
    if (g1) memset(g1, 0, sizeof(double) * d_ff * d);
    if (g3) memset(g3, 0, sizeof(double) * d_ff * d);
    if (g2) memset(g2, 0, sizeof(double) * d * d_ff);
    if (gde) memset(gde, 0, sizeof(double) * d);
    double* xd = (double*)malloc(sizeof(double) * d);
    for (int64_t t = 0; t < n; ++t) {
      const double* r = NULL;
      double dzt = 0.0;
      if (shared) {
        r = kept_s + rowlen * (size_t)(t * n_s + j);
      } else {
        int k = 0;
        while (k < K && idx[t * K + k] != j) ++k;
        if (k == K) continue;
        const int64_t p = t * K + k;
        dzt = dz[p];
        if (slot[p] >= 0) r = kept + rowlen * (size_t)slot[p];
      }
      for (int c = 0; c < d; ++c) xd[c] = load_val(u, act, t * d + c);
      if (gde)
        for (int c = 0; c < d; ++c) gde[c] += dzt * xd[c];
      if (!r) continue;
      const double *h = r, *da = r + d_ff, *dv = r + 2 * d_ff, *dy = r + 3 * d_ff;
      for (int jj = 0; jj < d_ff; ++jj)
        for (int c = 0; c < d; ++c) {
          if (g1) g1[(int64_t)jj * d + c] += da[jj] * xd[c];
          if (g3) g3[(int64_t)jj * d + c] += dv[jj] * xd[c];
        }
      if (g2)
        for (int c = 0; c < d; ++c)
          for (int jj = 0; jj < d_ff; ++jj) g2[(int64_t)c * d_ff + jj] += dy[c] * h[jj];
    }
    free(xd);
  }
  if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * n * K);
  if (gate_out) memcpy(gate_out, gate, sizeof(double) * n * K);
  if (dgate_out) memcpy(dgate_out, dg, sizeof(double) * n * K);
  if (dz_out) memcpy(dz_out, dz, sizeof(double) * n * K);
  free(idx); free(gate); free(sel); free(dg); free(dz); free(slot); free(kept); free(kept_s);
  return 0;
}

/*
 * FP64 CPU oracle for the routed NVFP4 W4A4 mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, table or constant generator
 * with the HIP library.
 *
 * Plain scalar loops in FP64, compiled without FMA contraction or fast math.
 * Each function follows one passage of the pages (cited by page and section):
 *
 *   [R1] capy-flash README v0.5.4 (spark.entire.vc), "What it does": routed
 *        experts partitioned by expert id; experts not resident computed with
 *        the GPU's W4A4 activation quantization.
 *   [R2] capy-flash README v0.5.4, "Serve": host-side experts encode their
 *        activations to 4 bits exactly as the GPU kernels do (W4A4), which
 *        makes an expert's result independent of the device that ran it.
 *   [R3] capy-flash README v0.5.4, synthetic test-artifact script: 512 NVFP4
 *        experts, top-10 routed plus a shared expert.
 *   [A1] Richland article, "What shipped": 48 MoE layers, 512 experts, 10
 *        routed + 1 shared; NVFP4 = E2M1 codes, UE4M3 block scales, FP32
 *        per-expert scale.
 *   [A2] Richland article, "Why it matters": partials accumulate in FP32;
 *        exchange payloads in BF16 vs FP16 with a 2^-k shift.
 *   [R4] capy-flash README v0.5.4, "Measured" (footnote on the tensor-core
 *        router): a reordered sum can pick another expert where two tie.
 *
 * Readings where the pages are silent (16-element blocks, scale = amax/6 with
 * round-to-nearest-even, SwiGLU, softmax over the k selected logits, shared
 * expert weight 1, low nibble first) are the plainest ones and are stated at
 * each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* F1. E2M1 (OCP 4-bit float): sign bit 3, exponent bits 2..1 (bias 1),
 * mantissa bit 0; exponent 0 is subnormal: 0.5*m.   [A1]                */
double orc_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* F2. UE4M3: the OCP FP8 E4M3 encoding without its sign bit (bit 7 must be
 * 0).  Exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent 0 is
 * subnormal m*2^-9; 0x7F is NaN.   [A1]                                  */
double orc_ue4m3(int code) {
  if (code & 0x80) return NAN;
  if (code == 0x7F) return NAN;
  int e = (code >> 3) & 15, m = code & 7;
  return (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
}

/* Q1. Block scale code: round-to-nearest-even of the exact quotient
 * amax/(6*g) onto the UE4M3 grid (codes 0..126), saturating at 448 (0x7E).
 * The decision compares amax with 6*g*(midpoint of two adjacent grid points);
 * midpoints have at most 5 significant bits, so 6*g*midpoint is exact in FP64
 * for a power-of-two g and the comparison is the exact one.  On an exact tie
 * the even code wins.                                                     */
int orc_scale_code(double amax, double g) {
  int c = 0;
  while (c < 126) {
    double mid = 0.5 * (orc_ue4m3(c) + orc_ue4m3(c + 1));
    double thr = 6.0 * g * mid;
    if (amax > thr) { c++; continue; }
    if (amax == thr && ((c + 1) & 1) == 0) c++;
    break;
  }
  return c;
}

/* Q2. Element code: round-to-nearest-even of |v|/s onto the E2M1 magnitudes
 * {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6; sign = signbit(v) always.
 * Comparisons use |v| against t*s for each midpoint t, exact in FP64.
 * s == 0 gives magnitude 0.                                                */
int orc_elem_code(double v, double s) {
  int mag = 0;
  if (s > 0.0) {
    double a = fabs(v);
    while (mag < 7) {
      double mid = 0.5 * (orc_e2m1(mag) + orc_e2m1(mag + 1));
      double thr = mid * s;
      if (a > thr) { mag++; continue; }
      if (a == thr && ((mag + 1) & 1) == 0) mag++;
      break;
    }
  }
  return mag | (signbit(v) ? 8 : 0);
}

/* Q1-Q3 over a row-major [rows][cols] matrix (cols % 16 == 0), global scale g
 * (a power of two).  codes [rows][cols/2]: element 2i in the low nibble of
 * byte i; scales [rows][cols/16].   [R1][R2]                               */
void orc_quant_rows(const double* v, int64_t rows, int64_t cols, double g, uint8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      const double* x = v + r * cols + b * 16;
      double amax = 0.0;
      for (int i = 0; i < 16; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
      int sc = orc_scale_code(amax, g);
      scales[r * (cols / 16) + b] = (uint8_t)sc;
      double s = orc_ue4m3(sc) * g;
      for (int i = 0; i < 16; i += 2) {
        int lo = orc_elem_code(x[i], s), hi = orc_elem_code(x[i + 1], s);
        codes[r * (cols / 2) + (b * 16 + i) / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* BF16 hidden states -> FP64 (exact). */
void orc_bf16_to_f64(const uint16_t* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_value(x[i]);
}

/* Round an FP64 value to the nearest BF16 (ties to even), directly from
 * FP64 (no intermediate FP32 rounding).  Returns the BF16 bit pattern.     */
uint16_t orc_round_bf16(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0;
  int e;
  frexp(v, &e);                       /* |v| in [2^(e-1), 2^e)            */
  int qexp = e - 8;                   /* 8 significant bits               */
  if (qexp < -133) qexp = -133;       /* BF16 subnormal quantum 2^-133    */
  double r = nearbyint(ldexp(v, -qexp)); /* default mode: ties to even   */
  float f = (float)ldexp(r, qexp);    /* exact: at most 8 bits            */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* Round to FP16 (ties to even), saturating at +-65504; returns the value.   */
double orc_round_f16_sat(double v) {
  if (v == 0.0) return v;
  if (v > 65504.0) return 65504.0;
  if (v < -65504.0) return -65504.0;
  int e;
  frexp(v, &e);
  int qexp = e - 11;
  if (qexp < -24) qexp = -24;
  double r = ldexp(nearbyint(ldexp(v, -qexp)), qexp);
  if (r > 65504.0) r = 65504.0;
  if (r < -65504.0) r = -65504.0;
  return r;
}

/* ------------------------------------------------------------------ */
/* R. Router logits l[t][e] = sum_h x[t][h] * Wr[e][h] in FP64 (every product
 * exact).   [R3][A1][R4]                                                  */
void orc_router_logits(const uint16_t* x, const float* wr, int64_t T, int64_t H, int64_t E, double* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t h = 0; h < H; ++h) acc += bf16_value(x[t * H + h]) * (double)wr[e * H + h];
      logits[t * E + e] = acc;
    }
}

/* Top-k by (logit descending, expert id ascending) and softmax over the k
 * selected logits: w_j = exp(l_j - l_1) / sum_i exp(l_i - l_1).
 * The selected slots are listed in that order.   [R3][A1]                 */
void orc_topk_softmax(const double* logits, int64_t T, int64_t E, int k, int32_t* idx, double* w) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    const double* l = logits + t * E;
    int32_t* out = idx + t * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int64_t e = 0; e < E; ++e) {
        int taken = 0;
        for (int q = 0; q < j; ++q)
          if (out[q] == e) taken = 1;
        if (taken) continue;
        if (best < 0 || l[e] > l[best]) best = (int)e; /* strict: lower id wins ties */
      }
      out[j] = best;
    }
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += exp(l[out[j]] - l[out[0]]);
    for (int j = 0; j < k; ++j) w[t * k + j] = exp(l[out[j]] - l[out[0]]) / den;
  }
}

/* P. Permutation: group the T*k (token, slot) pairs by expert, expert id
 * ascending, then token ascending.  off = exclusive prefix sum of the per-
 * expert counts (off[E] = T*k); row off[e]+r holds expert e's r-th pair;
 * pair id = t*k + j.  (Routed experts are partitioned by expert id [R1].)  */
void orc_permute(const int32_t* idx, int64_t T, int k, int64_t E, int32_t* off, int32_t* row2pair, int32_t* pair2row) {
  int64_t row = 0;
  for (int64_t e = 0; e < E; ++e) {
    off[e] = (int32_t)row;
    for (int64_t t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (idx[t * k + j] == e) {
          row2pair[row] = (int32_t)(t * k + j);
          pair2row[t * k + j] = (int32_t)row;
          row++;
        }
  }
  off[E] = (int32_t)row;
}

/* ------------------------------------------------------------------ */
/* NVFP4 x NVFP4 dot product of one activation row and one weight row over
 * 16-element blocks [b0, b1):
 *   sum_b dec(sa_b) * dec(sw_b) * sum_{i in b} e2m1(qa_i) * e2m1(qw_i)
 * in FP64 (each block term is exact).                                      */
static double nvfp4_dot(const uint8_t* qa, const uint8_t* sa, const uint8_t* qw, const uint8_t* sw, int64_t b0,
                        int64_t b1) {
  double acc = 0.0;
  for (int64_t b = b0; b < b1; ++b) {
    double inner = 0.0;
    for (int i = 0; i < 16; ++i) {
      int64_t c = b * 16 + i;
      int ca = (c & 1) ? (qa[c / 2] >> 4) : (qa[c / 2] & 15);
      int cw = (c & 1) ? (qw[c / 2] >> 4) : (qw[c / 2] & 15);
      inner += orc_e2m1(ca) * orc_e2m1(cw);
    }
    acc += orc_ue4m3(sa[b]) * orc_ue4m3(sw[b]) * inner;
  }
  return acc;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * X. Expert FFN for a list of rows.  Row r pairs activation row a_row[r]
 * (an index into xq/xs, i.e. a token) with expert a_exp[r] of the banks:
 *   W13 codes [n_exp][2I][H/2], scales [n_exp][2I][H/16], gscale [n_exp]
 *       (rows 0..I-1 gate, I..2I-1 up)
 *   W2  codes [n_exp][H][I/2],  scales [n_exp][H][I/16],  gscale [n_exp]
 *   g_i = G13 * g_in * dot(x, W13 row i),  u_i = same with row I+i   (FP64)
 *   h_i = fl32(silu(g_i) * u_i)                 (SwiGLU; rounded to FP32 because
 *                                                the A4 encoding reads FP32 h)
 *   (hq, hs) = A4(h) over 16-blocks of I with g_mid   [R2]
 *   y_n = G2 * g_mid * dot(hq row, W2 row n) over I-blocks [kb0, kb1)   [A2]
 * hq_in/hs_in (nullable) replace the oracle's own h codes (teacher forcing
 * after an accepted near-threshold difference).  Outputs may be NULL except y.
 */
void orc_expert_rows(int64_t n_rows, const int32_t* a_row, const int32_t* a_exp, const uint8_t* xq, const uint8_t* xs,
                     double g_in, const uint8_t* w13q, const uint8_t* w13s, const float* w13g, const uint8_t* w2q,
                     const uint8_t* w2s, const float* w2g, int64_t H, int64_t I, double g_mid, int64_t kb0,
                     int64_t kb1, const uint8_t* hq_in, const uint8_t* hs_in, double* g_out, double* u_out,
                     float* h_out, uint8_t* hq_out, uint8_t* hs_out, double* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t t = a_row[r], e = a_exp[r];
    const uint8_t* qa = xq + t * (H / 2);
    const uint8_t* sa = xs + t * (H / 16);
    double* hv = (double*)malloc(sizeof(double) * (size_t)I);
    uint8_t* hq = (uint8_t*)malloc((size_t)(I / 2));
    uint8_t* hs = (uint8_t*)malloc((size_t)(I / 16));
    const double G13 = (double)w13g[e], G2 = (double)w2g[e];
    for (int64_t i = 0; i < I; ++i) {
      const int64_t rg = e * 2 * I + i, ru = e * 2 * I + I + i;
      double g = G13 * g_in * nvfp4_dot(qa, sa, w13q + rg * (H / 2), w13s + rg * (H / 16), 0, H / 16);
      double u = G13 * g_in * nvfp4_dot(qa, sa, w13q + ru * (H / 2), w13s + ru * (H / 16), 0, H / 16);
      float h = (float)(silu(g) * u);
      hv[i] = (double)h;
      if (g_out) g_out[r * I + i] = g;
      if (u_out) u_out[r * I + i] = u;
      if (h_out) h_out[r * I + i] = h;
    }
    orc_quant_rows(hv, 1, I, g_mid, hq, hs);
    if (hq_out) memcpy(hq_out + r * (I / 2), hq, (size_t)(I / 2));
    if (hs_out) memcpy(hs_out + r * (I / 16), hs, (size_t)(I / 16));
    const uint8_t* hq_use = hq_in ? hq_in + r * (I / 2) : hq;
    const uint8_t* hs_use = hs_in ? hs_in + r * (I / 16) : hs;
    for (int64_t n = 0; n < H; ++n) {
      const int64_t rw = e * H + n;
      y[r * H + n] = G2 * g_mid * nvfp4_dot(hq_use, hs_use, w2q + rw * (I / 2), w2s + rw * (I / 16), kb0, kb1);
    }
    free(hv);
    free(hq);
    free(hs);
  }
}

/* C. Combine, one token per row of the inputs:
 *   out[q] = sum_j w[q][j] * y[q][j] + ysh[q] (+ residual[q])
 * summed in FP64 with w as given (the FP32 router weights); every selected
 * expert contributes, none is skipped.  y [n][k][H]; ysh [n][H] and
 * residual [n][H] (BF16) are nullable.  Writes out_f64 and/or out_bf16 (RNE
 * from FP64), both [n][H].                                                 */
void orc_combine(int64_t n, int k, int64_t H, const double* y, const float* w, const double* ysh,
                 const uint16_t* residual, double* out_f64, uint16_t* out_bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t q = 0; q < n; ++q) {
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) acc += (double)w[q * k + j] * y[(q * k + j) * H + c];
      if (ysh) acc += ysh[q * H + c];
      if (residual) acc += bf16_value(residual[q * H + c]);
      if (out_f64) out_f64[q * H + c] = acc;
      if (out_bf16) out_bf16[q * H + c] = orc_round_bf16(acc);
    }
  }
}

/* ------------------------------------------------------------------ */
/* A8: the 8-bit activation encoding of the W4A8 variant.  The pages name the
 * older W4A8 host path (capy-flash README v0.5.4, "Serve": activations of
 * host-computed experts in 8 bits, made the output depend on where an expert
 * ran) but not its format.  Read here as the A4 encoding with an 8-bit integer
 * element grid: the same 16-element blocks and UE4M3 block scale, chosen as
 * RNE(amax / (127 g)) (127 = the largest INT8 magnitude in place of E2M1's 6),
 * and element codes q = RNE(x / (s g)) on the integers, saturating at +-127
 * (two's complement; zero carries no sign).  The element value is q s g.     */
int orc_scale_code8(double amax, double g) {
  int c = 0;
  while (c < 126) {
    double mid = 0.5 * (orc_ue4m3(c) + orc_ue4m3(c + 1));
    double thr = 127.0 * g * mid; /* exact: <= 12 significant bits times 2^k */
    if (amax > thr) { c++; continue; }
    if (amax == thr && ((c + 1) & 1) == 0) c++;
    break;
  }
  return c;
}

/* q = RNE(|v| / s) on the integers 0..127 (ties to even), with the sign of v;
 * decided by exact comparisons of |v| with (m + 1/2) s; s == 0 gives 0.      */
int orc_int8_code(double v, double s) {
  if (!(s > 0.0)) return 0;
  double a = fabs(v);
  int m = 0;
  while (m < 127) {
    double thr = (m + 0.5) * s;
    if (a > thr) { m++; continue; }
    if (a == thr && ((m + 1) & 1) == 0) m++;
    break;
  }
  return signbit(v) ? -m : m;
}

/* A8 over a row-major [rows][cols] matrix: codes [rows][cols] int8, scales
 * [rows][cols/16].                                                        */
void orc_quant8_rows(const double* v, int64_t rows, int64_t cols, double g, int8_t* codes, uint8_t* scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < cols / 16; ++b) {
      const double* x = v + r * cols + b * 16;
      double amax = 0.0;
      for (int i = 0; i < 16; ++i)
        if (fabs(x[i]) > amax) amax = fabs(x[i]);
      int sc = orc_scale_code8(amax, g);
      scales[r * (cols / 16) + b] = (uint8_t)sc;
      double s = orc_ue4m3(sc) * g;
      for (int i = 0; i < 16; ++i) codes[r * cols + b * 16 + i] = (int8_t)orc_int8_code(x[i], s);
    }
  }
}

/* NVFP4 weight row times an A8 activation row over 16-element blocks [b0, b1):
 *   sum_b dec(sa_b) * dec(sw_b) * sum_{i in b} qa_i * e2m1(qw_i)    (FP64)  */
static double nvfp4_a8_dot(const int8_t* qa, const uint8_t* sa, const uint8_t* qw, const uint8_t* sw, int64_t b0,
                           int64_t b1) {
  double acc = 0.0;
  for (int64_t b = b0; b < b1; ++b) {
    double inner = 0.0;
    for (int i = 0; i < 16; ++i) {
      int64_t c = b * 16 + i;
      int cw = (c & 1) ? (qw[c / 2] >> 4) : (qw[c / 2] & 15);
      inner += (double)qa[c] * orc_e2m1(cw);
    }
    acc += orc_ue4m3(sa[b]) * orc_ue4m3(sw[b]) * inner;
  }
  return acc;
}

/* X with A8 activations (the W4A8 variant): as orc_expert_rows, with x and h
 * encoded by A8 (xq [T][H] int8, hq [n][I] int8).                          */
void orc_expert_rows_a8(int64_t n_rows, const int32_t* a_row, const int32_t* a_exp, const int8_t* xq,
                        const uint8_t* xs, double g_in, const uint8_t* w13q, const uint8_t* w13s, const float* w13g,
                        const uint8_t* w2q, const uint8_t* w2s, const float* w2g, int64_t H, int64_t I, double g_mid,
                        int64_t kb0, int64_t kb1, const int8_t* hq_in, const uint8_t* hs_in, double* g_out,
                        double* u_out, float* h_out, int8_t* hq_out, uint8_t* hs_out, double* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t t = a_row[r], e = a_exp[r];
    const int8_t* qa = xq + t * H;
    const uint8_t* sa = xs + t * (H / 16);
    double* hv = (double*)malloc(sizeof(double) * (size_t)I);
    int8_t* hq = (int8_t*)malloc((size_t)I);
    uint8_t* hs = (uint8_t*)malloc((size_t)(I / 16));
    const double G13 = (double)w13g[e], G2 = (double)w2g[e];
    for (int64_t i = 0; i < I; ++i) {
      const int64_t rg = e * 2 * I + i, ru = e * 2 * I + I + i;
      double g = G13 * g_in * nvfp4_a8_dot(qa, sa, w13q + rg * (H / 2), w13s + rg * (H / 16), 0, H / 16);
      double u = G13 * g_in * nvfp4_a8_dot(qa, sa, w13q + ru * (H / 2), w13s + ru * (H / 16), 0, H / 16);
      float h = (float)(silu(g) * u);
      hv[i] = (double)h;
      if (g_out) g_out[r * I + i] = g;
      if (u_out) u_out[r * I + i] = u;
      if (h_out) h_out[r * I + i] = h;
    }
    orc_quant8_rows(hv, 1, I, g_mid, hq, hs);
    if (hq_out) memcpy(hq_out + r * I, hq, (size_t)I);
    if (hs_out) memcpy(hs_out + r * (I / 16), hs, (size_t)(I / 16));
    const int8_t* hq_use = hq_in ? hq_in + r * I : hq;
    const uint8_t* hs_use = hs_in ? hs_in + r * (I / 16) : hs;
    for (int64_t n = 0; n < H; ++n) {
      const int64_t rw = e * H + n;
      y[r * H + n] = G2 * g_mid * nvfp4_a8_dot(hq_use, hs_use, w2q + rw * (I / 2), w2s + rw * (I / 16), kb0, kb1);
    }
    free(hv);
    free(hq);
    free(hs);
  }
}

/* ------------------------------------------------------------------ */
/* Optional shared-expert gate.  The pages print no gate on the shared expert
 * (they list it as always on [R3][A1]); the variant read here is the plainest
 * one: a per-token scalar g_t = sigmoid(z_t) with z_t = sum_h x[t][h] * wg[h]
 * (wg an FP32 vector of length H), the sum in FP64 over exact products and
 * the sigmoid 1 / (1 + exp(-z)) in FP64, rounded to FP32.  The shared
 * expert's output row of token t is multiplied by g_t.                     */
void orc_shared_gate(const uint16_t* x, const float* wg, int64_t T, int64_t H, float* g) {
  for (int64_t t = 0; t < T; ++t) {
    double z = 0.0;
    for (int64_t h = 0; h < H; ++h) z += bf16_value(x[t * H + h]) * (double)wg[h];
    g[t] = (float)(1.0 / (1.0 + exp(-z)));
  }
}

/* orc_round_bf16 over an array. */
void orc_round_bf16_array(const double* v, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_round_bf16(v[i]);
}

/* ------------------------------------------------------------------ */
/* Stack composition (a reading; the pages chain 48 MoE layers, Richland
 * article "What shipped", but print no block structure): before each MoE
 * layer the residual stream is RMS-normalised without a learned weight,
 * n = RNE_BF16( x / sqrt(mean_h x^2 + eps) ), everything in FP64; the layer's
 * output is added back to x in its combine.                              */
void orc_rms_norm(const uint16_t* x, int64_t T, int64_t H, double eps, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t h = 0; h < H; ++h) {
      uint32_t u = (uint32_t)x[t * H + h] << 16;
      float f;
      memcpy(&f, &u, 4);
      ss += (double)f * (double)f;
    }
    const double inv = 1.0 / sqrt(ss / (double)H + eps);
    for (int64_t h = 0; h < H; ++h) {
      uint32_t u = (uint32_t)x[t * H + h] << 16;
      float f;
      memcpy(&f, &u, 4);
      out[t * H + h] = orc_round_bf16((double)f * inv);
    }
  }
}

/*
 * Seeded synthetic inputs for the routed NVFP4 W4A4 mixture-of-experts layer.
 *
 * This module serves both the FP64 oracle and the GPU path and contains none
 * of the layer's own arithmetic (routing, activation quantization, expert
 * products, combine).  It only draws random numbers and turns FP64 weight
 * draws into a packed NVFP4 checkpoint, the form in which the layer receives
 * its expert weights (capy-flash README, "Model weights": the NVFP4 experts
 * come from NVIDIA's checkpoint unchanged, with no second quantization pass;
 * the layer itself never encodes a weight).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, 2014) used as a
 * counter-based generator.  Output i of stream `key` is the SplitMix64
 * finaliser applied to key + (i+1)*0x9E3779B97F4A7C15, i.e. the (i+1)-th
 * output of a SplitMix64 seeded with `key`.  Uniforms take the top 53 bits;
 * normals of the hidden states and router rows come from the Box-Muller
 * transform on the pair (2j, 2j+1): element 2j is the cosine branch and
 * element 2j+1 the sine branch.  Expert weights (billions of draws per layer)
 * use the ziggurat method of Marsaglia and Tsang (2000, 128 strips): normal n
 * of stream `key` reads its own counter stream seeded by output n of `key`,
 * so rejections never shift other elements.  Every element is a pure function
 * of (key, index): the result does not depend on the number of threads.
 *
 * Weight encoding (the synthetic checkpoint): per expert and per packed
 * tensor, G = fl32(amax / (6*448)); per 16-element block the UE4M3 scale code
 * nearest to amax_block / (6*G) (ties to the even code, saturating at 448);
 * each element the E2M1 code nearest to |w| / (scale*G) (ties to the even
 * code, saturating at 6, sign = sign of w).  "Nearest" is decided on the
 * exact quotient: |w| is compared with the grid midpoints times scale*G,
 * products that are exact in FP64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t gen_splitmix64(uint64_t key, uint64_t i) { return sm_mix(key + (i + 1) * GOLDEN); }

/* uniform in (0, 1): never 0, so log() in Box-Muller is finite */
static inline double u01(uint64_t key, uint64_t i) {
  return ((double)(gen_splitmix64(key, i) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

double gen_normal_at(uint64_t key, uint64_t j) {
  uint64_t p = j >> 1;
  double u1 = u01(key, 2 * p), u2 = u01(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (j & 1) ? r * sin(a) : r * cos(a);
}

/* ---- ziggurat normals (Marsaglia and Tsang, 2000) ----
 * 128 strips of equal area V under f(x) = exp(-x^2/2): strip 0 is the base
 * rectangle of width V/f(R) (its part beyond R is the tail), strip i >= 1 the
 * rectangle between heights f(zx[i]) and f(zx[i+1]) with zx[1] = R,
 * zx[i+1] = f^-1(f(zx[i]) + V/zx[i]) and zx[128] = 0.  A draw picks a strip
 * and a point z = U * zx[i]; inside the strip's inner rectangle (z <
 * zx[i+1]) it is accepted at once, otherwise the wedge (or, for strip 0, the
 * tail beyond R) is sampled exactly, and a rejection starts over. */
#define ZIG_R 3.442619855899
#define ZIG_V 9.91256303526217e-3
static double zx[129], zf[129];
static int zig_ready = 0;

static void build_ziggurat(void) {
  if (zig_ready) return;
  zx[0] = ZIG_V / exp(-0.5 * ZIG_R * ZIG_R);
  zx[1] = ZIG_R;
  for (int i = 1; i < 127; ++i) zx[i + 1] = sqrt(-2.0 * log(exp(-0.5 * zx[i] * zx[i]) + ZIG_V / zx[i]));
  zx[128] = 0.0;
  for (int i = 0; i <= 128; ++i) zf[i] = exp(-0.5 * zx[i] * zx[i]);
  zig_ready = 1;
}

/* uniform in (0, 1) from 53 bits */
static inline double u53(uint64_t r) { return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static double zig_normal(uint64_t key, uint64_t n) {
  const uint64_t sub = sm_mix(key + (n + 1) * GOLDEN); /* seed of this element's own stream */
  uint64_t r = sub, j = 0;
  for (;;) {
    const int i = (int)(r & 127u);
    const double sgn = (r & 128u) ? -1.0 : 1.0;
    const double z = u53(r) * zx[i];
    if (z < zx[i + 1]) return sgn * z;
    if (i == 0) { /* tail beyond R */
      for (;;) {
        const double a = -log(u53(gen_splitmix64(sub, j++))) / ZIG_R;
        const double b = -log(u53(gen_splitmix64(sub, j++)));
        if (b + b > a * a) return sgn * (ZIG_R + a);
      }
    }
    const double y = zf[i] + u53(gen_splitmix64(sub, j++)) * (zf[i + 1] - zf[i]);
    if (y < exp(-0.5 * z * z)) return sgn * z;
    r = gen_splitmix64(sub, j++);
  }
}

double gen_ziggurat_at(uint64_t key, uint64_t n) {
  build_ziggurat();
  return zig_normal(key, n);
}

/* IEEE round-to-nearest-even FP32 -> BF16 (finite inputs) */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[i] = RNE_BF16(fl32(scale * N(0,1)_i)), i in [0, n) */
void gen_normal_bf16(uint64_t key, double scale, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(scale * gen_normal_at(key, (uint64_t)i)));
}

/* out[r*cols + c] = fl32(row_scale[r] * N(0,1)_{r*cols+c}) */
void gen_normal_f32_rows(uint64_t key, const double* row_scale, int64_t rows, int64_t cols, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c)
      out[r * cols + c] = (float)(row_scale[r] * gen_normal_at(key, (uint64_t)(r * cols + c)));
}

/* ---- the two NVFP4 grids, enumerated from their bit layouts ---- */
static double e2m1_mag[8];   /* code 0..7: sign bit clear */
static double ue4m3_val[127]; /* codes 0..126 (0x7F is NaN) */
static int grids_ready = 0;

static void build_grids(void) {
  if (grids_ready) return;
  for (int c = 0; c < 8; ++c) {
    int e = (c >> 1) & 3, m = c & 1;
    e2m1_mag[c] = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  }
  for (int c = 0; c < 127; ++c) {
    int e = (c >> 3) & 15, m = c & 7;
    ue4m3_val[c] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  }
  grids_ready = 1;
}

/* UE4M3 code nearest to amax / g6 (ties to the even code, saturating at 448),
 * decided on the exact quotient: amax is compared with g6 times the midpoints
 * of the grid (each midpoint has <= 5 significant bits, g6 = 6 * fl32 value:
 * the products are exact in FP64). */
static int scale_code_exact(double amax, double g6) {
  int lo = 0, hi = 126; /* answer: number of midpoints below amax, in [lo, hi] */
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (0.5 * (ue4m3_val[mid] + ue4m3_val[mid + 1]) * g6 < amax) lo = mid + 1; else hi = mid;
  }
  if (lo < 126 && 0.5 * (ue4m3_val[lo] + ue4m3_val[lo + 1]) * g6 == amax && ((lo + 1) & 1) == 0) lo += 1;
  return lo;
}

/* E2M1 magnitude code nearest to a / s (a >= 0, s > 0), ties to the even
 * code, saturating at 6: a against the midpoints times s (exact products). */
static inline int elem_mag_exact(double a, double s) {
  return (a > 0.25 * s) + (a >= 0.75 * s) + (a > 1.25 * s) + (a >= 1.75 * s) + (a > 2.5 * s) + (a >= 3.5 * s) +
         (a > 5.0 * s);
}

/*
 * Draw an [n_exp][N][K] tensor of N(0, sigma^2) weights and pack it as NVFP4:
 *   codes  [n_exp][N][K/2]  (element 2i in the low nibble of byte i)
 *   scales [n_exp][N][K/16] (UE4M3 codes)
 *   gscale [n_exp]          (FP32)
 * Element (e, n, kk) uses normal index (e*N + n)*K + kk of stream `key`.
 */
int gen_nvfp4_bank(uint64_t key, double sigma, int64_t n_exp, int64_t N, int64_t K, uint8_t* codes,
                   uint8_t* scales, float* gscale) {
  if (K % 16 != 0) return -1;
  build_grids();
  build_ziggurat();
  int bad = 0;
#pragma omp parallel
  {
    /* one staging buffer per thread, reused across experts */
    double* w = (double*)malloc(sizeof(double) * (size_t)(N * K));
    if (!w) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t e = 0; e < n_exp; ++e) {
      if (!w) continue;
      const int64_t base = e * N * K;
      double amax = 0.0;
      for (int64_t i = 0; i < N * K; ++i) {
        w[i] = sigma * zig_normal(key, (uint64_t)(base + i));
        if (fabs(w[i]) > amax) amax = fabs(w[i]);
      }
      const float G = (float)(amax / (6.0 * 448.0));
      gscale[e] = G;
      const double g6 = 6.0 * (double)G;
      for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < K / 16; ++b) {
          const double* wb = w + n * K + b * 16;
          double bmax = 0.0;
          for (int j = 0; j < 16; ++j)
            if (fabs(wb[j]) > bmax) bmax = fabs(wb[j]);
          const int sc = G > 0.0f ? scale_code_exact(bmax, g6) : 0;
          scales[(e * N + n) * (K / 16) + b] = (uint8_t)sc;
          const double sv = ue4m3_val[sc] * (double)G;
          uint8_t* dst = codes + (e * N + n) * (K / 2) + b * 8;
          for (int j = 0; j < 16; j += 2) {
            int nib[2];
            for (int h = 0; h < 2; ++h) {
              const double v = wb[j + h];
              nib[h] = (sv > 0.0 ? elem_mag_exact(fabs(v), sv) : 0) | (signbit(v) ? 8 : 0);
            }
            dst[j / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
          }
        }
      }
    }
    free(w);
  }
  if (bad) return -2;
  return 0;
}

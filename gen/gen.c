/*
 * Seeded synthetic inputs for the routed NVFP4 W4A4 mixture-of-experts layer.
 *
 * This module serves both the FP64 oracle and the GPU path and contains none
 * of the layer's own arithmetic (routing, activation quantization, expert
 * products, combine).  It only draws random numbers and turns FP64 weight
 * draws into a packed NVFP4 checkpoint, the form in which the layer receives
 * its expert weights (capy-flash README, "Model weights": the NVFP4 experts
 * are used as published, not re-quantized; the layer itself never encodes a
 * weight).
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, 2014) used as a
 * counter-based generator.  Output i of stream `key` is the SplitMix64
 * finaliser applied to key + (i+1)*0x9E3779B97F4A7C15, i.e. the (i+1)-th
 * output of a SplitMix64 seeded with `key`.  Uniforms take the top 53 bits;
 * normals come from the Box-Muller transform on the pair (2j, 2j+1): element
 * 2j is the cosine branch and element 2j+1 the sine branch.  Every element is
 * a pure function of (key, index), so the result does not depend on the
 * number of OpenMP threads.
 *
 * Weight encoding (the synthetic checkpoint): per expert and per packed
 * tensor, G = fl32(amax / (6*448)); per 16-element block the UE4M3 scale code
 * nearest to amax_block / (6*G) (ties to the even code, saturating at 448);
 * each element the E2M1 code nearest to w / (scale*G) (ties to the even code,
 * saturating at 6, sign = sign of w).  "Nearest" is taken on the FP64
 * quotient by scanning the whole grid, which is slow but leaves nothing to
 * interpret.
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

/* normals 2p and 2p+1 of the stream at once (the same values as gen_normal_at) */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
  double u1 = u01(key, 2 * p), u2 = u01(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(a);
  *z1 = r * sin(a);
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

/* nearest grid point, ties to the even code; v >= 0; grid strictly ascending.
 * The distance to the grid is unimodal, so the nearest point is one of the two
 * neighbours of v, found by bisection. */
static int nearest_code(const double* grid, int n, double v) {
  if (v >= grid[n - 1]) return n - 1;
  int lo = 0, hi = n - 1; /* grid[lo] <= v < grid[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (grid[mid] <= v) lo = mid; else hi = mid;
  }
  double dl = v - grid[lo], dh = grid[hi] - v;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) ? hi : lo;
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
      for (int64_t i = 0; i < N * K; i += 2) { /* base and N*K are even */
        double z0, z1;
        normal_pair(key, (uint64_t)(base + i) >> 1, &z0, &z1);
        w[i] = sigma * z0;
        w[i + 1] = sigma * z1;
        if (fabs(w[i]) > amax) amax = fabs(w[i]);
        if (fabs(w[i + 1]) > amax) amax = fabs(w[i + 1]);
      }
      float G = (float)(amax / (6.0 * 448.0));
      gscale[e] = G;
      for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < K / 16; ++b) {
          const double* wb = w + n * K + b * 16;
          double bmax = 0.0;
          for (int j = 0; j < 16; ++j)
            if (fabs(wb[j]) > bmax) bmax = fabs(wb[j]);
          int sc = G > 0.0f ? nearest_code(ue4m3_val, 127, bmax / (6.0 * (double)G)) : 0;
          scales[(e * N + n) * (K / 16) + b] = (uint8_t)sc;
          double s = ue4m3_val[sc] * (double)G;
          for (int j = 0; j < 16; j += 2) {
            uint8_t nib[2];
            for (int h = 0; h < 2; ++h) {
              double v = wb[j + h];
              int mag = s > 0.0 ? nearest_code(e2m1_mag, 8, fabs(v) / s) : 0;
              nib[h] = (uint8_t)(mag | (signbit(v) ? 8 : 0));
            }
            codes[(e * N + n) * (K / 2) + (b * 16 + j) / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
          }
        }
      }
    }
    free(w);
  }
  if (bad) return -2;
  return 0;
}

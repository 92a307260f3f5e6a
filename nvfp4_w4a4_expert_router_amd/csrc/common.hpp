// Device helpers for the NVFP4 W4A4 MoE layer on gfx950: format decode,
// the exact (comparison-based) A4 encoder, BF16 rounding, wave utilities and
// the parameter blocks shared by the launchers.
//
// NVFP4 (Richland article, "What shipped"): E2M1 element codes, UE4M3 block
// scales, FP32 per-expert scale.  A4 (capy-flash README v0.5.4, "What it
// does" / "Serve"): activations encoded the same way before every expert.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- formats
// UE4M3 code (0..126) -> value: exponent field bits 6..3 (bias 7), mantissa
// bits 2..0; exponent 0 is subnormal m * 2^-9.
__device__ __forceinline__ float ue4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude code (0..7) -> value {0, .5, 1, 1.5, 2, 3, 4, 6}.
__device__ __forceinline__ float e2m1_mag_value(uint32_t m) {
  const uint32_t bits = m == 0 ? 0u : m == 1 ? 0x3F000000u : ((((m >> 1) + 126u) << 23) | ((m & 1u) << 22));
  return __uint_as_float(bits);
}

// E2M1 code (0..15) -> signed value.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const float v = e2m1_mag_value(c & 7u);
  return (c & 8u) ? -v : v;
}

// 6*g times the midpoint between UE4M3 codes c and c+1.  Midpoints have at
// most 5 significant bits; with g a power of two the product is exact.
__device__ __forceinline__ float scale_threshold(int c, float g6) {
  return (0.5f * (ue4m3_value((uint32_t)c) + ue4m3_value((uint32_t)c + 1u))) * g6;
}

// Block scale code = round-to-nearest-even of amax/(6g) on the UE4M3 grid,
// saturating at 448 (code 126).  Decided by exact comparisons: the code is the
// number of thresholds below amax, plus one on an exact tie whose upper
// neighbour is the even code.
__device__ __forceinline__ uint32_t scale_code(float amax, float g6) {
  int pos = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1)
    if (pos + step <= 126 && scale_threshold(pos + step - 1, g6) < amax) pos += step;
  if (pos < 126 && scale_threshold(pos, g6) == amax && ((pos + 1) & 1) == 0) pos += 1;
  return (uint32_t)pos;
}

// Element code = round-to-nearest-even of |v|/s on the E2M1 grid, saturating
// at 6; sign bit = sign of v.  Thresholds t*s are exact (t has <= 3
// significant bits, s <= 4).  Ties at .25, 1.25, 2.5, 5 stay on the lower
// (even) code, ties at .75, 1.75, 3.5 go up to the even code.
__device__ __forceinline__ uint32_t elem_code(float v, float s) {
  const float a = fabsf(v);
  uint32_t mag = 0;
  if (s > 0.0f)
    mag = (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) + (uint32_t)(a > 1.25f * s) +
          (uint32_t)(a >= 1.75f * s) + (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) +
          (uint32_t)(a > 5.0f * s);
  return mag | (__float_as_uint(v) >> 31 << 3);
}

// BF16 bits -> FP32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// FP32 -> BF16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// The s-th expert (0-based, ascending id) with a nonzero count in off[0..E].
// Called by a whole wave; every lane gets the same answer.  Returns -1 if
// fewer than s+1 experts are active.
__device__ __forceinline__ int find_active_expert(const int32_t* __restrict__ off, int E, int s, int* row0,
                                                  int* cnt) {
  const int lane = lane_id();
  int seen = 0;
  for (int base = 0; base < E; base += kWave) {
    const int e = base + lane;
    const int c = e < E ? off[e + 1] - off[e] : 0;
    const uint64_t m = __ballot(c > 0);
    const int n = __popcll(m);
    if (seen + n > s) {
      const int want = s - seen;
      const int pre = __popcll(m & ((1ull << lane) - 1ull));
      const uint64_t hm = __ballot(c > 0 && pre == want);
      const int ee = base + (__ffsll((long long)hm) - 1);
      *row0 = off[ee];
      *cnt = off[ee + 1] - off[ee];
      return ee;
    }
    seen += n;
  }
  return -1;
}

// ---------------------------------------------------------------- launch parameter blocks
struct FfnParams {
  int H, I, E, k, T, has_shared;
  int n_routed_slots;  // grid slots for routed experts (min(E, T*k))
  const int32_t* off;
  const int32_t* row2pair;
  const half_t* xh;  // [T][H] dequantized A4(x) without a_gscale_in
  moe_nvfp4_bank w13, w2, sh13, sh2;
  float g_in, g_mid;
  half_t* hh;  // [R][I] dequantized A4(h) without a_gscale_mid; R = T*k (+ T)
  float* h_dbg;
  uint8_t* hq_dbg;
  uint8_t* hs_dbg;
  float* y_rows;
  float* y_shared;
};

// launchers (one translation unit each)
hipError_t launch_quant_act(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, uint8_t* codes,
                            uint8_t* scales, half_t* deq, hipStream_t s);
size_t route_ws_bytes(int64_t T, int E);
hipError_t launch_route(const uint16_t* x, const float* W, int64_t T, int H, int E, int k, const float* logits_in,
                        int32_t* idx, float* w, void* ws, hipStream_t s);
size_t permute_ws_bytes(int64_t T, int E);
hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, int32_t* off, int32_t* r2p, int32_t* p2r,
                          void* ws, hipStream_t s);
hipError_t launch_ffn_gemv(const FfnParams& p, hipStream_t s);
hipError_t launch_combine(int64_t T, int H, int k, const float* y_rows, const float* y_shared, const int32_t* p2r,
                          const float* w, const uint16_t* residual, uint16_t* out, hipStream_t s);

}  // namespace moe

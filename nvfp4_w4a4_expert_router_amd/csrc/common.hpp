// Device helpers for the NVFP4 W4A4 MoE layer on gfx950: format decode,
// the exact (comparison-based) A4 encoder, BF16 rounding, wave utilities and
// the parameter blocks shared by the launchers.
//
// NVFP4 (Richland article, "What shipped"): E2M1 element codes, UE4M3 block
// scales, FP32 per-expert scale.  A4 (capy-flash README v0.5.4, "What it
// does" / "Serve"): activations encoded the same way before every expert.
#pragma once
#include <hip/hip_ext.h>
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
// Written without a branch as 2^(max(e,1) - 10) * (8 [e > 0] + m), exact.
__device__ __forceinline__ float ue4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t eb = e > 1u ? e : 1u;
  return __uint_as_float((eb + 117u) << 23) * (float)((e > 0u ? 8u : 0u) + m);
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
// neighbour is the even code.  The thresholds are non-decreasing in c, so the
// count is c exactly when t(c-1) < amax <= t(c).
//
// scale_code_search finds the count by binary search (7 threshold products);
// scale_code guesses it from amax/(6g) rounded on the UE4M3 grid and keeps the
// guess when the two bracketing thresholds confirm it.  The guess can only be
// wrong for amax within a few FP32 ulps of a threshold (or not a number); those
// lanes take the search.
__device__ __forceinline__ uint32_t scale_code_search(float amax, float g6) {
  int pos = 0;
#pragma unroll
  for (int step = 64; step >= 1; step >>= 1)
    if (pos + step <= 126 && scale_threshold(pos + step - 1, g6) < amax) pos += step;
  if (pos < 126 && scale_threshold(pos, g6) == amax && ((pos + 1) & 1) == 0) pos += 1;
  return (uint32_t)pos;
}

__device__ __forceinline__ uint32_t scale_code(float amax, float g6) {
  const float y = amax * __builtin_amdgcn_rcpf(g6);
  // normal range: exponent and three mantissa bits of y, rounded half up
  // (bits >> 20 = 8 * biased exponent + mantissa; UE4M3's bias is 120 below FP32's)
  const int cn = (int)((__float_as_uint(y) + 0x80000u) >> 20) - 960;
  // subnormal range (y < 2^-6): y in units of 2^-9
  const int cs = (int)(y * 512.0f + 0.5f);
  int c = y < 0.015625f ? cs : cn;
  c = c < 0 ? 0 : c > 126 ? 126 : c;
  const float t_lo = c > 0 ? scale_threshold(c - 1, g6) : -1.0f;
  const float t_hi = c < 126 ? scale_threshold(c, g6) : __builtin_inff();
  if (!(t_lo < amax && amax <= t_hi)) return scale_code_search(amax, g6);
  return (uint32_t)(c + (c < 126 && t_hi == amax && (c & 1) != 0 ? 1 : 0));
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

// elem_code for a block whose scale is known: s > 0, or +inf for scale code 0
// (then every magnitude code is 0).  The same seven thresholds and tie rules as
// elem_code, searched in three exact comparisons: 1.75s (>=), then 3.5s or .75s
// (>=), then 5s, 2.5s, 1.25s or .25s (>).
__device__ __forceinline__ uint32_t elem_code_s(float v, float s) {
  const float a = fabsf(v);
  const bool c4 = a >= 1.75f * s;
  const bool c2 = a >= (c4 ? 3.5f : 0.75f) * s;
  const bool c1 = a > (c4 ? (c2 ? 5.0f : 2.5f) : (c2 ? 1.25f : 0.25f)) * s;
  const uint32_t mag = (c4 ? 4u : 0u) + (c2 ? 2u : 0u) + (c1 ? 1u : 0u);
  return mag | (__float_as_uint(v) >> 31 << 3);
}

// elem_code_s with the block's seven threshold products formed once, for a
// block whose values are encoded many at a time (the same FP32 products, so
// the same codes).
struct E2M1Thresholds {
  float t025, t075, t125, t175, t25, t35, t5;
};
__device__ __forceinline__ E2M1Thresholds e2m1_thresholds(float s) {
  return {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
}
__device__ __forceinline__ uint32_t elem_code_t(float v, const E2M1Thresholds& T) {
  const float a = fabsf(v);
  const bool c4 = a >= T.t175;
  const bool c2 = a >= (c4 ? T.t35 : T.t075);
  const bool c1 = a > (c4 ? (c2 ? T.t5 : T.t25) : (c2 ? T.t125 : T.t025));
  const uint32_t mag = (c4 ? 4u : 0u) + (c2 ? 2u : 0u) + (c1 ? 1u : 0u);
  return mag | (__float_as_uint(v) >> 31 << 3);
}

// ---------------------------------------------------------------- A8 (the W4A8 variant)
// A8 keeps A4's 16-element blocks and UE4M3 block scale, chosen as
// RNE(amax / (127 g)) (scale_code with 127 g in place of 6 g: the thresholds
// 127 g x midpoint have at most 12 significant bits, exact in FP32), and
// encodes each element as q = RNE(|v| / s) on the integers, saturating at 127,
// with the sign of v (two's complement INT8; zero carries no sign).
//
// int8_code: a first guess from |v| times the reciprocal of s, then the exact
// thresholds (m +- 1/2) s (at most 8 + 4 significant bits, exact in FP32)
// move it to the rounding of the exact quotient, ties to the even integer.  The
// guess is off by at most one.  s = +inf (scale code 0) gives 0.
__device__ __forceinline__ int int8_code(float v, float s) {
  const float a = fabsf(v);
  int m = (int)__builtin_rintf(a * __builtin_amdgcn_rcpf(s));
  m = m > 127 ? 127 : m;
  if (m < 127) {
    const float up = ((float)m + 0.5f) * s;
    if (a > up || (a == up && (m & 1))) ++m;
  }
  if (m > 0) {
    const float dn = ((float)m - 0.5f) * s;
    if (a < dn || (a == dn && (m & 1))) --m;
  }
  return (__float_as_uint(v) >> 31) ? -m : m;
}

// 32 A8 codes (32 B: two 16-element blocks) times their UE4M3 scales (sc2: low
// byte = first block) -> 32 FP16 values at dst (16-byte aligned).  Each value
// q * s has at most 7 + 4 significant bits and magnitude at most 127 * 448:
// exact in FP16.
__device__ __forceinline__ void decode32_a8_fp16(uint4 q0, uint4 q1, uint32_t sc2, half_t* dst) {
  const float s0 = ue4m3_value(sc2 & 0xFFu), s1 = ue4m3_value((sc2 >> 8) & 0xFFu);
  const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  half8_t out[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float s = d < 2 ? s0 : s1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = w[2 * d + i / 4];
      const int q = (int)(int8_t)(uint8_t)(word >> (8 * (i & 3)));
      out[d][i] = (half_t)((float)q * s);
    }
  }
  half8_t* o = reinterpret_cast<half8_t*>(dst);
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = out[d];
}

// Two E2M1 codes (byte kByte of w, low nibble first) -> two exact FP16 values
template <int kByte>
__device__ __forceinline__ half2_t fp4x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, kByte);
}

// Two UE4M3 codes (low byte first) -> their values as FP16, exactly.  A code
// c = e:m (4 + 3 bits) placed at bit 7 of an FP16 word has the same exponent and
// mantissa fields, i.e. the value 2^(e-15)(1 + m/8) (or m 2^-17 when e = 0); FP16's
// bias exceeds UE4M3's by 8, so one multiply by 2^8 gives 2^(e-7)(1 + m/8) and
// m 2^-9 (codes up to 126: at most 448).
__device__ __forceinline__ half2_t ue4m3x2_to_half2(uint32_t sc2) {
  const uint32_t w = ((sc2 & 0xFFu) << 7) | ((sc2 & 0xFF00u) << 15);
  return __builtin_bit_cast(half2_t, w) * half2_t{(half_t)256.0f, (half_t)256.0f};
}

// 32 codes (16 B: two 16-element blocks) times their UE4M3 scales (sc2: low
// byte = first block) -> 32 FP16 values at dst (16-byte aligned).  Each
// product has at most 6 significant bits and lies in [2^-10, 2688]: exact.
__device__ __forceinline__ void decode32_fp16(uint4 q, uint32_t sc2, half_t* dst) {
  const half2_t sv = ue4m3x2_to_half2(sc2);
  const half2_t S0 = half2_t{sv[0], sv[0]}, S1 = half2_t{sv[1], sv[1]};
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  half8_t out[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const half2_t S = d < 2 ? S0 : S1;
    const half2_t a = fp4x2<0>(w[d]) * S, b = fp4x2<1>(w[d]) * S, c = fp4x2<2>(w[d]) * S, e = fp4x2<3>(w[d]) * S;
    out[d] = half8_t{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
  }
  half8_t* o = reinterpret_cast<half8_t*>(dst);
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = out[d];
}

// BF16 bits -> FP32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// FP32 -> BF16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// FP64 -> BF16 bits, round to nearest even (finite inputs; BF16 subnormal
// results go through FP32, where they are exact after this rounding)
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int e = (int)((u >> 52) & 0x7FF) - 1023;
  if (v == 0.0) return (uint16_t)sign;
  if (e < -126 || e > 127) return f32_to_bf16_rne((float)v);
  const unsigned long long m = u & 0xFFFFFFFFFFFFFull;
  unsigned long long q = m >> 45;                        // 7 mantissa bits
  const unsigned long long rest = m & ((1ull << 45) - 1);
  const unsigned long long half = 1ull << 44;
  uint32_t be = (uint32_t)(e + 127);
  if (rest > half || (rest == half && (q & 1ull))) {
    if (++q == 128ull) {
      q = 0ull;
      ++be;
    }
  }
  return (uint16_t)(sign | (be << 7) | (uint32_t)q);
}


// silu(z) = z * sigmoid(z) with the hardware exp2 and reciprocal (a few ulp; far
// inside the FP32 accumulation error of the sums that produce z).  Large negative
// z gives exp = inf and a signed zero, keeping the sign of the exact value.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// SwiGLU of raw sums: silu(G a) * (G b) for a common factor G > 0, as
// (a b) / ((1 + 2^(-G log2(e) a)) / G^2), with c = -G log2(e) and inv_g2 = 1 / G^2
// formed once per tile (the same few-ulp accuracy as silu).
__device__ __forceinline__ float swiglu_scaled(float a, float b, float c, float inv_g2) {
  const float e = __builtin_amdgcn_exp2f(c * a);
  return (a * b) * __builtin_amdgcn_rcpf(fmaf(e, inv_g2, inv_g2));
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes): 32-bit per-lane offsets, a
// wave-uniform scalar offset, and reads past the end return zero.  Word 3 is
// the gfx9-family raw-buffer configuration (32-bit data format).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// the same marked non-temporal (streamed weights read once per call: they
// should not displace data that is read again, such as the router rows)
__device__ __forceinline__ uint4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 4-byte store through a buffer resource (offsets at or past the resource's
// size are dropped: the offset is all in voff, so the range check covers it),
// with the non-temporal cache policy (bit 1 of the policy operand on this chip
// family: `nt`): for output written once and read much later, so it does not
// displace operands that are being reused in L2.
__device__ __forceinline__ void buffer_store4_nt(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, 0, 2);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;  // LDS destination of buffer-to-LDS loads
__device__ __forceinline__ void buffer_store8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}

// The values of lanes l % 32 and l % 32 + 32, in an order that depends only on
// the direction of v_permlane32_swap (one half of the wave exchanged between
// two registers; with the same value in both, one result holds the lower half's
// value in every lane and the other the upper half's).  Callers use the pair
// symmetrically or tag the values with their half.
__device__ __forceinline__ void lane_pair(uint32_t v, uint32_t* r0, uint32_t* r1) {
  const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  *r0 = p[0];
  *r1 = p[1];
}

// Workgroup b of the first n -> logical tile.  Workgroups are handed out round
// robin over the chip's 8 XCDs (b % 8), each with its own L2; XCD x gets one
// contiguous run of logical tiles, so tiles that are neighbours in logical
// order (sharing operands) run in the same L2.
__device__ __forceinline__ int xcd_tile(int b, int n) {
  const int x = b & 7, i = b >> 3, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + i;
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Wave-wide reductions and scans through DPP moves (no LDS round trips).
// Sum: quad_perm(1,0,3,2), quad_perm(2,3,0,1), row_half_mirror, row_mirror
// give 16-lane row sums in every lane; row_bcast:15 into rows 1 and 3, then
// row_bcast:31 into rows 2 and 3, leave the wave total in lane 63 (disabled
// rows add 0).  The order of the additions is fixed: deterministic.
template <int kCtrl, int kRowMask, bool kZeroOld>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_update_dpp(kZeroOld ? 0 : v, v, kCtrl, kRowMask, 0xF, true);
}

// max of |v| over each row of 16 lanes, returned in every lane of the row
// (non-negative floats order like their bit patterns)
__device__ __forceinline__ float row16_absmax(float v) {
  uint32_t u = __float_as_uint(v) & 0x7FFFFFFFu;
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));  // row_half_mirror
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));  // row_mirror
  return __uint_as_float(u);
}

// compile-time loop: f(IntC<0>{}) .. f(IntC<kN - 1>{})
template <int kV>
struct IntC {
  static constexpr int value = kV;
};
template <int kI, int kN, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (kI < kN) {
    f(IntC<kI>{});
    static_for<kI + 1, kN>(f);
  }
}

template <int kCtrl, int kRowMask, bool kZeroOld>
__device__ __forceinline__ double dpp_mov_f64(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const int lo = dpp_mov<kCtrl, kRowMask, kZeroOld>((int)(u & 0xFFFFFFFFull));
  const int hi = dpp_mov<kCtrl, kRowMask, kZeroOld>((int)(u >> 32));
  return __longlong_as_double(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// FP64 sum over the wave, returned in every lane
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_mov_f64<0xB1, 0xF, false>(v);
  v += dpp_mov_f64<0x4E, 0xF, false>(v);
  v += dpp_mov_f64<0x141, 0xF, false>(v);
  v += dpp_mov_f64<0x140, 0xF, false>(v);
  v += dpp_mov_f64<0x142, 0xA, true>(v);
  v += dpp_mov_f64<0x143, 0xC, true>(v);
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane((int)(u & 0xFFFFFFFFull), 63);
  const unsigned hi = __builtin_amdgcn_readlane((int)(u >> 32), 63);
  return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

// Inclusive prefix sum over the wave: row_shr:1, 2, 4, 8 within 16-lane rows
// (lanes without a source add 0), then the row totals through row_bcast:15 and
// row_bcast:31.
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += dpp_mov<0x111, 0xF, true>(v);
  v += dpp_mov<0x112, 0xF, true>(v);
  v += dpp_mov<0x114, 0xF, true>(v);
  v += dpp_mov<0x118, 0xF, true>(v);
  v += dpp_mov<0x142, 0xA, true>(v);
  v += dpp_mov<0x143, 0xC, true>(v);
  return v;
}

// Top k (k <= 32) of up to 512 values held 8 per lane (value v[j], id[j] < 1024;
// unused entries -inf), ordered by (value descending, id ascending).  Each entry
// is ranked by one 64-bit key: the double's bits mapped to an unsigned order
// with its lowest 10 bits replaced by 1023 - id, so a larger key ranks first
// (values within 2^-42 relative of each other rank by id: far inside the
// near-tie margin of a reordered FP64 sum).  tau = the k-th best of the 64
// lane heads (the best entry of each lane).  The k best heads are all at least
// tau, so every entry of the true top k is at least tau: only the entries >= tau
// (~k in total) are ranked against each other.  Lane r < k receives the r-th
// entry.  The heads and the candidates go through LDS and every lane compares
// against all of them with broadcast reads, 16 in flight (a single wave has no
// other wave to hide latency behind).  S: this wave's LDS scratch.
constexpr int kTopkScratch = 512 + 32;
struct __attribute__((aligned(16))) TopkScratch {
  uint64_t key[kTopkScratch];
  double val[kTopkScratch];
};

__device__ __forceinline__ uint64_t rank_key(double v, int id) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint64_t u = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (u & ~0x3FFull) | (uint64_t)(1023 - (id & 1023));
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane((int)(u & 0xFFFFFFFFull), l);
  const unsigned hi = __builtin_amdgcn_readlane((int)(u >> 32), l);
  return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const unsigned lo = __builtin_amdgcn_readlane((int)(v & 0xFFFFFFFFull), l);
  const unsigned hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void wave_topk512(const double (&v)[8], const int (&id)[8], int k, TopkScratch& S,
                                             double* out_v, int* out_id) {
  const int lane = (int)(threadIdx.x & 63);
  uint64_t key[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) key[j] = rank_key(v[j], id[j]);
  // this lane's head
  uint64_t hk = key[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) hk = key[j] > hk ? key[j] : hk;
  // rank of this lane's head among the 64 heads
  S.key[lane] = hk;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int hr = 0;
  const uint4* kp = reinterpret_cast<const uint4*>(S.key);  // two keys per 16-byte read
#pragma unroll 8
  for (int q = 0; q < 32; ++q) {
    const uint4 pk = kp[q];
    hr += (((uint64_t)pk.y << 32) | pk.x) > hk;
    hr += (((uint64_t)pk.w << 32) | pk.z) > hk;
  }
  const uint64_t at = __ballot(hr == k - 1);
  const int L = __ffsll((long long)at) - 1;
  const uint64_t tau = readlane_u64(hk, L);
  // candidates: the entries not behind tau, compacted in lane order
  bool cand[8];
  int m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    cand[j] = key[j] >= tau;
    m += cand[j];
  }
  const int incl = wave_incl_scan_i32(m);
  const int nc = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - m;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // the heads are read
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (cand[j]) {
      S.key[pos] = key[j];
      S.val[pos] = v[j];
      ++pos;
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // rank every candidate among the candidates (blocks of 64 held in lanes);
  // rank r < k goes to result slot r
  for (int c0 = 0; c0 < nc; c0 += kWave) {
    const int c = c0 + lane;
    const uint64_t ck = c < nc ? S.key[c] : 0ull;
    const double cv = c < nc ? S.val[c] : 0.0;
    int r = 0;
    // 16 reads in flight per round; the last round's reads past nc stay inside
    // the scratch (nc <= 512 < kTopkScratch - 15) and are masked
    for (int q = 0; q < nc; q += 16)
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint64_t kq = S.key[q + u];
        r += (q + u < nc) & (kq > ck);
      }
    if (c < nc && r < k) {  // results after the 512 candidate slots
      S.key[512 + r] = ck;
      S.val[512 + r] = cv;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    *out_v = S.val[512 + lane];
    *out_id = 1023 - (int)(S.key[512 + lane] & 0x3FFull);
  }
}

__device__ __forceinline__ float topk_softmax_weight(double my_v, int k) {
  const int lane = (int)(threadIdx.x & 63);
  const unsigned long long u = __double_as_longlong(my_v);
  const double top = __longlong_as_double(
      ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(u >> 32), 0) << 32) |
      (unsigned)__builtin_amdgcn_readlane((int)(u & 0xFFFFFFFFull), 0));
  const double ex = lane < k ? exp(my_v - top) : 0.0;
  return (float)(ex / wave_sum_f64(ex));
}

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
// Fused decode routing (moe_layer_forward, T <= 4): FP64 logits and A4(x)
// from the router kernel; top k, softmax weights, permutation and slot table
// formed in the gate/up kernel's workgroups from those logits.
struct RouteDecodeParams {
  const uint16_t* x;   // [T][H] BF16
  const float* W;      // [E][H]
  int T, H, E, k;
  float g_in;
  double* logits;      // [T][E]
  uint8_t* xq;         // [T][H/2]
  uint8_t* xs;         // [T][H/16]
  int32_t* idx;
  float* w;
  int32_t* off;
  int32_t* r2p;
  int32_t* p2r;
  int4* slot_tab;      // [T*k]
  const float* wg;     // [H] shared-expert gate vector (null: no gate)
  float* gate;         // [T] gate values out (when wg is set)
  int act8;            // A8 codes of x (one INT8 per element, xq [T][H]) instead of A4
  int pre_norm;        // x is normed first (RMS norm, norm_eps) and the normed rows go to xn
  double norm_eps;
  uint16_t* xn;        // [T][H] BF16
};

struct FfnParams {
  int H, I, E, k, T, has_shared;
  int n_routed_slots;  // grid slots for routed experts (min(E, T*k))
  const int32_t* off;
  const int32_t* row2pair;
  const uint16_t* x;  // [T][H] BF16 hidden states
  const half_t* xh;   // [T][H] dequantized A4(x) without a_gscale_in (generic kernels)
  moe_nvfp4_bank w13, w2, sh13, sh2;
  moe_nvfp4_bank w13k, w2k, sh13k, sh2k;  // K-step-major copies (codes null: absent)
  float* y_tok;  // decode: optional copy of the routed output rows in token-major (pair) order
  float g_in, g_mid;
  half_t* hh;  // [R][I] dequantized A4(h) without a_gscale_mid; R = T*k (+ T)
  float* h_dbg;
  uint8_t* hq_dbg;
  uint8_t* hs_dbg;
  float* y_rows;
  float* y_shared;
  // decode kernels only: the shared expert takes one slot per token
  int shared_split;
  // fused decode call with the down projection and combine in one kernel:
  // routed slot s is pair s (token s / k, rank s % k) and h rows are indexed
  // by pair id (in the workspace; y_rows keep the permuted order)
  int pair_rows;
  // decode kernels: A4(x) codes [T][H/2] and scales [T][H/16]
  const uint8_t* xq;
  const uint8_t* xs;
  // decode kernels, fused path: routed slot s -> {expert (or -1), first row,
  // rows, tokens of the rows (one byte each)}; null: slots from expert_off
  const int4* slot_tab;
  // down projection over the elements [kc0, kc1) of I only (a K-split
  // partial; the full sum is kc0 = 0, kc1 = I).  Generic and matrix-core
  // kernels; kc0, kc1 multiples of 32 (of 64 on the matrix cores).
  int kc0, kc1;
  // optional gate of the shared expert: [T] FP32 per-token factors (null: none);
  // a shared output row is fl32(fl32(G * sum) * sh_gate[t])
  const float* sh_gate;
  // activation encoding: 0 = A4 (E2M1 codes, two per byte), 1 = A8 (INT8 codes,
  // one per byte) for x codes, h codes and their dumps
  int act8;
  // fused decode path (slot_tab set): the routing inputs and outputs; the
  // gate/up kernel's routed workgroups select from rq.logits and its last
  // workgroup publishes the outputs
  RouteDecodeParams rq;
  // fused decode path, down projection with the combine: residual [T][H] BF16
  // (nullable) and the layer output [T][H] BF16
  const uint16_t* residual;
  uint16_t* out;
};

// Launch with optional events that take the kernel's own start (e0) and end
// (e1) timestamps (the dispatch's, not the host's view of the stream); with
// neither it is a plain launch.
template <typename F, typename... Args>
inline hipError_t launch_timed(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, hipEvent_t e0,
                               hipEvent_t e1, Args... args) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}

// the event pair of a kernel that has nothing to do: both taken at this point
inline hipError_t record_idle(hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (e0 && hipEventRecord(e0, s) != hipSuccess) return hipErrorInvalidValue;
  if (e1 && hipEventRecord(e1, s) != hipSuccess) return hipErrorInvalidValue;
  return hipSuccess;
}

// launchers (one translation unit each); the event pairs (nullable) time the
// kernel named by each, as launch_timed does
hipError_t launch_quant_act(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, uint8_t* codes,
                            uint8_t* scales, half_t* deq, hipStream_t s, hipEvent_t e0 = nullptr,
                            hipEvent_t e1 = nullptr, int act_bits = 4);
size_t route_ws_bytes(int64_t T, int E, int H, int mode);
bool route_mode_supported(int H, int E, int mode);
hipError_t launch_pack_router(const float* W, int E, int H, uint16_t* pieces, hipStream_t s);
// per-token gate of the shared expert: gate[t] = fl32(sigmoid(x_t . wg)), the
// dot in FP64 over exact products
hipError_t launch_shared_gate(const uint16_t* x, const float* wg, int64_t T, int H, float* gate, hipStream_t s);
hipError_t launch_route(const uint16_t* x, const float* W, int64_t T, int H, int E, int k, const float* logits_in,
                        int32_t* idx, float* w, void* ws, int mode, const uint16_t* pieces, hipStream_t s);
size_t permute_ws_bytes(int64_t T, int E);
hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, int32_t* off, int32_t* r2p, int32_t* p2r,
                          void* ws, hipStream_t s);
hipError_t launch_ffn_gateup(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_ffn_down(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
// decode kernels (T <= 8, H <= 2048, I / 32 a power of two <= 64)
bool ffn_decode_supported(int H, int I, int64_t T);
hipError_t launch_gateup_decode(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
bool fused_decode_supported(int H, int I, int E, int k, int64_t T);
bool route_decode_supported(int H, int E, int k, int64_t T);
hipError_t launch_route_decode(const RouteDecodeParams& q, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_down_decode(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
bool down_combine_decode_supported(int H, int I, int k, int has_shared);
hipError_t launch_down_combine_decode(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
// matrix-core grouped GEMM (prefill): H % 128 == 0, I % 64 == 0, E <= 1000
bool ffn_mfma_supported(int H, int I, int E, int64_t T, int k);
size_t ffn_mfma_ws_bytes(int E, int64_t T, int k, int has_shared);
hipError_t launch_ffn_mfma(const FfnParams& p, int32_t* tile_start, hipStream_t s, hipEvent_t* ev);
hipError_t launch_pack_kmajor(const uint8_t* codes, const uint8_t* scales, int n_exp, int N, int K, uint8_t* codes_out,
                              uint8_t* scales_out, hipStream_t s);
// weight-streaming kernels (H % 256 == 0, I / 32 a power of two <= 64)
bool ffn_stream_supported(int H, int I);
hipError_t launch_gateup_stream(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_down_stream(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_rms_norm(const uint16_t* x, int64_t T, int H, double eps, uint16_t* out, hipStream_t s);
hipError_t launch_combine_f32(int64_t T, int H, int k, const float* y_rows, const float* y_shared, const int32_t* p2r,
                             const float* w, float* out, hipStream_t s);
hipError_t launch_combine(int64_t T, int H, int k, const float* y_rows, const float* y_shared, const int32_t* p2r,
                          const float* w, const uint16_t* residual, uint16_t* out, hipStream_t s);

}  // namespace moe

// Router-weighted combine: out[t] = RNE_BF16(sum_j w[t][j] * y[pair2row[t*k+j]]
// + y_shared[t] + residual[t]) in FP32, j ascending.  Every selected expert
// contributes; none is dropped (capy-flash README v0.7.7, "Benchmarks");
// partials stay in FP32 until the single final rounding (Richland article,
// "Why it matters").  HBM-bound: (k+1) FP32 rows read and one BF16 row written
// per token.  One thread per 4 output columns, 128-bit loads.
#include "common.hpp"

namespace moe {

// 16-byte load marked non-temporal: the rows are read once, so they need not
// displace other lines in the caches
__device__ __forceinline__ float4 load_once(const float* p) {
  const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// kMaxK: a bound on k fixed at compile time (the row arrays live in registers;
// a tight bound keeps more waves resident: 0.37 -> 0.32 ms at 15,360 tokens, k = 10)
template <int kMaxK>
__global__ __launch_bounds__(256) void k_combine(int64_t T, int H, int k, const float* __restrict__ y_rows,
                                                 const float* __restrict__ y_shared, const int32_t* __restrict__ p2r,
                                                 const float* __restrict__ w, const uint16_t* __restrict__ residual,
                                                 uint16_t* __restrict__ out) {
  const int per_row = H / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= T * per_row) return;
  const int64_t t = gid / per_row;
  const int c4 = (int)(gid % per_row) * 4;
  // all row indices and weights first, then every row load, then the sums in
  // slot order (loads in flight together instead of one round trip per slot)
  int64_t r[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      r[j] = p2r ? p2r[t * k + j] : t * k + j;  // no map: the rows are in token-major order
      wj[j] = w[t * k + j];
    }
  }
  float4 y[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j)
    if (j < k) y[j] = load_once(y_rows + r[j] * H + c4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      acc.x = fmaf(wj[j], y[j].x, acc.x);
      acc.y = fmaf(wj[j], y[j].y, acc.y);
      acc.z = fmaf(wj[j], y[j].z, acc.z);
      acc.w = fmaf(wj[j], y[j].w, acc.w);
    }
  }
  if (y_shared) {
    const float4 y = load_once(y_shared + t * H + c4);
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  if (residual) {
    const uint2 rv = *reinterpret_cast<const uint2*>(residual + t * H + c4);
    acc.x += __uint_as_float(rv.x << 16);
    acc.y += __uint_as_float(rv.x & 0xFFFF0000u);
    acc.z += __uint_as_float(rv.y << 16);
    acc.w += __uint_as_float(rv.y & 0xFFFF0000u);
  }
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + t * H + c4) = make_uint2(lo, hi);
}

// The un-rounded FP32 layer output without residual (a K-split partial when
// the rows are partials): out[t] = sum_j w[t][j] y[pair2row[t*k+j]] + y_shared[t],
// with the same fused multiply-adds in the same order as k_combine, so that
// k_combine's output is the BF16 rounding of this sum (plus the residual).
__global__ __launch_bounds__(256) void k_combine_f32(int64_t T, int H, int k, const float* __restrict__ y_rows,
                                                     const float* __restrict__ y_shared,
                                                     const int32_t* __restrict__ p2r, const float* __restrict__ w,
                                                     float* __restrict__ out) {
  const int per_row = H / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= T * per_row) return;
  const int64_t t = gid / per_row;
  const int c4 = (int)(gid % per_row) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[t * k + j];
    const float4 y = *reinterpret_cast<const float4*>(y_rows + (int64_t)p2r[t * k + j] * H + c4);
    acc.x = fmaf(wj, y.x, acc.x);
    acc.y = fmaf(wj, y.y, acc.y);
    acc.z = fmaf(wj, y.z, acc.z);
    acc.w = fmaf(wj, y.w, acc.w);
  }
  if (y_shared) {
    const float4 y = *reinterpret_cast<const float4*>(y_shared + t * H + c4);
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  *reinterpret_cast<float4*>(out + t * H + c4) = acc;
}

hipError_t launch_combine_f32(int64_t T, int H, int k, const float* y_rows, const float* y_shared, const int32_t* p2r,
                             const float* w, float* out, hipStream_t s) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, H, k, y_rows, y_shared,
                     p2r, w, out);
  return hipGetLastError();
}

hipError_t launch_combine(int64_t T, int H, int k, const float* y_rows, const float* y_shared, const int32_t* p2r,
                          const float* w, const uint16_t* residual, uint16_t* out, hipStream_t s) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (k <= 4)
    hipLaunchKernelGGL(k_combine<4>, grid, block, 0, s, T, H, k, y_rows, y_shared, p2r, w, residual, out);
  else if (k <= 8)
    hipLaunchKernelGGL(k_combine<8>, grid, block, 0, s, T, H, k, y_rows, y_shared, p2r, w, residual, out);
  else if (k <= 12)
    hipLaunchKernelGGL(k_combine<12>, grid, block, 0, s, T, H, k, y_rows, y_shared, p2r, w, residual, out);
  else if (k <= 16)
    hipLaunchKernelGGL(k_combine<16>, grid, block, 0, s, T, H, k, y_rows, y_shared, p2r, w, residual, out);
  else
    hipLaunchKernelGGL(k_combine<32>, grid, block, 0, s, T, H, k, y_rows, y_shared, p2r, w, residual, out);
  return hipGetLastError();
}

}  // namespace moe

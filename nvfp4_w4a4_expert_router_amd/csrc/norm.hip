// Parameter-free RMS norm of BF16 rows, the composition used to chain MoE
// layers into a stack (the pages run 48 MoE layers, Richland article "What
// shipped", but print no block structure): n = RNE_BF16(x / sqrt(mean x^2 +
// eps)).  One wave per row; the sum of squares (exact products), the scale and
// the product are FP64 and the result is rounded once to BF16, so the output
// does not depend on the order of the sum beyond the last FP64 bit.
#include "common.hpp"

namespace moe {

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

__global__ __launch_bounds__(256) void k_rms_norm(const uint16_t* __restrict__ x, int64_t T, int H, double eps,
                                                  uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = lane_id();
  const uint16_t* row = x + t * H;
  double ss = 0.0;
  for (int h = lane; h < H; h += kWave) {
    const double v = bf16_to_f32(row[h]);
    ss = fma(v, v, ss);
  }
  ss = wave_sum_f64(ss);
  const double inv = 1.0 / sqrt(ss / (double)H + eps);
  for (int h = lane; h < H; h += kWave) out[t * H + h] = f64_to_bf16_rne((double)bf16_to_f32(row[h]) * inv);
}

hipError_t launch_rms_norm(const uint16_t* x, int64_t T, int H, double eps, uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rms_norm, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, T, H, eps, out);
  return hipGetLastError();
}

}  // namespace moe

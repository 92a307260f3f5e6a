// Parameter-free RMS norm of BF16 rows, the composition used to chain MoE
// layers into a stack (the pages run 48 MoE layers, Richland article "What
// shipped", but print no block structure): n = RNE_BF16(x / sqrt(mean x^2 +
// eps)).  The sum of squares (exact products), the scale and the product are
// FP64 and the result is rounded once to BF16, so the output does not depend on
// the order of the sum beyond the last FP64 bit.
#include "common.hpp"

namespace moe {

// One workgroup per row: each thread holds 8 consecutive elements (one 16-byte
// load, a second round only for H > 2048), the FP64 sum of squares goes
// through the wave sums and LDS, and the thread scales and stores its own
// elements (one 16-byte store), so the row is read from memory once.
constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void k_rms_norm(const uint16_t* __restrict__ x, int64_t T, int H,
                                                           double eps, uint16_t* __restrict__ out) {
  __shared__ double wsum[kNormThreads / kWave];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6;
  const uint16_t* row = x + t * H;
  uint16_t* orow = out + t * H;
  double ss = 0.0;
  if (H % 8 == 0) {
    for (int h0 = 8 * tid; h0 < H; h0 += 8 * kNormThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + h0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xFFFF0000u);
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
      }
    }
  } else {
    for (int h = tid; h < H; h += kNormThreads) {
      const double v = bf16_to_f32(row[h]);
      ss = fma(v, v, ss);
    }
  }
  ss = wave_sum_f64(ss);
  if ((tid & (kWave - 1)) == 0) wsum[wave] = ss;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int w = 0; w < kNormThreads / kWave; ++w) tot += wsum[w];
  const double inv = 1.0 / sqrt(tot / (double)H + eps);
  if (H % 8 == 0) {
    for (int h0 = 8 * tid; h0 < H; h0 += 8 * kNormThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + h0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f64_to_bf16_rne((double)__uint_as_float(w[i] << 16) * inv);
        const uint32_t hi = f64_to_bf16_rne((double)__uint_as_float(w[i] & 0xFFFF0000u) * inv);
        o[i] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(orow + h0) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    for (int h = tid; h < H; h += kNormThreads) orow[h] = f64_to_bf16_rne((double)bf16_to_f32(row[h]) * inv);
  }
}

hipError_t launch_rms_norm(const uint16_t* x, int64_t T, int H, double eps, uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rms_norm, dim3((unsigned)T), dim3(kNormThreads), 0, s, x, T, H, eps, out);
  return hipGetLastError();
}

}  // namespace moe

// A4 activation encoding (capy-flash README v0.5.4, "What it does" / "Serve":
// the GPU's W4A4 activation quantization, reproduced exactly wherever an expert
// runs).  One thread per 16-element block: amax, UE4M3 scale by exact
// comparison, E2M1 codes, and optionally the dequantized FP16 block
// e2m1(code) * ue4m3(scale) (exact in FP16: <= 6 significant bits, magnitude
// in [2^-10, 2688]) for the matrix-core operands.  HBM-bound: 32 B (BF16) or
// 64 B (FP32) read and 9 B (+32 B FP16) written per block.
#include "common.hpp"

namespace moe {

template <bool kBf16>
__global__ __launch_bounds__(256) void k_quant_act(const void* __restrict__ x, int64_t nblocks, float g, float g6,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                   half_t* __restrict__ deq) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[16];
  if (kBf16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 16);
    const uint4 a0 = src[0], a1 = src[1];
    const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = src[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = scale_code(amax, g6);
  const float sv = ue4m3_value(sc);
  // the block's seven threshold products once, then three comparisons per
  // element (elem_code's thresholds and tie rules; scale code 0 encodes zeros)
  const E2M1Thresholds Tb = e2m1_thresholds(sc ? sv * g : __builtin_inff());
  uint32_t packed[2] = {0u, 0u};
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    c[i] = elem_code_t(v[i], Tb);
    packed[i >> 3] |= c[i] << (4 * (i & 7));
  }
  reinterpret_cast<uint2*>(codes)[b] = make_uint2(packed[0], packed[1]);
  scales[b] = (uint8_t)sc;
  if (deq) {
    half8_t h0, h1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h0[i] = (half_t)(e2m1_value(c[i]) * sv);
      h1[i] = (half_t)(e2m1_value(c[8 + i]) * sv);
    }
    half8_t* dst = reinterpret_cast<half8_t*>(deq + b * 16);
    dst[0] = h0;
    dst[1] = h1;
  }
}

// A8 encoding (the W4A8 variant): one thread per 16-element block, INT8 codes
// (one byte per element), the UE4M3 scale, and optionally the dequantized FP16
// block q * ue4m3(scale) (exact in FP16).
template <bool kBf16>
__global__ __launch_bounds__(256) void k_quant_act8(const void* __restrict__ x, int64_t nblocks, float g, float g127,
                                                    int8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                    half_t* __restrict__ deq) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[16];
  if (kBf16) {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 16);
    const uint4 a0 = src[0], a1 = src[1];
    const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = src[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = scale_code(amax, g127);
  const float sv = ue4m3_value(sc);
  const float s = sc ? sv * g : __builtin_inff();
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
  int q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    q[i] = int8_code(v[i], s);
    packed[i >> 2] |= ((uint32_t)q[i] & 0xFFu) << (8 * (i & 3));
  }
  reinterpret_cast<uint4*>(codes)[b] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[b] = (uint8_t)sc;
  if (deq) {
    half8_t h0, h1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      h0[i] = (half_t)((float)q[i] * sv);
      h1[i] = (half_t)((float)q[8 + i] * sv);
    }
    half8_t* dst = reinterpret_cast<half8_t*>(deq + b * 16);
    dst[0] = h0;
    dst[1] = h1;
  }
}

hipError_t launch_quant_act(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, uint8_t* codes,
                            uint8_t* scales, half_t* deq, hipStream_t s, hipEvent_t e0, hipEvent_t e1,
                            int act_bits) {
  const int64_t nblocks = rows * (int64_t)(cols / 16);
  if (nblocks == 0) return record_idle(s, e0, e1);
  const dim3 grid((unsigned)((nblocks + 255) / 256)), block(256);
  if (act_bits == 8) {
    int8_t* c8 = reinterpret_cast<int8_t*>(codes);
    const float g127 = 127.0f * gscale;
    if (dtype == MOE_DTYPE_BF16)
      return launch_timed(k_quant_act8<true>, grid, block, 0, s, e0, e1, x, nblocks, gscale, g127, c8, scales, deq);
    return launch_timed(k_quant_act8<false>, grid, block, 0, s, e0, e1, x, nblocks, gscale, g127, c8, scales, deq);
  }
  const float g6 = 6.0f * gscale;
  if (dtype == MOE_DTYPE_BF16)
    return launch_timed(k_quant_act<true>, grid, block, 0, s, e0, e1, x, nblocks, gscale, g6, codes, scales, deq);
  return launch_timed(k_quant_act<false>, grid, block, 0, s, e0, e1, x, nblocks, gscale, g6, codes, scales, deq);
}

}  // namespace moe

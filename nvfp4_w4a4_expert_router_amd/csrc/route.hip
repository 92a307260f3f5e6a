// Router: logits over the experts, top-k per token and softmax over the
// selected logits (512 experts, top-10 routed: capy-flash README v0.5.4,
// synthetic test-artifact script; Richland article, "What shipped").
//
// A sum in another order can pick the other of two nearly tied experts
// (capy-flash README v0.5.4, "Measured", footnote on the tensor-core router).
// To make the decision independent of the summation order, the selection is
// taken on FP64 logits, computed only where they matter:
//   pass A  FP32 logits l32 with a known worst-case error: every logit is a
//           sum whose longest rounding path has d roundings, so
//           |l32 - l| <= gamma_d * sum_h |x_h W_eh| <= gamma_d ||x|| ||W_e||
//           (Cauchy-Schwarz), gamma_d = d u / (1 - d u), u = 2^-24.  The same
//           pass returns ||W_e||.
//   pass B  per token: interval [l32 - r_e, l32 + r_e]; an expert can be in the
//           top k only if its upper end reaches the k-th largest lower end.
//           Those candidates (k plus the few near the boundary) get an FP64
//           dot product with exact products (BF16 x FP32 fits in 53 bits);
//           top k of the candidates by (FP64 logit desc, id asc), softmax in
//           FP64, weights rounded to FP32.
// Two experts whose router rows agree wherever x is nonzero get identical
// logits in both passes, so the tie rule (lower id first) decides.
#include "common.hpp"

namespace moe {

// ---------------------------------------------------------------- pass A, prefill: tiled GEMM
// logits[t][e] = sum_h x[t][h] * W[e][h].  Tile 64 tokens x 64 experts, K step 16,
// 256 threads with 4x4 outputs each.  Each K step is summed into a fresh
// partial (16 roundings) before joining the running sum (H/16 roundings):
// rounding depth 16 + H/16.
constexpr int RT = 64, RE = 64, RK = 16;

__global__ __launch_bounds__(256) void k_router_logits_tiled(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ W, int T, int H, int E,
                                                             float* __restrict__ logits) {
  __shared__ float xs[RK][RT + 4];
  __shared__ float ws[RK][RE + 4];
  const int t0 = blockIdx.y * RT, e0 = blockIdx.x * RE;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int h0 = 0; h0 < H; h0 += RK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + q * 256;
      const int r = idx >> 4, c = idx & 15;
      const int t = t0 + r, e = e0 + r;
      xs[c][r] = (t < T) ? bf16_to_f32(x[(int64_t)t * H + h0 + c]) : 0.0f;
      ws[c][r] = (e < E) ? W[(int64_t)e * H + h0 + c] : 0.0f;
    }
    __syncthreads();
    float part[4][4] = {};
#pragma unroll
    for (int c = 0; c < RK; ++c) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ws[c][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) part[i][j] = fmaf(a[i], b[j], part[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += part[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + tx * 4 + j;
      if (e < E) logits[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

// ||W_e||_2 for every expert (FP32 sum of squares, one wave per expert).
__global__ __launch_bounds__(256) void k_router_norms(const float* __restrict__ W, int H, int E,
                                                      float* __restrict__ wnorm) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int lane = lane_id();
  float s = 0.0f;
  for (int h = lane; h < H; h += kWave) {
    const float w = W[(int64_t)e * H + h];
    s = fmaf(w, w, s);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (lane == 0) wnorm[e] = sqrtf(s);
}

// ---------------------------------------------------------------- pass A, decode: GEMV
// For a few tokens: one wave per expert row; lane l owns a contiguous slice of
// H/64 elements (sequential FMA), then a 6-level butterfly: rounding depth
// H/64 + 6.  The wave also returns ||W_e||.  x is staged once per workgroup in LDS.
constexpr int kGemvMaxT = 8;

__global__ __launch_bounds__(256) void k_router_logits_gemv(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ W, int T, int H, int E,
                                                            float* __restrict__ logits, float* __restrict__ wnorm) {
  extern __shared__ float xsh[];  // [T][H]
  for (int i = threadIdx.x; i < T * H; i += blockDim.x) xsh[i] = bf16_to_f32(x[i]);
  __syncthreads();
  const int lane = lane_id();
  const int per = H / kWave;  // H is a multiple of 64 here
  const int waves = (int)(gridDim.x * (blockDim.x / kWave));
  for (int e = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6); e < E; e += waves) {
    const float* wr = W + (int64_t)e * H + lane * per;
    float acc[kGemvMaxT] = {};
    float sq = 0.0f;
    for (int i = 0; i < per; i += 4) {
      const float4 w = *reinterpret_cast<const float4*>(wr + i);
      sq = fmaf(w.x, w.x, sq);
      sq = fmaf(w.y, w.y, sq);
      sq = fmaf(w.z, w.z, sq);
      sq = fmaf(w.w, w.w, sq);
#pragma unroll
      for (int t = 0; t < kGemvMaxT; ++t) {
        if (t < T) {
          const float* xr = xsh + t * H + lane * per + i;
          float a = acc[t];
          a = fmaf(xr[0], w.x, a);
          a = fmaf(xr[1], w.y, a);
          a = fmaf(xr[2], w.z, a);
          a = fmaf(xr[3], w.w, a);
          acc[t] = a;
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sq += __shfl_xor(sq, m);
#pragma unroll
      for (int t = 0; t < kGemvMaxT; ++t) acc[t] += __shfl_xor(acc[t], m);
    }
    if (lane == 0) {
      wnorm[e] = sqrtf(sq);
#pragma unroll
      for (int t = 0; t < kGemvMaxT; ++t)
        if (t < T) logits[(int64_t)t * E + e] = acc[t];
    }
  }
}

// ---------------------------------------------------------------- pass B
constexpr int kMaxPerLane = 16;  // E <= 1024
constexpr int kMaxCand = 1024;

__device__ __forceinline__ bool better_f(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }
__device__ __forceinline__ bool better_d(double v, int e, double bv, int be) {
  return v > bv || (v == bv && e < be);
}

struct RouteB {
  const float* logits;  // [T][E] FP32: pass-A logits, or caller's logits (refine == 0)
  const float* wnorm;   // [E] (refine only)
  const uint16_t* x;    // [T][H] (refine only)
  const float* W;       // [E][H] (refine only)
  int64_t T;
  int H, E, k, refine;
  float gamma;  // error coefficient of pass A, already inflated
  int32_t* idx;
  float* w;
};

// One wave per token, 4 tokens per workgroup.
__global__ __launch_bounds__(256) void k_route_select(RouteB p) {
  __shared__ double cval[4][kMaxCand];
  __shared__ int cid[4][kMaxCand];
  const int wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= p.T) return;
  const int lane = lane_id();
  const int E = p.E, H = p.H, k = p.k;
  const float* row = p.logits + t * E;
  float v[kMaxPerLane], rad[kMaxPerLane];
  const int nper = (E + kWave - 1) / kWave;

  float xn = 0.0f;
  if (p.refine) {  // ||x_t||_2, inflated for its own rounding
    float s = 0.0f;
    for (int h = lane; h < H; h += kWave) {
      const float a = bf16_to_f32(p.x[t * H + h]);
      s = fmaf(a, a, s);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    xn = sqrtf(s) * 1.001f;
  }
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + kWave * j;
    const bool ok = j < nper && e < E;
    v[j] = ok ? row[e] : -INFINITY;
    rad[j] = (ok && p.refine) ? p.gamma * xn * (p.wnorm[e] * 1.001f) + 1e-30f : 0.0f;
  }
  // k-th largest lower end (ties by id do not matter for the value)
  uint32_t taken = 0;
  float lk = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + kWave * j;
      const float lo = v[j] - rad[j];
      if (j < nper && e < E && !((taken >> j) & 1u) && better_f(lo, e, bv, be)) {
        bv = lo;
        be = e;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oe = __shfl_xor(be, m);
      if (better_f(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
    lk = bv;
  }
  // candidates in ascending id order: upper end reaches lk
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + kWave * j;
    const bool c = j < nper && e < E && v[j] + rad[j] >= lk;
    const uint64_t m = __ballot(c);
    if (c) {
      const int pos = ncand + __popcll(m & ((1ull << lane) - 1ull));
      cid[wave][pos] = e;
      cval[wave][pos] = (double)v[j];
    }
    ncand += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (p.refine) {
    // exact-product FP64 dot for each candidate
    for (int c = 0; c < ncand; ++c) {
      const int e = cid[wave][c];
      const float* wr = p.W + (int64_t)e * H;
      double s = 0.0;
      for (int h = lane; h < H; h += kWave) s += (double)bf16_to_f32(p.x[t * H + h]) * (double)wr[h];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
      if (lane == 0) cval[wave][c] = s;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  // top k of the candidates by (value desc, id asc); lane owns candidates lane + 64 q
  double cv[kMaxPerLane];
  int ce[kMaxPerLane];
#pragma unroll
  for (int q = 0; q < kMaxPerLane; ++q) {
    const int c = lane + kWave * q;
    cv[q] = c < ncand ? cval[wave][c] : -INFINITY;
    ce[q] = c < ncand ? cid[wave][c] : 0x7FFFFFFF;
  }
  double my_v = 0.0, top_v = 0.0;
  int my_e = 0;
  uint32_t ctaken = 0;
  for (int r = 0; r < k; ++r) {
    double bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q)
      if (lane + kWave * q < ncand && !((ctaken >> q) & 1u) && better_d(cv[q], ce[q], bv, be)) {
        bv = cv[q];
        be = ce[q];
      }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const double ov = __shfl_xor(bv, m);
      const int oe = __shfl_xor(be, m);
      if (better_d(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q)
      if (lane + kWave * q < ncand && ce[q] == be) ctaken |= 1u << q;
    if (r == 0) top_v = bv;
    if (lane == r) {
      my_v = bv;
      my_e = be;
    }
  }
  const double ex = lane < k ? exp(my_v - top_v) : 0.0;
  double total = 0.0;
  for (int j = 0; j < k; ++j) total += __shfl(ex, j);
  if (lane < k) {
    p.idx[t * k + lane] = my_e;
    p.w[t * k + lane] = (float)(ex / total);
  }
}

// ---------------------------------------------------------------- launchers
static float gamma_for_depth(int d) {
  const double u = 0x1p-24;
  return (float)(1.01 * d * u / (1.0 - d * u));
}

size_t route_ws_bytes(int64_t T, int E) {
  return (size_t)(T * E) * sizeof(float) + 256 + (size_t)E * sizeof(float);
}

hipError_t launch_route(const uint16_t* x, const float* W, int64_t T, int H, int E, int k, const float* logits_in,
                        int32_t* idx, float* w, void* ws, hipStream_t s) {
  RouteB p;
  p.T = T;
  p.H = H;
  p.E = E;
  p.k = k;
  p.idx = idx;
  p.w = w;
  p.x = x;
  p.W = W;
  if (logits_in) {
    p.logits = logits_in;
    p.wnorm = nullptr;
    p.refine = 0;
    p.gamma = 0.0f;
  } else {
    float* lg = static_cast<float*>(ws);
    float* wn = reinterpret_cast<float*>(static_cast<char*>(ws) + ((size_t)(T * E) * sizeof(float) + 255) / 256 * 256);
    if (T <= kGemvMaxT && H % (4 * kWave) == 0 && (size_t)T * H * sizeof(float) <= 64 * 1024) {
      const size_t lds = (size_t)T * H * sizeof(float);
      const int blocks = (E + 3) / 4 < 128 ? (E + 3) / 4 : 128;
      hipLaunchKernelGGL(k_router_logits_gemv, dim3(blocks), dim3(256), lds, s, x, W, (int)T, H, E, lg, wn);
      p.gamma = gamma_for_depth(H / kWave + 6);
    } else {
      const dim3 grid((unsigned)((E + RE - 1) / RE), (unsigned)((T + RT - 1) / RT));
      hipLaunchKernelGGL(k_router_logits_tiled, grid, dim3(256), 0, s, x, W, (int)T, H, E, lg);
      hipLaunchKernelGGL(k_router_norms, dim3((E + 3) / 4), dim3(256), 0, s, W, H, E, wn);
      p.gamma = gamma_for_depth(RK + H / RK);
    }
    p.logits = lg;
    p.wnorm = wn;
    p.refine = 1;
  }
  hipLaunchKernelGGL(k_route_select, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe

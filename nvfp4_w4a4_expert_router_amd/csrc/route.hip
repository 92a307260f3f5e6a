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

// ---------------------------------------------------------------- decode: FP64 GEMV
// For a few tokens the router weights (E x H x 4 bytes) are streamed once and
// every logit is summed in FP64 from exact products, so no refinement pass is
// needed.  One wave per expert row; lane l owns elements [l*H/64, (l+1)*H/64)
// (loaded with 128-bit loads, all issued before the arithmetic), then a
// butterfly over the wave.
constexpr int kGemvMaxT = 8;
constexpr int kGemvPer = 32;  // elements per lane per pass (H = 2048 is one pass)

__global__ __launch_bounds__(256) void k_router_gemv64(const uint16_t* __restrict__ x, const float* __restrict__ W,
                                                      int T, int H, int E, double* __restrict__ logits) {
  const int lane = lane_id();
  const int waves = (int)(gridDim.x * (blockDim.x / kWave));
  for (int e = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x >> 6); e < E; e += waves) {
    double acc[kGemvMaxT] = {};
    for (int h0 = lane * kGemvPer; h0 < H; h0 += kWave * kGemvPer) {
      float4 w[kGemvPer / 4];
#pragma unroll
      for (int i = 0; i < kGemvPer / 4; ++i) w[i] = *reinterpret_cast<const float4*>(W + (int64_t)e * H + h0 + 4 * i);
#pragma unroll
      for (int t = 0; t < kGemvMaxT; ++t) {
        if (t >= T) break;
        uint4 xv[kGemvPer / 8];
#pragma unroll
        for (int i = 0; i < kGemvPer / 8; ++i) xv[i] = *reinterpret_cast<const uint4*>(x + (int64_t)t * H + h0 + 8 * i);
        double a = acc[t];
#pragma unroll
        for (int i = 0; i < kGemvPer / 8; ++i) {
          const uint32_t q[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
          const float4 w0 = w[2 * i], w1 = w[2 * i + 1];
          const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a = fma((double)__uint_as_float(q[j] << 16), (double)wf[2 * j], a);
            a = fma((double)__uint_as_float(q[j] & 0xFFFF0000u), (double)wf[2 * j + 1], a);
          }
        }
        acc[t] = a;
      }
    }
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) {
      if (t >= T) break;
      double a = acc[t];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) a += __shfl_xor(a, m);
      if (lane == 0) logits[(int64_t)t * E + e] = a;
    }
  }
}

// ---------------------------------------------------------------- pass B: selection
constexpr int kMaxPerLane = 16;  // E <= 1024
constexpr int kMaxCand = 1024;

__device__ __forceinline__ bool better(double v, int e, double bv, int be) { return v > bv || (v == bv && e < be); }

enum { kSelF32 = 0, kSelF64 = 1, kSelRefine = 2 };

struct RouteB {
  const float* l32;     // [T][E] caller logits (kSelF32) or pass-A FP32 logits (kSelRefine)
  const double* l64;    // [T][E] FP64 logits (kSelF64)
  const float* wnorm;   // [E] (kSelRefine)
  const uint16_t* x;    // [T][H] (kSelRefine)
  const float* W;       // [E][H] (kSelRefine)
  int64_t T;
  int H, E, k, mode;
  float gamma;  // error coefficient of pass A, already inflated (kSelRefine)
  int32_t* idx;
  float* w;
};

// FP64 dot of x_t (BF16) with router row e over this lane's slice: exact products.
__device__ __forceinline__ double dot64_lane(const uint16_t* __restrict__ xr, const float* __restrict__ wr, int H,
                                             int lane) {
  double a = 0.0;
  for (int h0 = lane * 32; h0 < H; h0 += kWave * 32) {
    uint4 xv[4];
    float4 w[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const uint4*>(xr + h0 + 8 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const float4*>(wr + h0 + 4 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t q[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
      const float wf[8] = {w[2 * i].x, w[2 * i].y, w[2 * i].z, w[2 * i].w,
                           w[2 * i + 1].x, w[2 * i + 1].y, w[2 * i + 1].z, w[2 * i + 1].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a = fma((double)__uint_as_float(q[j] << 16), (double)wf[2 * j], a);
        a = fma((double)__uint_as_float(q[j] & 0xFFFF0000u), (double)wf[2 * j + 1], a);
      }
    }
  }
  return a;
}

// One wave per token, 4 tokens per workgroup.
__global__ __launch_bounds__(256) void k_route_select(RouteB p) {
  __shared__ double cval[4][kMaxCand];
  __shared__ int cid[4][kMaxCand];
  const int wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= p.T) return;
  const int lane = lane_id();
  const int E = p.E, H = p.H, k = p.k;
  const int nper = (E + kWave - 1) / kWave;
  double v[kMaxPerLane];
  float rad[kMaxPerLane];
  int vid[kMaxPerLane];  // expert id of v[j]

  float xn = 0.0f;
  if (p.mode == kSelRefine) {  // ||x_t||_2, inflated for its own rounding
    float sq = 0.0f;
    for (int h = lane; h < H; h += kWave) {
      const float a = bf16_to_f32(p.x[t * H + h]);
      sq = fmaf(a, a, sq);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sq += __shfl_xor(sq, m);
    xn = sqrtf(sq) * 1.001f;
  }
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + kWave * j;
    const bool ok = j < nper && e < E;
    vid[j] = ok ? e : 0x7FFFFFFF;
    if (!ok) {
      v[j] = -INFINITY;
      rad[j] = 0.0f;
    } else if (p.mode == kSelF64) {
      v[j] = p.l64[t * E + e];
      rad[j] = 0.0f;
    } else {
      v[j] = (double)p.l32[t * E + e];
      rad[j] = p.mode == kSelRefine ? p.gamma * xn * (p.wnorm[e] * 1.001f) + 1e-30f : 0.0f;
    }
  }
  int ncand = 0;
  if (p.mode == kSelRefine) {
    // k-th largest lower end
    uint32_t taken = 0;
    double lk = 0.0;
    for (int r = 0; r < k; ++r) {
      double bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + kWave * j;
        const double lo = v[j] - (double)rad[j];
        if (j < nper && e < E && !((taken >> j) & 1u) && better(lo, e, bv, be)) {
          bv = lo;
          be = e;
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ov = __shfl_xor(bv, m);
        const int oe = __shfl_xor(be, m);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
      lk = bv;
    }
    // candidates (ascending id): upper end reaches lk; FP64 logits for them
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = lane + kWave * j;
      const bool c = j < nper && e < E && v[j] + (double)rad[j] >= lk;
      const uint64_t m = __ballot(c);
      if (c) cid[wave][ncand + __popcll(m & ((1ull << lane) - 1ull))] = e;
      ncand += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const uint16_t* xr = p.x + t * H;
    for (int c = 0; c < ncand; c += 2) {
      const int e0 = cid[wave][c];
      const int e1 = c + 1 < ncand ? cid[wave][c + 1] : e0;
      double a0 = dot64_lane(xr, p.W + (int64_t)e0 * H, H, lane);
      double a1 = dot64_lane(xr, p.W + (int64_t)e1 * H, H, lane);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        a0 += __shfl_xor(a0, m);
        a1 += __shfl_xor(a1, m);
      }
      if (lane == 0) {
        cval[wave][c] = a0;
        if (c + 1 < ncand) cval[wave][c + 1] = a1;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the candidates replace the per-lane values: lane owns candidates lane + 64 q
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q) {
      const int c = lane + kWave * q;
      v[q] = c < ncand ? cval[wave][c] : -INFINITY;
      vid[q] = c < ncand ? cid[wave][c] : 0x7FFFFFFF;
    }
  }
  // top k by (value desc, id asc) over the entries with a valid id
  double my_v = 0.0, top_v = 0.0;
  int my_e = 0;
  const int nvalid = p.mode == kSelRefine ? ncand : E;
  if (nvalid <= 8 * kWave) {
    double v8[8];
    int id8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool ok = vid[q] != 0x7FFFFFFF;
      v8[q] = ok ? v[q] : -INFINITY;
      id8[q] = vid[q];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    wave_topk512(v8, id8, k, cval[wave], cid[wave], &my_v, &my_e);
    const float wk = topk_softmax_weight(my_v, k);
    if (lane < k) {
      p.idx[t * k + lane] = my_e;
      p.w[t * k + lane] = wk;
    }
    return;
  } else {
    uint32_t taken = 0;
    for (int r = 0; r < k; ++r) {
      double bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q) {
        if (vid[q] != 0x7FFFFFFF && !((taken >> q) & 1u) && better(v[q], vid[q], bv, be)) {
          bv = v[q];
          be = vid[q];
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const double ov = __shfl_xor(bv, m);
        const int oe = __shfl_xor(be, m);
        if (better(ov, oe, bv, be)) {
          bv = ov;
          be = oe;
        }
      }
#pragma unroll
      for (int q = 0; q < kMaxPerLane; ++q)
        if (vid[q] == be) taken |= 1u << q;
      if (r == 0) top_v = bv;
      if (lane == r) {
        my_v = bv;
        my_e = be;
      }
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
hipError_t launch_router_logits64(const uint16_t* x, const float* W, int64_t T, int H, int E, double* logits,
                                  hipStream_t s) {
  hipLaunchKernelGGL(k_router_gemv64, dim3((unsigned)((E + 3) / 4)), dim3(256), 0, s, x, W, (int)T, H, E, logits);
  return hipGetLastError();
}

static float gamma_for_depth(int d) {
  const double u = 0x1p-24;
  return (float)(1.01 * d * u / (1.0 - d * u));
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

size_t route_ws_bytes(int64_t T, int E) {
  const size_t lg = T <= kGemvMaxT ? (size_t)(T * E) * sizeof(double) : (size_t)(T * E) * sizeof(float);
  return align256(lg) + align256((size_t)E * sizeof(float));
}

hipError_t launch_route(const uint16_t* x, const float* W, int64_t T, int H, int E, int k, const float* logits_in,
                        int32_t* idx, float* w, void* ws, hipStream_t s) {
  RouteB p = {};
  p.T = T;
  p.H = H;
  p.E = E;
  p.k = k;
  p.idx = idx;
  p.w = w;
  p.x = x;
  p.W = W;
  if (logits_in) {
    p.l32 = logits_in;
    p.mode = kSelF32;
  } else if (T <= kGemvMaxT) {
    double* lg = static_cast<double*>(ws);
    const int blocks = (E + 3) / 4;
    hipLaunchKernelGGL(k_router_gemv64, dim3(blocks), dim3(256), 0, s, x, W, (int)T, H, E, lg);
    p.l64 = lg;
    p.mode = kSelF64;
  } else {
    float* lg = static_cast<float*>(ws);
    float* wn = reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)(T * E) * sizeof(float)));
    const dim3 grid((unsigned)((E + RE - 1) / RE), (unsigned)((T + RT - 1) / RT));
    hipLaunchKernelGGL(k_router_logits_tiled, grid, dim3(256), 0, s, x, W, (int)T, H, E, lg);
    hipLaunchKernelGGL(k_router_norms, dim3((E + 3) / 4), dim3(256), 0, s, W, H, E, wn);
    p.l32 = lg;
    p.wnorm = wn;
    p.gamma = gamma_for_depth(RK + H / RK);
    p.mode = kSelRefine;
  }
  hipLaunchKernelGGL(k_route_select, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe

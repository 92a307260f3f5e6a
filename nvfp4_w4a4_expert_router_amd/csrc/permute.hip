// Token -> expert permutation: the T*k (token, slot) pairs grouped by expert id
// (ascending), tokens ascending within an expert; pair id p = t*k + j.  Routed
// experts are addressed by id (capy-flash README v0.5.4, "What it does").
//
// Integer work only; the result is unique.  Ranks inside an expert segment
// come from per-wave bit masks: each lane (one token) sets its bit in the mask
// of every expert it selected (atomic OR, order-free), then a token's rank
// among the chunk's tokens of that expert is the popcount of the mask bits
// below it.  Three kernels: per-chunk counts, a scan over (chunk, expert), and
// the scatter.  A token selects k distinct experts, so one bit per token and
// expert suffices.
#include "common.hpp"

namespace moe {

constexpr int kChunkTok = 256;  // tokens per workgroup (4 waves x 64)
constexpr int kMaxE = 1024;  // the scan's one thread per expert

// Fill this wave's masks for a chunk: masks[wave][e] bit lane = token (chunk base
// + 64*wave + lane) selected e.
__device__ __forceinline__ void build_masks(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                            unsigned long long (*masks)[kMaxE], int64_t t0) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  for (int e = lane; e < E; e += kWave) masks[wave][e] = 0ull;
  __syncthreads();
  const int64_t t = t0 + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicOr(&masks[wave][e], 1ull << lane);  // invalid ids are dropped
    }
  __syncthreads();
}

__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                    int32_t* __restrict__ cnt /*[nchunk][E]*/) {
  __shared__ unsigned long long masks[4][kMaxE];
  build_masks(idx, T, k, E, masks, (int64_t)blockIdx.x * kChunkTok);
  for (int e = threadIdx.x; e < E; e += 256)
    cnt[(int64_t)blockIdx.x * E + e] =
        __popcll(masks[0][e]) + __popcll(masks[1][e]) + __popcll(masks[2][e]) + __popcll(masks[3][e]);
}

// One workgroup of 1024 threads: thread e walks the chunks in order (base of
// expert e in chunk c relative to the expert's segment = sum of earlier chunks'
// counts; loads in batches of 16, all in flight together), then a scan over
// experts (per wave, then over the 16 wave totals) gives expert_off.  The
// scatter adds expert_off to the relative bases.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ cnt /*in counts, out bases*/, int nchunk,
                                                    int E, int32_t* __restrict__ off) {
  __shared__ int32_t wtot[16];
  const int e = threadIdx.x, wave = e >> 6, lane = lane_id();
  int run = 0;
  if (e < E)
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = c0 + i < nchunk ? cnt[(int64_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i < nchunk) cnt[(int64_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
  const int incl = wave_incl_scan_i32(run);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wtot[w];
  if (e < E) off[e] = before + incl - run;
  if (e == E - 1) off[E] = before + incl;
}

__global__ __launch_bounds__(256) void k_perm_scatter(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                      const int32_t* __restrict__ base /*[nchunk][E]*/,
                                                      const int32_t* __restrict__ off, int32_t* __restrict__ r2p,
                                                      int32_t* __restrict__ p2r) {
  __shared__ unsigned long long masks[4][kMaxE];
  const int64_t t0 = (int64_t)blockIdx.x * kChunkTok;
  build_masks(idx, T, k, E, masks, t0);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int64_t t = t0 + threadIdx.x;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if (e < 0 || e >= E) continue;
    int r = off[e] + base[(int64_t)blockIdx.x * E + e];
    for (int w = 0; w < wave; ++w) r += __popcll(masks[w][e]);
    r += __popcll(masks[wave][e] & below);
    const int32_t p = (int32_t)(t * k + j);
    r2p[r] = p;
    p2r[p] = r;
  }
}

// Up to 256 tokens: one workgroup does count, scan and scatter (one launch).
__global__ __launch_bounds__(256) void k_perm_single(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                     int32_t* __restrict__ off, int32_t* __restrict__ r2p,
                                                     int32_t* __restrict__ p2r) {
  __shared__ unsigned long long masks[4][kMaxE];
  __shared__ int32_t base[kMaxE];
  __shared__ int32_t part[256];
  build_masks(idx, T, k, E, masks, 0);
  // per-thread run of up to 4 experts, then a scan over the 256 runs
  const int tid = threadIdx.x;
  const int per = (E + 255) / 256;
  int run = 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) {
      base[e] = run;
      run += __popcll(masks[0][e]) + __popcll(masks[1][e]) + __popcll(masks[2][e]) + __popcll(masks[3][e]);
    }
  }
  part[tid] = run;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int add = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int excl = tid > 0 ? part[tid - 1] : 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) {
      base[e] += excl;
      off[e] = base[e];
    }
  }
  if (tid == 255) off[E] = part[255];
  __syncthreads();
  const int wave = tid >> 6, lane = lane_id();
  const int64_t t = tid;
  if (t >= T) return;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if (e < 0 || e >= E) continue;
    int r = base[e];
    for (int w = 0; w < wave; ++w) r += __popcll(masks[w][e]);
    r += __popcll(masks[wave][e] & below);
    const int32_t pr = (int32_t)(t * k + j);
    r2p[r] = pr;
    p2r[pr] = r;
  }
}

size_t permute_ws_bytes(int64_t T, int E) {
  const int64_t nchunk = (T + kChunkTok - 1) / kChunkTok;
  return (size_t)(nchunk * E) * sizeof(int32_t);
}

hipError_t launch_permute(const int32_t* idx, int64_t T, int k, int E, int32_t* off, int32_t* r2p, int32_t* p2r,
                          void* ws, hipStream_t s) {
  const int nchunk = (int)((T + kChunkTok - 1) / kChunkTok);
  if (nchunk == 1) {
    hipLaunchKernelGGL(k_perm_single, dim3(1), dim3(256), 0, s, idx, T, k, E, off, r2p, p2r);
    return hipGetLastError();
  }
  int32_t* cnt = static_cast<int32_t*>(ws);
  if (nchunk > 0) hipLaunchKernelGGL(k_perm_count, dim3(nchunk), dim3(256), 0, s, idx, T, k, E, cnt);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, cnt, nchunk, E, off);
  if (nchunk > 0) hipLaunchKernelGGL(k_perm_scatter, dim3(nchunk), dim3(256), 0, s, idx, T, k, E, cnt, off, r2p, p2r);
  return hipGetLastError();
}

}  // namespace moe

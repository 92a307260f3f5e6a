// Expert FFN for prefill chunks: grouped GEMM on the matrix cores.
//
// NVFP4 operands are decoded exactly to FP16 (Richland article, "What
// shipped": E2M1 codes times UE4M3 block scales): an E2M1 value times a UE4M3
// scale has at most 6 significant bits and lies in [2^-10, 2688], so it is an
// exact FP16 normal number.  The block scale therefore rides on the element and
// the product of two decoded operands is exact in FP32; the matrix core sums in
// FP32 (Richland article, "Why it matters": FP32 partials) and the per-expert
// FP32 scales multiply the result once.  The A4 activations arrive already
// dequantized to FP16 (x from the A4 kernel, h from this file's epilogue).
//
// Work decomposition: the rows of each expert segment (permuted-row order) are
// cut into 128-row tiles; a work item is (row tile, column tile).  A small
// kernel turns expert_off into the prefix of tile counts; each workgroup
// binary-searches its row tile.  Work items of one column tile sit 8 apart in
// the grid, so with round-robin workgroup placement they share an XCD and its
// L2 for the expert's weight slice.
//
// G1 (gate/up): 128 rows x (64 gate + 64 up) columns, K = H in steps of 64;
// wave w computes rows 64*(w/2).. and h columns 32*(w%2).. for both gate and
// up, so SwiGLU pairs meet in the same lane; the epilogue forms h, encodes its
// 16-column blocks (amax across the 16 lanes of a DPP row) and stores the
// dequantized FP16 h.  G2 (down): 128 rows x 128 output columns, K = I.
#include "common.hpp"

namespace moe {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsStride = kBK + 8;  // halfs per LDS row (+16 B against bank conflicts)

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));


// row tile -> (expert slot, first row in the segment); slot E = shared expert
__device__ __forceinline__ int find_tile(const int32_t* __restrict__ tile_start, int nseg, int mt) {
  int lo = 0, hi = nseg;  // last seg with tile_start[seg] <= mt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_start[mid] <= mt) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace

// tile_start[s] = number of 128-row tiles of segments < s; segments 0..E-1 are the
// routed experts, segment E the shared expert (T rows), tile_start[E+1] = total.
__global__ __launch_bounds__(1024) void k_tile_map(const int32_t* __restrict__ off, int E, int T, int has_shared,
                                                   int32_t* __restrict__ tile_start) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int n = tid < E ? (off[tid + 1] - off[tid] + kBM - 1) / kBM : (tid == E && has_shared ? (T + kBM - 1) / kBM : 0);
  part[tid] = n;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int add = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  if (tid <= E + 1) tile_start[tid] = tid > 0 ? part[tid - 1] : 0;
}

// One K step of 64: each thread carries 16 B of codes and the two UE4M3 scales
// of one A row and of one B row (32 elements each).
struct Stage {
  uint4 aq, bq;
  uint32_t as, bs;
};

// A (activation rows, A4 codes) x B (weight rows, NVFP4 codes), both decoded to
// FP16 in LDS; 4 waves, wave (wm, wn) owns a 64 x 64 quadrant as 2 x 2 MFMA tiles.
// kGateUp: B rows 0..63 are gate columns, 64..127 the matching up columns, and
// wave w covers h columns 32*(w%2).. of both.
template <bool kGateUp>
__device__ __forceinline__ void tile_mma(const uint8_t* __restrict__ arow_q, const uint8_t* __restrict__ arow_s,
                                         const uint8_t* __restrict__ brow_q, const uint8_t* __restrict__ brow_s,
                                         int K, half_t* As, half_t* Bs, floatx16 (&acc)[2][2]) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int r = tid >> 1, hf = tid & 1;  // loader row and 32-element half of the K step
  const int wm = (wave >> 1) * 64;
  const int wn = kGateUp ? (wave & 1) * 32 : (wave & 1) * 64;
  auto fetch = [&](int k0, Stage& st) {
    st.aq = *reinterpret_cast<const uint4*>(arow_q + k0 / 2 + hf * 16);
    st.as = *reinterpret_cast<const uint16_t*>(arow_s + k0 / 16 + hf * 2);
    st.bq = *reinterpret_cast<const uint4*>(brow_q + k0 / 2 + hf * 16);
    st.bs = *reinterpret_cast<const uint16_t*>(brow_s + k0 / 16 + hf * 2);
  };
  Stage st;
  fetch(0, st);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();  // the previous step's fragments are read
    decode32_fp16(st.aq, st.as, &As[r * kLdsStride + hf * 32]);
    decode32_fp16(st.bq, st.bs, &Bs[r * kLdsStride + hf * 32]);
    __syncthreads();
    if (k0 + kBK < K) fetch(k0 + kBK, st);  // next step in flight during the MFMAs
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      half8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const half8_t*>(&As[(wm + 32 * i + (lane & 31)) * kLdsStride + ko]);
      if (kGateUp) {
        b[0] = *reinterpret_cast<const half8_t*>(&Bs[(wn + (lane & 31)) * kLdsStride + ko]);
        b[1] = *reinterpret_cast<const half8_t*>(&Bs[(64 + wn + (lane & 31)) * kLdsStride + ko]);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = *reinterpret_cast<const half8_t*>(&Bs[(wn + 32 * j + (lane & 31)) * kLdsStride + ko]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------- G1
// h codes + scales of every row go to hq / hs (permuted rows, then shared rows);
// the down GEMM reads them back as its A operand.
__global__ __launch_bounds__(256) void k_gateup_mfma(FfnParams p, const int32_t* __restrict__ tile_start,
                                                     const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
                                                     uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ __align__(16) half_t As[kBM * kLdsStride];
  __shared__ __align__(16) half_t Bs[kBN * kLdsStride];
  const int H = p.H, I = p.I, T = p.T, E = p.E;
  const int n_nt = I / 64;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
  const int nseg = E + 1;
  if (mt >= tile_start[nseg]) return;
  const int seg = find_tile(tile_start, nseg, mt);
  const bool shared = seg == E;
  const int seg_row0 = shared ? 0 : p.off[seg];
  const int seg_rows = shared ? T : p.off[seg + 1] - p.off[seg];
  const int m0 = (mt - tile_start[seg]) * kBM;
  const uint8_t* codes = shared ? p.sh13.codes : p.w13.codes + (int64_t)seg * 2 * I * (H / 2);
  const uint8_t* scales = shared ? p.sh13.scales : p.w13.scales + (int64_t)seg * 2 * I * (H / 16);
  const float G = (shared ? p.sh13.gscale[0] : p.w13.gscale[seg]) * p.g_in;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int r = tid >> 1;
  // A row r: the token of tile row r (rows past the segment reuse token 0; dropped)
  int atok = 0;
  if (m0 + r < seg_rows) atok = shared ? m0 + r : p.row2pair[seg_row0 + m0 + r] / p.k;
  // B row r: 0..63 gate columns nt*64.., 64..127 the up columns
  const int64_t wrow = r < 64 ? (int64_t)nt * 64 + r : (int64_t)I + nt * 64 + (r - 64);
  floatx16 acc[2][2] = {};
  tile_mma<true>(xq + (int64_t)atok * (H / 2), xs + (int64_t)atok * (H / 16), codes + wrow * (H / 2),
                 scales + wrow * (H / 16), H, As, Bs, acc);
  // epilogue: lane holds h column wn + (lane & 31) of rows 8*(q/4) + 4*(lane/32) + q%4
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 32;
  const int col = nt * 64 + wn + (lane & 31);
  const float g6 = 6.0f * p.g_mid;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = wm + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      const float g = G * acc[i][0][q], u = G * acc[i][1][q];
      const float h = silu(g) * u;
      float amax = fabsf(h);
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      amax = fmaxf(amax, __shfl_xor(amax, 4));
      amax = fmaxf(amax, __shfl_xor(amax, 8));
      const uint32_t scode = scale_code(amax, g6);
      const float sv = ue4m3_value(scode);
      const uint32_t c = elem_code(h, sv * p.g_mid);
      const uint32_t c_hi = __shfl_xor(c, 1);
      if (m0 + m < seg_rows) {
        const int64_t orow = shared ? (int64_t)T * p.k + m0 + m : (int64_t)seg_row0 + m0 + m;
        const uint8_t byte = (uint8_t)(c | (c_hi << 4));
        if ((col & 1) == 0) hq[orow * (I / 2) + col / 2] = byte;
        if ((col & 15) == 0) hs[orow * (I / 16) + col / 16] = (uint8_t)scode;
        if (p.h_dbg) p.h_dbg[orow * I + col] = h;
        if (p.hq_dbg && (col & 1) == 0) p.hq_dbg[orow * (I / 2) + col / 2] = byte;
        if (p.hs_dbg && (col & 15) == 0) p.hs_dbg[orow * (I / 16) + col / 16] = (uint8_t)scode;
      }
    }
  }
}

// ---------------------------------------------------------------- G2
__global__ __launch_bounds__(256) void k_down_mfma(FfnParams p, const int32_t* __restrict__ tile_start,
                                                   const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs) {
  __shared__ __align__(16) half_t As[kBM * kLdsStride];
  __shared__ __align__(16) half_t Bs[kBN * kLdsStride];
  const int H = p.H, I = p.I, T = p.T, E = p.E;
  const int n_nt = H / kBN;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
  const int nseg = E + 1;
  if (mt >= tile_start[nseg]) return;
  const int seg = find_tile(tile_start, nseg, mt);
  const bool shared = seg == E;
  const int seg_row0 = shared ? 0 : p.off[seg];
  const int seg_rows = shared ? T : p.off[seg + 1] - p.off[seg];
  const int m0 = (mt - tile_start[seg]) * kBM;
  const uint8_t* codes = shared ? p.sh2.codes : p.w2.codes + (int64_t)seg * H * (I / 2);
  const uint8_t* scales = shared ? p.sh2.scales : p.w2.scales + (int64_t)seg * H * (I / 16);
  const float G = (shared ? p.sh2.gscale[0] : p.w2.gscale[seg]) * p.g_mid;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int r = tid >> 1;
  const int arow_i = m0 + r < seg_rows ? m0 + r : 0;
  const int64_t hrow = shared ? (int64_t)T * p.k + arow_i : (int64_t)seg_row0 + arow_i;
  const int64_t wrow = (int64_t)nt * kBN + r;
  floatx16 acc[2][2] = {};
  const int kc0 = p.kc0;  // K range [kc0, kc1) of I (the full sum: 0, I)
  tile_mma<false>(hq + hrow * (I / 2) + kc0 / 2, hs + hrow * (I / 16) + kc0 / 16, codes + wrow * (I / 2) + kc0 / 2,
                  scales + wrow * (I / 16) + kc0 / 16, p.kc1 - kc0, As, Bs, acc);
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nt * kBN + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = wm + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (m0 + m < seg_rows) {
          float* dst = shared ? p.y_shared + (int64_t)(m0 + m) * H : p.y_rows + (int64_t)(seg_row0 + m0 + m) * H;
          dst[n] = G * acc[i][j][q];
        }
      }
    }
}

// ---------------------------------------------------------------- launchers
bool ffn_mfma_supported(int H, int I, int E) {
  return H % kBN == 0 && H % kBK == 0 && I % 64 == 0 && I % kBK == 0 && E <= 1000;
}

size_t ffn_mfma_ws_bytes(int E) { return (size_t)(E + 2) * sizeof(int32_t); }

hipError_t launch_ffn_mfma(const FfnParams& p, int32_t* tile_start, const uint8_t* xq, const uint8_t* xs,
                           uint8_t* hq, uint8_t* hs, hipStream_t s, hipEvent_t* ev) {
  const int64_t P = (int64_t)p.T * p.k;
  const int64_t max_tiles = (P + kBM - 1) / kBM + (P < p.E ? P : p.E) + (p.has_shared ? (p.T + kBM - 1) / kBM : 0);
  hipLaunchKernelGGL(k_tile_map, dim3(1), dim3(1024), 0, s, p.off, p.E, p.T, p.has_shared, tile_start);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_timed(k_gateup_mfma, dim3((unsigned)(max_tiles * (p.I / 64))), dim3(256), 0, s, ev ? ev[2] : nullptr,
                   ev ? ev[3] : nullptr, p, (const int32_t*)tile_start, xq, xs, hq, hs);
  if (e != hipSuccess) return e;
  return launch_timed(k_down_mfma, dim3((unsigned)(max_tiles * (p.H / kBN))), dim3(256), 0, s, ev ? ev[4] : nullptr,
                      ev ? ev[5] : nullptr, p, (const int32_t*)tile_start, (const uint8_t*)hq, (const uint8_t*)hs);
}

}  // namespace moe

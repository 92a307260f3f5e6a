// Expert FFN by weight streaming: each selected expert's NVFP4 rows are read
// once from HBM and dotted with the (few) activation rows routed to it.  This
// is the decode-shaped path (1-4 tokens: every weight byte is used by about one
// row, so the work is bound by streaming the packed weights).
//
// Per 16-element block the product is exact in FP32: e2m1 * dequantized A4
// activation has <= 8 significant bits and a block sum of 16 such products
// stays an exact multiple of the activation scale; the block result times the
// weight's UE4M3 scale is exact too, and blocks are accumulated in FP32
// (Richland article, "Why it matters": partials accumulate in FP32).
//
// Kernel F1 (gate/up + SwiGLU + A4(h)): one workgroup per (expert slot, block
// of 16 intermediate columns).  The 32 weight rows (16 gate + 16 up) are split
// over 8 threads each; thread (row, j) accumulates the 32-element chunks j,
// j+8, ... of its row in order, and the 8 partials are summed in a fixed order
// (deterministic).  Then 16 lanes per activation row form h = silu(g) * u,
// encode the 16-block and write the dequantized FP16 h for the down kernel.
// Kernel F2 (down): one workgroup per (expert slot, 32 rows of W2).
#include "common.hpp"

namespace moe {

constexpr int kRB = 4;      // activation rows processed together
constexpr int kSub = 8;     // threads per weight row
constexpr int kWRows = 32;  // weight rows per workgroup (256 threads / kSub)

// dot of one 32-element chunk: weight codes (16 B), two UE4M3 scales, FP16 activations
__device__ __forceinline__ float chunk_dot(uint4 q, uint32_t s0, uint32_t s1, const half_t* __restrict__ a) {
  const uint32_t words[4] = {q.x, q.y, q.z, q.w};
  const half8_t* a8 = reinterpret_cast<const half8_t*>(a);
  float blk[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t word = words[2 * b + w];
      const half8_t av = a8[2 * b + w];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += e2m1_value((word >> (4 * i)) & 15u) * (float)av[i];
    }
    blk[b] = acc;
  }
  return blk[0] * ue4m3_value(s0) + blk[1] * ue4m3_value(s1);
}

struct SlotInfo {
  int e, row0, nrows;
  bool shared;
};

__device__ __forceinline__ bool resolve_slot(const FfnParams& p, int slot, SlotInfo* si) {
  if (p.has_shared && slot == p.n_routed_slots) {
    si->e = 0;
    si->row0 = 0;
    si->nrows = p.T;
    si->shared = true;
    return true;
  }
  si->shared = false;
  si->e = find_active_expert(p.off, p.E, slot, &si->row0, &si->nrows);
  return si->e >= 0;
}

// token of an activation row: routed rows through row2pair, shared rows are tokens
__device__ __forceinline__ int row_token(const FfnParams& p, const SlotInfo& si, int r) {
  return si.shared ? r : p.row2pair[si.row0 + r] / p.k;
}

// output row index into hh / debug dumps
__device__ __forceinline__ int64_t out_row(const FfnParams& p, const SlotInfo& si, int r) {
  return si.shared ? (int64_t)p.T * p.k + r : (int64_t)si.row0 + r;
}

__global__ __launch_bounds__(256) void k_ffn_gateup(FfnParams p) {
  const int n_hb = p.I / 16;
  const int hb = blockIdx.x % n_hb, slot = blockIdx.x / n_hb;
  SlotInfo si;
  if (!resolve_slot(p, slot, &si)) return;
  const moe_nvfp4_bank& B = si.shared ? p.sh13 : p.w13;
  const int H = p.H, I = p.I;
  const int64_t rowb = H / 2, srow = H / 16;
  const uint8_t* Q = B.codes + (int64_t)si.e * 2 * I * rowb;
  const uint8_t* S = B.scales + (int64_t)si.e * 2 * I * srow;
  const float G = B.gscale[si.e] * p.g_in;

  const int tid = threadIdx.x;
  const int wr = tid / kSub, sub = tid % kSub;  // weight row 0..31 (0-15 gate, 16-31 up), sub-thread
  const int64_t wrow = wr < 16 ? (int64_t)hb * 16 + wr : (int64_t)I + hb * 16 + (wr - 16);
  const uint8_t* q_row = Q + wrow * rowb;
  const uint8_t* s_row = S + wrow * srow;
  const int nch = H / 32;

  __shared__ float part[kRB][kWRows][kSub + 1];
  __shared__ int toks[kRB];

  for (int r0 = 0; r0 < si.nrows; r0 += kRB) {
    const int nr = min(kRB, si.nrows - r0);
    if (tid < nr) toks[tid] = row_token(p, si, r0 + tid);
    __syncthreads();
    float acc[kRB] = {};
    for (int ch = sub; ch < nch; ch += kSub) {
      const uint4 q = *reinterpret_cast<const uint4*>(q_row + ch * 16);
      const uint32_t s0 = s_row[2 * ch], s1 = s_row[2 * ch + 1];
#pragma unroll
      for (int rr = 0; rr < kRB; ++rr)
        if (rr < nr) acc[rr] += chunk_dot(q, s0, s1, p.xh + (int64_t)toks[rr] * H + ch * 32);
    }
#pragma unroll
    for (int rr = 0; rr < kRB; ++rr) part[rr][wr][sub] = acc[rr];
    __syncthreads();
    // 16 lanes per activation row: lane i owns h column hb*16 + i
    if (tid < kRB * 16) {
      const int rr = tid / 16, i = tid % 16;
      float gsum = 0.0f, usum = 0.0f;
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        gsum += part[rr][i][j];
        usum += part[rr][16 + i][j];
      }
      const float g = G * gsum, u = G * usum;
      const float h = silu(g) * u;
      float amax = fabsf(h);
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
      const uint32_t sc = scale_code(amax, (p.act8 ? 127.0f : 6.0f) * p.g_mid);
      const float sv = ue4m3_value(sc);
      const uint32_t c = p.act8 ? (uint32_t)int8_code(h, sc ? sv * p.g_mid : __builtin_inff())
                                : elem_code(h, sv * p.g_mid);
      const uint32_t c_hi = __shfl_down(c, 1, 16);
      if (rr < nr) {
        const int64_t orow = out_row(p, si, r0 + rr);
        const int64_t col = (int64_t)hb * 16 + i;
        p.hh[orow * I + col] = p.act8 ? (half_t)((float)(int)c * sv) : (half_t)(e2m1_value(c) * sv);
        if (p.h_dbg) p.h_dbg[orow * I + col] = h;
        if (p.hq_dbg && p.act8) p.hq_dbg[orow * I + col] = (uint8_t)(c & 0xFFu);
        if (p.hq_dbg && !p.act8 && (i & 1) == 0) p.hq_dbg[orow * (I / 2) + col / 2] = (uint8_t)(c | (c_hi << 4));
        if (p.hs_dbg && i == 0) p.hs_dbg[orow * (I / 16) + hb] = (uint8_t)sc;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_ffn_down(FfnParams p) {
  const int n_nb = p.H / kWRows;
  const int nb = blockIdx.x % n_nb, slot = blockIdx.x / n_nb;
  SlotInfo si;
  if (!resolve_slot(p, slot, &si)) return;
  const moe_nvfp4_bank& B = si.shared ? p.sh2 : p.w2;
  const int H = p.H, I = p.I;
  const int64_t rowb = I / 2, srow = I / 16;
  const uint8_t* Q = B.codes + (int64_t)si.e * H * rowb;
  const uint8_t* S = B.scales + (int64_t)si.e * H * srow;
  const float G = B.gscale[si.e] * p.g_mid;

  const int tid = threadIdx.x;
  const int wr = tid / kSub, sub = tid % kSub;
  const int64_t n = (int64_t)nb * kWRows + wr;
  const uint8_t* q_row = Q + n * rowb;
  const uint8_t* s_row = S + n * srow;
  const int ch0 = p.kc0 / 32, ch1 = p.kc1 / 32;  // K range of the down projection
  __shared__ float part[kRB][kWRows][kSub + 1];

  for (int r0 = 0; r0 < si.nrows; r0 += kRB) {
    const int nr = min(kRB, si.nrows - r0);
    float acc[kRB] = {};
    for (int ch = ch0 + sub; ch < ch1; ch += kSub) {
      const uint4 q = *reinterpret_cast<const uint4*>(q_row + ch * 16);
      const uint32_t s0 = s_row[2 * ch], s1 = s_row[2 * ch + 1];
#pragma unroll
      for (int rr = 0; rr < kRB; ++rr)
        if (rr < nr) acc[rr] += chunk_dot(q, s0, s1, p.hh + out_row(p, si, r0 + rr) * I + ch * 32);
    }
#pragma unroll
    for (int rr = 0; rr < kRB; ++rr) part[rr][wr][sub] = acc[rr];
    __syncthreads();
    if (tid < kRB * kWRows) {
      const int rr = tid / kWRows, w = tid % kWRows;
      if (rr < nr) {
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < kSub; ++j) sum += part[rr][w][j];
        const float y = G * sum;
        const int64_t col = (int64_t)nb * kWRows + w;
        if (si.shared)
          p.y_shared[(int64_t)(r0 + rr) * H + col] = p.sh_gate ? y * p.sh_gate[r0 + rr] : y;
        else
          p.y_rows[(int64_t)(si.row0 + r0 + rr) * H + col] = y;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_ffn_gateup(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const int slots = p.n_routed_slots + (p.has_shared ? 1 : 0);
  if (slots == 0) return record_idle(s, ev_before, ev_after);
  return launch_timed(k_ffn_gateup, dim3((unsigned)(slots * (p.I / 16))), dim3(256), 0, s, ev_before, ev_after, p);
}

hipError_t launch_ffn_down(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const int slots = p.n_routed_slots + (p.has_shared ? 1 : 0);
  if (slots == 0) return record_idle(s, ev_before, ev_after);
  return launch_timed(k_ffn_down, dim3((unsigned)(slots * (p.H / kWRows))), dim3(256), 0, s, ev_before, ev_after,
                      p);
}

}  // namespace moe

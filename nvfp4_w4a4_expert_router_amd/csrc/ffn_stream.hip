// Expert FFN by weight streaming, tuned for decode (a few tokens: each weight
// byte of a selected expert is used by about one activation row, so the work
// is bound by streaming packed NVFP4 weights from HBM).
//
// Arithmetic (Richland article, "What shipped" / "Why it matters": E2M1 codes,
// UE4M3 block scales, FP32 per-expert scale, FP32 accumulation):
//   weight nibbles -> FP16 with v_cvt_scalef32_pk_f16_fp4 (scale 1.0: exact
//   E2M1 values); the activation is the dequantized A4 value e2m1 * ue4m3
//   (exact in FP16); v_dot2_f32_f16 sums a 16-element block, exactly (the
//   block sum is a multiple of the activation scale below 2^12 of it); the
//   block sum times the weight's UE4M3 scale is exact; blocks accumulate in
//   FP32; the per-expert scale is applied once at the end.
//
// Kernel G (gate/up + SwiGLU + A4(h)), one workgroup per (expert slot, block of
// 16 intermediate columns): the 32 weight rows (16 gate, 16 up) are read with
// 8 threads per row, every load issued before any arithmetic.  The block's
// activation rows are A4-encoded from BF16 into LDS by the workgroup itself
// (no separate launch).  8-lane butterflies finish each row's dot product in a
// fixed order; 16 lanes per activation row then form h = silu(g) * u, encode
// the 16-block and store the dequantized FP16 h for the down kernel.
// Kernel D (down), one workgroup per (expert slot, 2048/(I/32) rows of W2):
// I/32 lanes per row, 8 rows per thread, all loads issued up front.
#include "common.hpp"

namespace moe {

// ---------------------------------------------------------------- helpers
// Slot -> expert: the s-th expert with a nonzero count.  Lane l scans experts
// [l*G, l*G+G) (G = ceil(E/64)); every load is issued at once.
__device__ __forceinline__ int active_expert(const int32_t* __restrict__ off, int E, int s, int* row0, int* cnt) {
  const int lane = lane_id();
  const int G = (E + kWave - 1) / kWave;  // <= 16
  int o[17];
#pragma unroll
  for (int i = 0; i < 17; ++i) {
    const int e = lane * G + i;
    o[i] = (i <= G && e <= E) ? off[e] : 0;
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = lane * G + i;
    if (i < G && e < E && o[i + 1] > o[i]) m |= 1u << i;
  }
  const int n = __popc(m);
  int incl = n;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  const int excl = incl - n;
  const bool mine = s >= excl && s < incl;
  const uint64_t who = __ballot(mine);
  if (who == 0) return -1;
  const int L = __ffsll((long long)who) - 1;
  int e = -1, r0 = 0, c = 0;
  if (mine) {
    int want = s - excl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((m >> i) & 1u) {
        if (want == 0 && e < 0) {
          e = lane * G + i;
          r0 = o[i];
          c = o[i + 1] - o[i];
        }
        --want;
      }
    }
  }
  *row0 = __shfl(r0, L);
  *cnt = __shfl(c, L);
  return __shfl(e, L);
}

struct Slot {
  int e, row0, nrows;
  bool shared;
};

__device__ __forceinline__ bool slot_expert(const FfnParams& p, int slot, Slot* si) {
  if (p.has_shared && slot == p.n_routed_slots) {
    *si = Slot{0, 0, p.T, true};
    return true;
  }
  si->shared = false;
  si->e = active_expert(p.off, p.E, slot, &si->row0, &si->nrows);
  return si->e >= 0;
}

// 8 weight nibbles (one dword) against 8 FP16 activations, accumulated into c
__device__ __forceinline__ float dot8(uint32_t w, half8_t a, float c) {
  c = __builtin_amdgcn_fdot2(fp4x2<0>(w), half2_t{a[0], a[1]}, c, false);
  c = __builtin_amdgcn_fdot2(fp4x2<1>(w), half2_t{a[2], a[3]}, c, false);
  c = __builtin_amdgcn_fdot2(fp4x2<2>(w), half2_t{a[4], a[5]}, c, false);
  c = __builtin_amdgcn_fdot2(fp4x2<3>(w), half2_t{a[6], a[7]}, c, false);
  return c;
}

// one 32-element chunk: codes (16 B = two blocks), the two UE4M3 scales packed
// in sc2 (block 0 in the low byte), 32 FP16 activations
__device__ __forceinline__ float chunk32(uint4 q, uint32_t sc2, half8_t a0, half8_t a1, half8_t a2, half8_t a3) {
  float b0 = dot8(q.x, a0, 0.0f);
  b0 = dot8(q.y, a1, b0);
  float b1 = dot8(q.z, a2, 0.0f);
  b1 = dot8(q.w, a3, b1);
  return b0 * ue4m3_value(sc2 & 0xFFu) + b1 * ue4m3_value((sc2 >> 8) & 0xFFu);
}

// ---------------------------------------------------------------- kernel G
constexpr int kGSub = 8;    // threads per weight row
constexpr int kGRows = 32;  // weight rows per workgroup
constexpr int kGChunks = 8; // 32-element chunks per thread held in registers
constexpr int kGRB = 4;     // activation rows per pass

__global__ __launch_bounds__(256) void k_gateup_stream(FfnParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);                                        // [kGRB][H]
  float* gu = reinterpret_cast<float*>(smem + (size_t)kGRB * p.H * sizeof(half_t));    // [kGRB][32]
  int* toks = reinterpret_cast<int*>(gu + kGRB * kGRows);                                // [kGRB]

  const int I = p.I, H = p.H;
  const int n_hb = I / 16;
  const int hb = blockIdx.x % n_hb, slot = blockIdx.x / n_hb;
  Slot si;
  if (!slot_expert(p, slot, &si)) return;
  const moe_nvfp4_bank& B = si.shared ? p.sh13 : p.w13;
  const float G = B.gscale[si.e] * p.g_in;
  const int tid = threadIdx.x;
  const int r = tid / kGSub, sub = tid % kGSub;
  const int64_t wrow = (int64_t)si.e * 2 * I + (r < 16 ? hb * 16 + r : I + hb * 16 + (r - 16));
  const uint8_t* qrow = B.codes + wrow * (H / 2);
  const uint8_t* srow = B.scales + wrow * (H / 16);
  const int per = H / (32 * kGSub);  // chunks per thread (H % 256 == 0)

  // weights of the first group, issued before the activation staging
  uint4 q[kGChunks];
  uint32_t sc[kGChunks];
#pragma unroll
  for (int j = 0; j < kGChunks; ++j) {
    const int ch = sub + kGSub * j;
    if (j < per) {
      q[j] = *reinterpret_cast<const uint4*>(qrow + ch * 16);
      sc[j] = *reinterpret_cast<const uint16_t*>(srow + ch * 2);
    }
  }
  const float g6 = 6.0f * p.g_in;
  for (int r0 = 0; r0 < si.nrows; r0 += kGRB) {
    const int nr = min(kGRB, si.nrows - r0);
    if (tid < nr) toks[tid] = si.shared ? r0 + tid : p.row2pair[si.row0 + r0 + tid] / p.k;
    __syncthreads();
    // A4(x) of the activation rows into LDS, one 16-block per task
    for (int task = tid; task < nr * (H / 16); task += 256) {
      const int rr = task / (H / 16), b = task % (H / 16);
      const uint4* src = reinterpret_cast<const uint4*>(p.x + (int64_t)toks[rr] * H + b * 16);
      const uint4 v0 = src[0], v1 = src[1];
      const uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      float v[16];
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(wv[i] << 16);
        v[2 * i + 1] = __uint_as_float(wv[i] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(v[2 * i]), fabsf(v[2 * i + 1])));
      }
      half8_t h0, h1;
      if (p.act8) {  // A8: INT8 codes on a scale from amax / 127
        const uint32_t scode = scale_code(amax, 127.0f * p.g_in);
        const float sv = ue4m3_value(scode);
        const float s = scode ? sv * p.g_in : __builtin_inff();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          h0[i] = (half_t)((float)int8_code(v[i], s) * sv);
          h1[i] = (half_t)((float)int8_code(v[8 + i], s) * sv);
        }
      } else {
        const uint32_t scode = scale_code(amax, g6);
        const float sv = ue4m3_value(scode);
        const float s = sv * p.g_in;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          h0[i] = (half_t)(e2m1_value(elem_code(v[i], s)) * sv);
          h1[i] = (half_t)(e2m1_value(elem_code(v[8 + i], s)) * sv);
        }
      }
      half8_t* dst = reinterpret_cast<half8_t*>(xs + (size_t)rr * H + b * 16);
      dst[0] = h0;
      dst[1] = h1;
    }
    __syncthreads();
    float acc[kGRB] = {};
    for (int g0 = 0; g0 < per; g0 += kGChunks) {
      if (g0 > 0) {  // further groups (H > 2048)
#pragma unroll
        for (int j = 0; j < kGChunks; ++j) {
          const int ch = sub + kGSub * (g0 + j);
          if (g0 + j < per) {
            q[j] = *reinterpret_cast<const uint4*>(qrow + ch * 16);
            sc[j] = *reinterpret_cast<const uint16_t*>(srow + ch * 2);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kGChunks; ++j) {
        if (g0 + j >= per) break;
        const int ch = sub + kGSub * (g0 + j);
#pragma unroll
        for (int rr = 0; rr < kGRB; ++rr) {
          if (rr >= nr) break;
          const half8_t* a = reinterpret_cast<const half8_t*>(xs + (size_t)rr * H + ch * 32);
          acc[rr] += chunk32(q[j], sc[j], a[0], a[1], a[2], a[3]);
        }
      }
    }
    if (per > kGChunks && r0 + kGRB < si.nrows) {  // reload group 0 for the next rows
#pragma unroll
      for (int j = 0; j < kGChunks; ++j) {
        const int ch = sub + kGSub * j;
        q[j] = *reinterpret_cast<const uint4*>(qrow + ch * 16);
        sc[j] = *reinterpret_cast<const uint16_t*>(srow + ch * 2);
      }
    }
    // 8-lane butterfly: the row's full dot product in every lane of the group
#pragma unroll
    for (int rr = 0; rr < kGRB; ++rr) {
#pragma unroll
      for (int m = 1; m < kGSub; m <<= 1) acc[rr] += __shfl_xor(acc[rr], m);
      if (sub == 0) gu[rr * kGRows + r] = acc[rr];
    }
    __syncthreads();
    if (tid < kGRB * 16) {
      const int rr = tid / 16, i = tid % 16;
      const float g = G * gu[rr * kGRows + i], u = G * gu[rr * kGRows + 16 + i];
      const float h = silu(g) * u;
      float amax = fabsf(h);
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
      const uint32_t scode = scale_code(amax, (p.act8 ? 127.0f : 6.0f) * p.g_mid);
      const float sv = ue4m3_value(scode);
      const uint32_t c = p.act8 ? (uint32_t)int8_code(h, scode ? sv * p.g_mid : __builtin_inff())
                                : elem_code(h, sv * p.g_mid);
      const uint32_t c_hi = __shfl_down(c, 1, 16);
      if (rr < nr) {
        const int64_t orow = si.shared ? (int64_t)p.T * p.k + r0 + rr : (int64_t)si.row0 + r0 + rr;
        const int64_t col = (int64_t)hb * 16 + i;
        p.hh[orow * I + col] = p.act8 ? (half_t)((float)(int)c * sv) : (half_t)(e2m1_value(c) * sv);
        if (p.h_dbg) p.h_dbg[orow * I + col] = h;
        if (p.hq_dbg && p.act8) p.hq_dbg[orow * I + col] = (uint8_t)(c & 0xFFu);
        if (p.hq_dbg && !p.act8 && (i & 1) == 0) p.hq_dbg[orow * (I / 2) + col / 2] = (uint8_t)(c | (c_hi << 4));
        if (p.hs_dbg && i == 0) p.hs_dbg[orow * (I / 16) + hb] = (uint8_t)scode;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- kernel D
constexpr int kDRows = 8;  // W2 rows per thread

__global__ __launch_bounds__(256) void k_down_stream(FfnParams p, int lpr_log2) {
  const int I = p.I, H = p.H;
  const int lpr = 1 << lpr_log2;  // lanes per row = I / 32
  const int rpp = 256 >> lpr_log2;  // rows per pass
  const int rows_wg = rpp * kDRows;
  const int n_nb = (H + rows_wg - 1) / rows_wg;
  const int nb = blockIdx.x % n_nb, slot = blockIdx.x / n_nb;
  Slot si;
  if (!slot_expert(p, slot, &si)) return;
  const moe_nvfp4_bank& B = si.shared ? p.sh2 : p.w2;
  const float G = B.gscale[si.e] * p.g_mid;
  const int tid = threadIdx.x;
  const int ch = tid & (lpr - 1), rp = tid >> lpr_log2;
  const int n0 = nb * rows_wg + rp;
  uint4 q[kDRows];
  uint32_t sc[kDRows];
#pragma unroll
  for (int j = 0; j < kDRows; ++j) {
    const int n = n0 + rpp * j;
    if (n < H) {
      const int64_t row = (int64_t)si.e * H + n;
      q[j] = *reinterpret_cast<const uint4*>(B.codes + row * (I / 2) + ch * 16);
      sc[j] = *reinterpret_cast<const uint16_t*>(B.scales + row * (I / 16) + ch * 2);
    }
  }
  for (int rr = 0; rr < si.nrows; ++rr) {
    const int64_t orow = si.shared ? (int64_t)p.T * p.k + rr : (int64_t)si.row0 + rr;
    const half8_t* a = reinterpret_cast<const half8_t*>(p.hh + orow * I + ch * 32);
    const half8_t a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    float part[kDRows];
#pragma unroll
    for (int j = 0; j < kDRows; ++j) part[j] = chunk32(q[j], sc[j], a0, a1, a2, a3);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      if (m >= lpr) break;
#pragma unroll
      for (int j = 0; j < kDRows; ++j) part[j] += __shfl_xor(part[j], m);
    }
    if (ch == 0) {
      float* dst = si.shared ? p.y_shared + (int64_t)rr * H : p.y_rows + ((int64_t)si.row0 + rr) * H;
      const float gr = si.shared && p.sh_gate ? p.sh_gate[rr] : 1.0f;  // shared row rr is token rr
#pragma unroll
      for (int j = 0; j < kDRows; ++j) {
        const int n = n0 + rpp * j;
        if (n < H) dst[n] = si.shared && p.sh_gate ? (G * part[j]) * gr : G * part[j];
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
bool ffn_stream_supported(int H, int I) {
  const int lpr = I / 32;
  return H % 256 == 0 && lpr >= 1 && lpr <= 64 && (lpr & (lpr - 1)) == 0;
}

hipError_t launch_gateup_stream(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const int slots = p.n_routed_slots + (p.has_shared ? 1 : 0);
  const size_t lds = (size_t)kGRB * p.H * sizeof(half_t) + kGRB * kGRows * sizeof(float) + kGRB * sizeof(int);
  if (slots == 0) return record_idle(s, ev_before, ev_after);
  return launch_timed(k_gateup_stream, dim3((unsigned)(slots * (p.I / 16))), dim3(256), (uint32_t)lds, s, ev_before,
                      ev_after, p);
}

hipError_t launch_down_stream(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const int slots = p.n_routed_slots + (p.has_shared ? 1 : 0);
  int lg = 0;
  while ((1 << lg) < p.I / 32) ++lg;
  const int rows_wg = (256 >> lg) * kDRows;
  const int n_nb = (p.H + rows_wg - 1) / rows_wg;
  if (slots == 0) return record_idle(s, ev_before, ev_after);
  return launch_timed(k_down_stream, dim3((unsigned)(slots * n_nb)), dim3(256), 0, s, ev_before, ev_after, p, lg);
}

}  // namespace moe

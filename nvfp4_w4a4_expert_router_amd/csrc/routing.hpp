// Routing of a decode batch (T <= 4 tokens) from its FP64 logits, inside one
// 256-thread workgroup: the top k of every token (wave t takes token t),
// softmax weights, the permutation (expert ascending, token ascending) and the
// slot table of the decode expert kernels.  Top-k routing over 512 experts
// with 10 routed per token (capy-flash README v0.5.4, synthetic test-artifact
// script; Richland article, "What shipped").
//
// route_select works in LDS only and ends with a barrier; route_publish writes
// the call's routing outputs.  The fused decode gate/up kernel runs
// route_select in each routed workgroup (which then knows its slot's expert
// without a dependent load of a table written by another kernel) and one extra
// workgroup runs both and publishes.
#pragma once
#include "common.hpp"

namespace moe {

constexpr int kRdMaxT = 4;  // one wave per token
constexpr int kRdMaxE = 512;

struct RoutingLds {
  TopkScratch ts[kRdMaxT];      // top-k scratch, one per token wave
  unsigned int tmask[kRdMaxE];  // tokens that chose expert e (bit t)
  int off[kRdMaxE + 1];
  int nzr[kRdMaxE];          // experts with pairs and a smaller id (slot of the expert)
  int4 slot[kRdMaxT * 32];   // slot table
  int wsum[4], wnz[4];       // per-wave totals of the scan
};

// ---------------------------------------------------------------- shared-expert gate
// z = sum_h x[t][h] * wg[h] over one wave (FP64 sums of exact BF16 x FP32
// products, a fixed reduction order), then
// gate = fl32(1 / (1 + exp(-z))) in FP64.  An optional gate on the shared
// expert is not on the pages (they list the shared expert as always on); this
// is the plainest form such a gate takes.
__device__ __forceinline__ float shared_gate_wave(const uint16_t* __restrict__ xr, const float* __restrict__ wg,
                                                  int H) {
  const int lane = lane_id();
  double a = 0.0;
  if (H % 8 == 0) {  // 8 elements per lane and step (16-byte loads, four steps in flight)
#pragma unroll 4
    for (int h = 8 * lane; h < H; h += 8 * kWave) {
      const uint4 xv = *reinterpret_cast<const uint4*>(xr + h);
      const float4 w0 = *reinterpret_cast<const float4*>(wg + h);
      const float4 w1 = *reinterpret_cast<const float4*>(wg + h + 4);
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      const float wf[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a = fma((double)__uint_as_float(xw[i] << 16), (double)wf[2 * i], a);
        a = fma((double)__uint_as_float(xw[i] & 0xFFFF0000u), (double)wf[2 * i + 1], a);
      }
    }
  } else {
    for (int h = 2 * lane; h < H; h += 2 * kWave) {
      const uint32_t xv = *reinterpret_cast<const uint32_t*>(xr + h);
      const float2 w = *reinterpret_cast<const float2*>(wg + h);
      a = fma((double)__uint_as_float(xv << 16), (double)w.x, a);
      a = fma((double)__uint_as_float(xv & 0xFFFF0000u), (double)w.y, a);
    }
  }
  const double z = wave_sum_f64(a);
  return (float)(1.0 / (1.0 + exp(-z)));
}

// this lane's selected expert and weight (lanes < k of waves < T), and the
// number of slots (experts with at least one pair)
struct RouteSel {
  int my_e;
  float my_w;
  int n_slots;
};

// Rows of an expert are in token order, so a pair's row is the expert's offset
// plus the number of earlier tokens in the expert's token mask.  kWeights:
// also form the softmax weights (only the publishing workgroup needs them).
template <bool kWeights>
__device__ __forceinline__ RouteSel route_select(const RouteDecodeParams& q, RoutingLds& R) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int T = q.T, E = q.E, k = q.k;
  // the logits loads first; the token masks are cleared while they are in flight
  double v[8];
  int id[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + kWave * j;
    const bool ok = wave < T && e < E;
    v[j] = ok ? q.logits[(int64_t)wave * E + e] : -INFINITY;
    id[j] = ok ? e : 0x7FFFFFFF;
  }
  for (int e = tid; e < E; e += 256) R.tmask[e] = 0u;
  __syncthreads();
  RouteSel rs = {0, 0.0f, 0};
  if (wave < T) {
    double my_v = 0.0;
    wave_topk512(v, id, k, R.ts[wave], &my_v, &rs.my_e);
    if (kWeights) rs.my_w = topk_softmax_weight(my_v, k);
    if (lane < k) atomicOr(&R.tmask[rs.my_e], 1u << wave);
  }
  __syncthreads();
  // scan over the experts, thread tid owning experts 2 tid and 2 tid + 1 (E <=
  // 512): pair counts and nonzero counts, wave scans, then the wave totals
  unsigned int tm[2];
  int c[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = 2 * tid + j;
    tm[j] = e < E ? R.tmask[e] : 0u;
    c[j] = __popc(tm[j]);
  }
  const int sc = c[0] + c[1], snz = (c[0] > 0) + (c[1] > 0);
  const int ic = wave_incl_scan_i32(sc), inz = wave_incl_scan_i32(snz);
  if (lane == kWave - 1) {
    R.wsum[wave] = ic;
    R.wnz[wave] = inz;
  }
  __syncthreads();
  int rc = ic - sc, rnz = inz - snz;
  for (int w = 0; w < wave; ++w) {
    rc += R.wsum[w];
    rnz += R.wnz[w];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int e = 2 * tid + j;
    if (e < E) {
      R.off[e] = rc;
      R.nzr[e] = rnz;
    }
    // slot entry: expert, first row, rows, tokens (one byte each, ascending);
    // at most 4 tokens (bits of tm), peeled without a loop
    const unsigned int t1 = tm[j] & (tm[j] - 1u), t2 = t1 & (t1 - 1u), t3 = t2 & (t2 - 1u);
    auto low = [](unsigned int t) { return t ? (unsigned)(__ffs(t) - 1) : 0u; };  // bytes past the count: 0
    const unsigned int toks = low(tm[j]) | low(t1) << 8 | low(t2) << 16 | low(t3) << 24;
    if (c[j] > 0) R.slot[rnz] = make_int4(e, rc, c[j], (int)toks);
    rc += c[j];
    rnz += c[j] > 0;
  }
  if (tid == 255) R.off[E] = rc;  // the last thread's running count is the total
  __syncthreads();
  rs.n_slots = R.wnz[0] + R.wnz[1] + R.wnz[2] + R.wnz[3];
  return rs;
}

// the call's routing outputs: expert_off, the slot table, ids, weights, the
// permutation and the shared expert's gate values
__device__ __forceinline__ void route_publish(const RouteDecodeParams& q, const RoutingLds& R, const RouteSel& rs) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int T = q.T, E = q.E, k = q.k, P = T * k;
  for (int e = tid; e <= E; e += 256) q.off[e] = R.off[e];
  for (int s = tid; s < P; s += 256) q.slot_tab[s] = s < rs.n_slots ? R.slot[s] : make_int4(-1, 0, 0, 0);
  if (wave < T && lane < k) {
    const int pi = wave * k + lane;
    const int row = R.off[rs.my_e] + __popc(R.tmask[rs.my_e] & ((1u << wave) - 1u));
    q.idx[pi] = rs.my_e;
    q.w[pi] = rs.my_w;
    q.p2r[pi] = row;
    q.r2p[row] = pi;
  }
  if (q.wg && wave < T) {  // the shared expert's gate of token `wave`
    const float g = shared_gate_wave(q.x + (int64_t)wave * q.H, q.wg, q.H);
    if (lane == 0) q.gate[wave] = g;
  }
}

}  // namespace moe

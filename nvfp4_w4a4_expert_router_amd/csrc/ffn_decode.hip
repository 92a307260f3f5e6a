// Expert FFN for decode batches (T <= 8 tokens), weight streaming with every
// load of a workgroup issued in one burst.
//
// At decode each selected expert's weights are used by about one token, so
// the kernels are bound by streaming packed NVFP4 bytes from HBM, and with
// only ~40 experts per call the time is mostly memory latency.  Two choices
// follow from that:
//   * each gate/up thread holds 16 x 16 B of weight codes plus their scales in
//     registers (a down-projection thread 8, which doubles the workgroups of
//     the smaller W2 burst), so one round of resident workgroups covers the
//     whole call;
//   * loads are issued in dependency order with nothing else in between:
//     HIP's vmcnt waits are in order, so a load issued after the weight burst
//     could not be consumed before the whole burst had arrived.
// Arithmetic is the one of the streaming kernels: FP4->FP16 conversion (exact
// E2M1 values), v_dot2_f32_f16 over a 16-element block (exact), times the
// weight's UE4M3 scale (exact), FP32 accumulation (Richland article, "What
// shipped" and "Why it matters").  Dot products are finished by recursive
// halving across lanes (fixed pairing: deterministic).
#include <type_traits>

#include "common.hpp"
#include "routing.hpp"

namespace moe {

bool ffn_stream_supported(int H, int I);

namespace {

// A pointer that is the same in every lane, held as a scalar value, in the
// global address space (so that loads through it are global, not flat, loads).
template <typename P>
__device__ __forceinline__ const __attribute__((address_space(1))) P* uniform_ptr(const P* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const __attribute__((address_space(1))) P*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float dot8(uint32_t w, half8_t a, float c) {
  c = __builtin_amdgcn_fdot2(fp4x2<0>(w), half2_t{a[0], a[1]}, c, false);
  c = __builtin_amdgcn_fdot2(fp4x2<1>(w), half2_t{a[2], a[3]}, c, false);
  c = __builtin_amdgcn_fdot2(fp4x2<2>(w), half2_t{a[4], a[5]}, c, false);
  c = __builtin_amdgcn_fdot2(fp4x2<3>(w), half2_t{a[6], a[7]}, c, false);
  return c;
}

// 32 elements: codes (two blocks), scales of the two blocks in sc2 (low byte
// first), FP16 activations a[0..3]
__device__ __forceinline__ float chunk32(uint4 q, uint32_t sc2, const half8_t* a) {
  float b0 = dot8(q.x, a[0], 0.0f);
  b0 = dot8(q.y, a[1], b0);
  float b1 = dot8(q.z, a[2], 0.0f);
  b1 = dot8(q.w, a[3], b1);
  // one fixed contraction, so every kernel that uses it rounds alike
  return __builtin_fmaf(b0, ue4m3_value(sc2 & 0xFFu), b1 * ue4m3_value((sc2 >> 8) & 0xFFu));
}

// Opaque copy: keeps the compiler from hoisting the FP4 decode of loop-
// invariant weights out of the activation-row loop (which would hold 256
// decoded registers per thread and cut occupancy).
__device__ __forceinline__ uint4 opaque(uint4 v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
  return v;
}

// The value of lane l ^ m (m <= 8) by DPP: quad permutations for 1 and 2, the
// half-row mirror then a quad reversal for 4, a rotation by 8 within the row
// for 8 (lane layouts checked on the device).
template <int m>
__device__ __forceinline__ float xor_lane(float v) {
  const int u = __float_as_int(v);
  if constexpr (m == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0xB1, 0xF, 0xF, true));
  if constexpr (m == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x4E, 0xF, 0xF, true));
  if constexpr (m == 4) {
    const int h = __builtin_amdgcn_update_dpp(0, u, 0x141, 0xF, 0xF, true);  // row_half_mirror
    return __int_as_float(__builtin_amdgcn_update_dpp(0, h, 0x1B, 0xF, 0xF, true));  // quad_perm [3,2,1,0]
  }
  if constexpr (m == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x128, 0xF, 0xF, true));  // row_ror:8
  static_assert(m == 1 || m == 2 || m == 4 || m == 8, "DPP exchange within a row");
  return v;
}

// keep + the partner's send for the pair (x kept by lanes without bit m, y by
// lanes with it; the other value is sent): for m = 16 and 32 one
// v_permlane16/32_swap of (x, y) leaves each lane's keep in one result and
// its partner's send in the other.
template <int m>
__device__ __forceinline__ float pair_sum(float x, float y, bool upper) {
  if constexpr (m == 32) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(y), false, false);
    return __int_as_float(p[0]) + __int_as_float(p[1]);
  } else if constexpr (m == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(y), false, false);
    return __int_as_float(p[0]) + __int_as_float(p[1]);
  } else {
    const float send = upper ? x : y;
    const float keep = upper ? y : x;
    return keep + xor_lane<m>(send);
  }
}

// max(own, lane l ^ m) of a 64-bit value: DPP within a row for m <= 8; for
// m = 16 and 32 one permlane swap of (v, v) leaves the lane's own value in one
// result and its partner's in the other, so the max of the two is the same.
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int m>
__device__ __forceinline__ uint64_t max_with_partner(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  if constexpr (m <= 8) {
    const uint32_t plo = (uint32_t)__float_as_int(xor_lane<m>(__int_as_float((int)lo)));
    const uint32_t phi = (uint32_t)__float_as_int(xor_lane<m>(__int_as_float((int)hi)));
    return umax64(v, ((uint64_t)phi << 32) | plo);
  } else {
    static_assert(m == 16 || m == 32, "partner distance");
    const auto pl = m == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                            : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto ph = m == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                            : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return umax64(((uint64_t)ph[0] << 32) | pl[0], ((uint64_t)ph[1] << 32) | pl[1]);
  }
}

// The expert holding the j-th largest (0-based) of the wave's 512 selection
// keys (lane l holds experts l + 64 q in key[q]; keys are distinct, since each
// carries its expert id, so the j-th is the j-th of the top-k order: logit
// descending, equal logits by lower id).  Registers only: each lane sorts its 8
// keys (a 19-comparator network), then j + 1 rounds take the wave maximum of
// the lanes' leading keys (butterfly over the 64 lanes) and the lane that held
// it drops it.  Every lane returns the same id.
__device__ __forceinline__ int wave_jth_expert(uint64_t (&key)[8], int j) {
  auto ce = [&](int a, int b) {
    const uint64_t x = key[a], y = key[b];
    key[a] = umax64(x, y);
    key[b] = x > y ? y : x;
  };
  ce(0, 2); ce(1, 3); ce(4, 6); ce(5, 7);
  ce(0, 4); ce(1, 5); ce(2, 6); ce(3, 7);
  ce(0, 1); ce(2, 3); ce(4, 5); ce(6, 7);
  ce(2, 4); ce(3, 5);
  ce(1, 4); ce(3, 6);
  ce(1, 2); ce(3, 4); ce(5, 6);
  for (int r = 0;; ++r) {
    uint64_t m = key[0];
    m = max_with_partner<1>(m);
    m = max_with_partner<2>(m);
    m = max_with_partner<4>(m);
    m = max_with_partner<8>(m);
    m = max_with_partner<16>(m);
    m = max_with_partner<32>(m);
    if (r == j) return 1023 - (int)(__builtin_amdgcn_readfirstlane((uint32_t)m) & 0x3FFu);
    if (key[0] == m) {  // one lane: keys are distinct
#pragma unroll
      for (int q = 0; q < 7; ++q) key[q] = key[q + 1];
      key[7] = 0;  // below every key of a finite or infinite logit
    }
  }
}

// Sum v[0..15] over aligned groups of kG lanes by recursive halving (all steps
// resolved at compile time; each step adds a lane's kept value and its
// partner's, so the sums do not depend on how the values move).  Afterwards
// lane l holds the group total of indices base + i for i < max(1, kN / kG),
// where base adds `half` for every halving step whose mask bit the lane has.
template <int kG, int kN>
struct ReduceScatter {
  __device__ __forceinline__ static void run(float (&v)[16], int lane) {
    if constexpr (kG > 1) {
      constexpr int m = kG / 2;
      const bool upper = (lane & m) != 0;
      if constexpr (kN > 1) {
        constexpr int half = kN / 2;
#pragma unroll
        for (int i = 0; i < half; ++i) v[i] = pair_sum<m>(v[i], v[half + i], upper);
        ReduceScatter<m, half>::run(v, lane);
      } else {
        v[0] = pair_sum<m>(v[0], v[0], upper);
        ReduceScatter<m, 1>::run(v, lane);
      }
    }
  }
  __device__ __forceinline__ static int base(int lane) {
    if constexpr (kG > 1 && kN > 1) {
      constexpr int m = kG / 2, half = kN / 2;
      return ((lane & m) ? half : 0) + ReduceScatter<m, half>::base(lane);
    } else {
      return 0;
    }
  }
};

// Slot -> expert (the s-th expert with a nonzero count), one round trip.
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
  // the same in every lane: make it wave-uniform (scalar) for the compiler
  *row0 = __builtin_amdgcn_readfirstlane(__shfl(r0, L));
  *cnt = __builtin_amdgcn_readfirstlane(__shfl(c, L));
  return __builtin_amdgcn_readfirstlane(__shfl(e, L));
}

}  // namespace

constexpr int kDecMaxT = 4;  // the 4-token verify window; larger batches use the streaming kernels

// ---------------------------------------------------------------- gate/up
// Slots: [0, n_routed_slots) routed experts in ascending id order; then the
// shared expert, one slot per token (so no workgroup carries T activation rows).
// A routed slot's expert comes from the slot table of the fused path (one
// load) or from expert_off (one round trip and a wave scan).  The A4 codes of
// x are read from the workspace and decoded to FP16 in LDS while the weight
// burst is in flight.
constexpr int kGuCols = 32;  // intermediate columns per workgroup (gate and up rows: 2 kGuCols)
// kA8: the W4A8 variant (x and h encoded by A8: INT8 codes, one byte each).
// kTable (the fused decode call): each routed workgroup selects the routing of
// all T tokens from the FP64 logits in LDS (route_select) and takes its slot's
// entry from it; the grid's last workgroup also publishes the routing outputs
// (ids, weights, permutation, slot table, shared gate) for the later kernels.
// kPair (with kTable, when the down projection runs with the combine): routed
// slot s is the pair s = t k + j (token t's j-th expert), so its workgroup
// needs only token t's top k (no permutation of the batch), and writes its h
// row at pair s; an expert chosen by several tokens is streamed once per token.
constexpr int kJ = kGuCols / 2;  // weight rows per wave: kJ/2 gate, kJ/2 up
struct GateUpLds {
  half_t xs[kDecMaxT * 2048];  // A4(x) dequantized without g, [T][H]
  uint8_t sct[4][kJ][128];     // each wave's rows' block scales (H/16 bytes)
  float gu[kDecMaxT][2 * kGuCols];
  int toks[kDecMaxT];
};
union DecodeLds {
  RoutingLds route;  // before the weight burst
  GateUpLds gu;      // from the weight burst on
};

template <bool kTable, bool kA8, bool kPair>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_gateup_decode(FfnParams p) {
  static_assert(kTable || !kPair, "pair slots belong to the fused call");
  __shared__ __align__(16) DecodeLds lds;
  half_t* const xs = lds.gu.xs;
  auto& sct = lds.gu.sct;
  auto& gu = lds.gu.gu;
  int* const toks = lds.gu.toks;
  if (kTable && blockIdx.x == gridDim.x - 1) {  // the publishing workgroup
    const RouteSel rs = route_select<true>(p.rq, lds.route);
    route_publish(p.rq, lds.route, rs);
    return;
  }
  const int H = p.H, I = p.I, T = p.T;
  const int n_cg = I / kGuCols;
  const int cg = blockIdx.x % n_cg, slot = blockIdx.x / n_cg;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id();
  const int sh_slot = slot - p.n_routed_slots;
  const bool shared = p.has_shared && sh_slot >= 0;
  // 1. the A4(x) codes (32 elements per thread), then the routing of the
  // batch (fused call, routed slot) from its FP64 logits
  int4 ent = make_int4(0, 0, 0, 0);
  const int xchunks = H / 32;
  const int xt = tid / xchunks, xc = tid % xchunks;
  const bool xmine = xt < T;  // T * H / 32 <= 256
  uint4 xq4 = make_uint4(0u, 0u, 0u, 0u), xq4b = make_uint4(0u, 0u, 0u, 0u);
  uint32_t xs2 = 0u;
  if (xmine) {
    if (kA8) {
      const uint4* src = reinterpret_cast<const uint4*>(p.xq + (size_t)xt * H + xc * 32);
      xq4 = src[0];
      xq4b = src[1];
    } else {
      xq4 = *reinterpret_cast<const uint4*>(p.xq + (size_t)xt * (H / 2) + xc * 16);
    }
    xs2 = *reinterpret_cast<const uint16_t*>(p.xs + (size_t)xt * (H / 16) + xc * 2);
  }
  if (kTable && kPair && !shared) {
    // every wave finds token t's j-th expert by itself (registers only, so no
    // LDS hand-off or barrier): the order of the routing's top k
    const int t = slot / p.k, j = slot % p.k;
    uint64_t key[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int ee = l + kWave * q;
      const bool ok = ee < p.E;
      key[q] = rank_key(ok ? p.rq.logits[(int64_t)t * p.E + ee] : -INFINITY, ok ? ee : 0x7FFFFFFF);
    }
    ent = make_int4(wave_jth_expert(key, j), slot, 1, t);
  } else if (kTable && !shared) {
    const RouteSel rs = route_select<false>(p.rq, lds.route);
    ent = slot < rs.n_slots ? lds.route.slot[slot] : make_int4(-1, 0, 0, 0);
    __syncthreads();  // the routing's LDS is reused from here on
  }
  // 2. this slot's expert and activation rows
  int e, row0, nrows;
  if (shared) {
    e = 0;
    row0 = p.shared_split ? sh_slot : 0;
    nrows = p.shared_split ? 1 : T;
  } else if (kTable) {
    e = __builtin_amdgcn_readfirstlane(ent.x);
    row0 = __builtin_amdgcn_readfirstlane(ent.y);
    nrows = __builtin_amdgcn_readfirstlane(ent.z);
    if (e < 0) return;
  } else {
    e = active_expert(p.off, p.E, slot, &row0, &nrows);
    if (e < 0) return;
  }
  // tokens of the rows and the per-expert scale, then the weight burst (buffer
  // loads: one instruction per 16 B, the row stride in the scalar offset)
  int tok = 0;
  if (!kTable && !shared && tid < nrows) tok = p.row2pair[row0 + tid] / p.k;
  const uint8_t* bcodes = shared ? p.sh13.codes : p.w13.codes;
  const uint8_t* bscales = shared ? p.sh13.scales : p.w13.scales;
  const float gsc = (shared ? p.sh13.gscale : p.w13.gscale)[e];
  const int nch = H / 32;
  const uint32_t qrow = (uint32_t)H / 2, srow = (uint32_t)H / 16;
  const auto rq = buffer_rsrc(bcodes + (int64_t)e * 2 * I * qrow, 2u * I * qrow);
  const auto rs = buffer_rsrc(bscales + (int64_t)e * 2 * I * srow, 2u * I * srow);
  // j < kJ/2: gate column cg*kGuCols + w + 4j; j >= kJ/2: up column w + 4(j - kJ/2) (+ I)
  auto rowoff = [&](int j) { return j < kJ / 2 ? (uint32_t)(4 * j) : (uint32_t)I + 4u * (j - kJ / 2); };
  // the scales of the wave's kJ rows go to LDS first, by transfers of 8 rows
  // (8 lanes x 16 B per row; bytes past a row's H/16 are never read): 2-byte
  // loads per lane and row would cost a load instruction each
#pragma unroll
  for (int c = 0; c < kJ / 8; ++c) {
    const int j = 8 * c + (l >> 3);
    const uint32_t voff = ((uint32_t)(cg * kGuCols + w) + rowoff(j)) * srow + (uint32_t)(l & 7) * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&sct[w][8 * c][0], 16, voff, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // the code burst is issued after the scale transfers
  // lanes past the row's chunks read past the buffer: zeros
  const uint32_t vq = l < nch ? (uint32_t)(cg * kGuCols + w) * qrow + l * 16u : 0x80000000u;
  uint4 q[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) q[j] = buffer_load16_nt(rq, vq, rowoff(j) * qrow);
  __builtin_amdgcn_sched_barrier(0);
  const float G = gsc * p.g_in;
  // 3. A4(x) to FP16 in LDS while the weights are in flight
  if (xmine) {
    if (kA8)
      decode32_a8_fp16(xq4, xq4b, xs2, xs + (size_t)xt * H + xc * 32);
    else
      decode32_fp16(xq4, xs2, xs + (size_t)xt * H + xc * 32);
  }
  if (tid < nrows)
    toks[tid] = shared ? row0 + tid : kPair ? ent.w : kTable ? (int)(((unsigned)ent.w >> (8 * tid)) & 0xFFu) : tok;
  // the scale transfers are complete once at most the kJ code loads are in flight
  static_assert(kJ == 16, "vmcnt immediate below");
  __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt 16, expcnt 7, lgkmcnt 15
  uint32_t sc[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) sc[j] = *reinterpret_cast<const uint16_t*>(&sct[w][j][2 * l]);
  __syncthreads();
  // 4. dot products, one activation row at a time (the first row straight from
  // the loaded codes; later rows through opaque copies, so the compiler cannot
  // keep the decoded weights of the first row live across the loop)
  auto dot_row = [&](int rr, auto reload) {
    half8_t a[4];
    const half8_t* src = reinterpret_cast<const half8_t*>(xs + (size_t)toks[rr] * H + l * 32);
    if (l < nch) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = src[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = half8_t{};
    }
    float acc[16];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      acc[j] = chunk32(decltype(reload)::value ? opaque(q[j]) : q[j], sc[j], a);
      __builtin_amdgcn_sched_barrier(0);  // one chunk at a time: bounded live registers
    }
    ReduceScatter<64, kJ>::run(acc, l);
    // row w + 4j of the tile: gate column w + 4j, or up column w + 4j - kGuCols
    if ((l & (64 / kJ - 1)) == 0) gu[rr][w + 4 * ReduceScatter<64, kJ>::base(l)] = acc[0];
  };
  if (nrows > 0) dot_row(0, std::false_type{});
  for (int rr = 1; rr < nrows; ++rr) dot_row(rr, std::true_type{});
  __syncthreads();
  // 5. SwiGLU + A4(h): kGuCols lanes per activation row (each 16-element block
  // a DPP row of 16 lanes); block maxima and code pairing by DPP, pairs of FP16
  // values stored by the even lanes
  for (int task = tid; task < nrows * kGuCols; task += 256) {
    const int rr = task / kGuCols, i = task % kGuCols;
    const float g = G * gu[rr][i], u = G * gu[rr][kGuCols + i];
    const float h = silu(g) * u;
    const float amax = row16_absmax(h);
    const int64_t orow = shared ? (int64_t)T * p.k + row0 + rr : (int64_t)row0 + rr;
    const int64_t col = (int64_t)cg * kGuCols + i;
    if (kA8) {
      const uint32_t scode = scale_code(amax, 127.0f * p.g_mid);
      const float sv = ue4m3_value(scode);
      const int q = int8_code(h, scode ? sv * p.g_mid : __builtin_inff());
      p.hh[orow * I + col] = (half_t)((float)q * sv);  // exact: <= 11 significant bits
      if (p.hq_dbg) p.hq_dbg[orow * I + col] = (uint8_t)(q & 0xFF);
      if (p.hs_dbg && (i & 15) == 0) p.hs_dbg[orow * (I / 16) + col / 16] = (uint8_t)scode;
    } else {
      const uint32_t scode = scale_code(amax, 6.0f * p.g_mid);
      const float sv = ue4m3_value(scode);
      const uint32_t c = elem_code_s(h, scode ? sv * p.g_mid : __builtin_inff());
      const uint32_t c2 = c | ((uint32_t)__builtin_amdgcn_mov_dpp((int)c, 0xB1, 0xF, 0xF, true) << 4);
      const half2_t hd = fp4x2<0>(c2) * half2_t{(half_t)sv, (half_t)sv};  // exact: <= 6 significant bits
      if ((i & 1) == 0) *reinterpret_cast<uint32_t*>(p.hh + orow * I + col) = __builtin_bit_cast(uint32_t, hd);
      if (p.hq_dbg && (i & 1) == 0) p.hq_dbg[orow * (I / 2) + col / 2] = (uint8_t)c2;
      if (p.hs_dbg && (i & 15) == 0) p.hs_dbg[orow * (I / 16) + col / 16] = (uint8_t)scode;
    }
    if (p.h_dbg) p.h_dbg[orow * I + col] = h;
  }
}

// ---------------------------------------------------------------- down
// W2 rows n, I/32 chunks per row = kLPR lanes per row, 64/kLPR rows per wave
// instruction.  Thread (w, l): chunk l % kLPR of rows
// n0 + (64/kLPR) * (w + 4 j) + l / kLPR, j < kDownLoads.  Eight row loads per
// thread (half a gate/up thread's) give twice the workgroups of sixteen, which
// the few dozen slots of a decode step need to cover the chip.
constexpr int kDownLoads = 8;
template <int kLPR, bool kTable>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_down_decode(FfnParams p) {
  constexpr int kJ = kDownLoads;
  constexpr int kRPI = 64 / kLPR;       // rows per wave instruction
  constexpr int kRowsWG = 4 * kJ * kRPI;
  const int H = p.H, I = p.I, T = p.T;
  const int n_nb = (H + kRowsWG - 1) / kRowsWG;
  const int nb = blockIdx.x % n_nb, slot = blockIdx.x / n_nb;
  const int tid = threadIdx.x, w = tid >> 6, l = lane_id();
  int e, row0, nrows;
  const int sh_slot = slot - p.n_routed_slots;
  const bool shared = p.has_shared && sh_slot >= 0;
  if (shared) {
    e = 0;
    row0 = p.shared_split ? sh_slot : 0;
    nrows = p.shared_split ? 1 : T;
  } else if (kTable) {
    const int4 ent = p.slot_tab[slot];
    e = __builtin_amdgcn_readfirstlane(ent.x);
    row0 = __builtin_amdgcn_readfirstlane(ent.y);
    nrows = __builtin_amdgcn_readfirstlane(ent.z);
    if (e < 0) return;
  } else {
    e = active_expert(p.off, p.E, slot, &row0, &nrows);
    if (e < 0) return;
  }
  const uint8_t* bcodes = shared ? p.sh2.codes : p.w2.codes;
  const uint8_t* bscales = shared ? p.sh2.scales : p.w2.scales;
  const float gsc = (shared ? p.sh2.gscale : p.w2.gscale)[e];
  const int ch = l % kLPR;
  const int base_n = nb * kRowsWG + l / kLPR;
  // activation chunk of the first row, then the weight burst
  const int64_t hrow0 = shared ? (int64_t)T * p.k + row0 : (int64_t)row0;
  half8_t a[4];
  {
    const half8_t* src = reinterpret_cast<const half8_t*>(p.hh + hrow0 * I + ch * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = src[i];
  }
  const uint32_t qrow = (uint32_t)I / 2, srow = (uint32_t)I / 16;
  const auto rq = buffer_rsrc(bcodes + (int64_t)e * H * qrow, (uint32_t)H * qrow);
  const auto rs = buffer_rsrc(bscales + (int64_t)e * H * srow, (uint32_t)H * srow);
  // the scales of the wave's rows first: load j covers kRPI consecutive rows,
  // whose scales are one 128-byte run (kRPI rows x 2 kLPR bytes); the kJ runs
  // go to LDS by one transfer (8 lanes x 16 B per run), and lane l's two bytes
  // of run j sit at byte 2 l (l = row in the run x kLPR + chunk)
  static_assert(kJ * 8 == kWave, "one 16-byte piece per lane");
  __shared__ __align__(16) uint8_t sct[4][kJ][128];
  {
    const uint32_t run0 = (uint32_t)(nb * kRowsWG + kRPI * (w + 4 * (l >> 3)));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&sct[w][0][0], 16, run0 * srow + (uint32_t)(l & 7) * 16u,
                                             0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);  // the code burst is issued after the scale transfer
  const uint32_t n_lane = (uint32_t)(base_n + kRPI * w);
  const uint32_t vq = n_lane * qrow + ch * 16u;
  uint4 q[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j)  // rows past H read past the buffer: zeros
    q[j] = buffer_load16(rq, vq, (uint32_t)(4 * kRPI * j) * qrow);
  __builtin_amdgcn_sched_barrier(0);
  // the scale transfer is complete once at most the kJ code loads are in flight
  static_assert(kJ == 8, "vmcnt immediate below");
  __builtin_amdgcn_s_waitcnt(0xF78);  // vmcnt 8, expcnt 7, lgkmcnt 15
  uint32_t sc[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) sc[j] = *reinterpret_cast<const uint16_t*>(&sct[w][j][2 * l]);
  const float G = gsc * p.g_mid;
  float* dst0 = shared ? p.y_shared + (int64_t)row0 * H : p.y_rows + (int64_t)row0 * H;
  const float* gate = shared && p.sh_gate ? p.sh_gate + row0 : nullptr;  // shared rows are tokens row0..
  // pair ids of the slot's rows for the token-major copy (loaded with the burst in flight)
  int pair[kDecMaxT] = {};
  const bool tok_copy = p.y_tok != nullptr && !shared;
  if (tok_copy)
#pragma unroll
    for (int rr = 0; rr < kDecMaxT; ++rr)
      if (rr < nrows) pair[rr] = p.row2pair[row0 + rr];
  for (int rr = 0; rr < nrows; ++rr) {
    if (rr > 0) {
      const half8_t* src = reinterpret_cast<const half8_t*>(p.hh + (hrow0 + rr) * I + ch * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = src[i];
    }
    float acc[16];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      acc[j] = chunk32(opaque(q[j]), sc[j], a);
      __builtin_amdgcn_sched_barrier(0);
    }
    ReduceScatter<kLPR, kJ>::run(acc, l);
    constexpr int kKeep = kJ / kLPR > 1 ? kJ / kLPR : 1;
    const bool writer = kLPR <= kJ || (l & (kLPR / kJ - 1)) == 0;
    if (writer) {
      const int jb = ReduceScatter<kLPR, kJ>::base(l);
#pragma unroll
      for (int i = 0; i < kKeep; ++i) {
        const int n = base_n + kRPI * (w + 4 * (jb + i));
        if (n < H) {
          dst0[(int64_t)rr * H + n] = gate ? (G * acc[i]) * gate[rr] : G * acc[i];
          if (tok_copy) {
            int pr = pair[0];
#pragma unroll
            for (int r2 = 1; r2 < kDecMaxT; ++r2) pr = rr == r2 ? pair[r2] : pr;
            p.y_tok[(int64_t)pr * H + n] = G * acc[i];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down + combine
// Fused decode path: one workgroup per (token t, kDcCols output columns).
// Lane group j (kLPR lanes, one per 32-element chunk of I) takes the j-th
// expert of the token in rank order (j = k: the shared expert), loads that
// expert's kDcCols W2 rows and the token's h row, and forms the rows' dot
// products with the down kernel's per-lane chunks and lane reduction (the same
// FP32 values).  The rows are written to y_rows / y_shared as the down kernel
// writes them, and the workgroup then combines its columns in LDS in the
// combine kernel's order (j ascending, FMA with the router weight, then the
// shared row, then the residual, one BF16 rounding).  That takes the combine
// kernel and one kernel boundary off the decode chain; the price is that an
// expert chosen by several tokens is read once per token (from the caches
// after the first).
constexpr int kDcCols = 4;  // measured: 4 columns 30.4 us per step at T = 4, 8: 30.7, 16: 31.1
template <int kLPR>
__global__ __launch_bounds__(256) void k_down_combine_decode(FfnParams p) {
  constexpr int kSrow = 2 * kLPR;  // scale bytes per W2 row (I / 16)
  constexpr int kSPieces = kDcCols * kSrow / 16;  // 16-byte scale pieces per expert
  const int H = p.H, I = p.I, T = p.T, k = p.k;
  const int n_cb = H / kDcCols;
  const int t = blockIdx.x / n_cb, n0 = (blockIdx.x % n_cb) * kDcCols;
  const int tid = threadIdx.x, l = lane_id();
  const int j = tid / kLPR, c = tid % kLPR;
  const int n_e = k + (p.has_shared ? 1 : 0);
  const bool live = j < n_e;
  const bool shared = live && j == k;
  __shared__ __align__(16) uint8_t sct[256 / kLPR][kDcCols * kSrow];
  __shared__ float ycomb[256 / kLPR][kDcCols];
  __shared__ float wsh[256 / kLPR];
  // 1. the loads that need no other load, issued together by every lane (at
  // in-range addresses, so that no branch leaves the wait counts uncertain):
  // the pair's expert, permuted row and router weight (written by the
  // routing's publishing workgroup) and the h chunk when its row is known
  // (the shared row; a routed row with pair rows)
  const int pid = t * k + j;
  const bool routed = live && !shared;
  const int pq = routed ? pid : 0;
  const int e_ld = p.rq.idx[pq], y_ld = p.rq.p2r[pq];
  const float w_ld = p.rq.w[pq];
  const bool h_early = live && (shared || p.pair_rows);
  half8_t a[4];
  {
    const int64_t hrow = shared ? (int64_t)T * k + t : h_early ? (int64_t)pid : 0;
    const half8_t* src = reinterpret_cast<const half8_t*>(p.hh + hrow * I + 32 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = src[i];
  }
  __builtin_amdgcn_sched_barrier(0);
  const int e = routed ? e_ld : 0, yrow = routed ? y_ld : 0;
  const float wj = routed ? w_ld : 0.0f;
  // the banks' pointers as wave-uniform values first, then chosen per lane
  // group (selecting between the two structs would fetch the chosen one's
  // fields with vector loads from the argument segment)
  typedef const __attribute__((address_space(1))) uint8_t* gbytes_t;
  typedef const __attribute__((address_space(1))) u32x4* gu32x4_t;
  const gbytes_t bcodes = shared ? uniform_ptr(p.sh2.codes) : uniform_ptr(p.w2.codes);
  const gbytes_t bscales = shared ? uniform_ptr(p.sh2.scales) : uniform_ptr(p.w2.scales);
  const __attribute__((address_space(1))) float* bg = shared ? uniform_ptr(p.sh2.gscale) : uniform_ptr(p.w2.gscale);
  // (ids are non-negative: zero extension, so nothing waits for the loaded id
  // before the loads that do not need it are issued)
  const int64_t row0 = (int64_t)((uint64_t)(uint32_t)e * (uint32_t)H) + n0;
  // 2. the loads that need the expert, in the order they are consumed: the
  // rows' block scales (one 16-byte piece per lane), the h chunk (permuted
  // rows), the gscale, then the code burst
  constexpr int kSPL = (kSPieces + kLPR - 1) / kLPR;  // pieces per lane
  uint4 scv[kSPL];
#pragma unroll
  for (int i = 0; i < kSPL; ++i) scv[i] = make_uint4(0u, 0u, 0u, 0u);
  uint4 q[kDcCols];
  float gsc = 0.0f;
  if (live) {
#pragma unroll
    for (int i = 0; i < kSPL; ++i)
      if (c + kLPR * i < kSPieces) {
        const u32x4 v = *reinterpret_cast<gu32x4_t>(bscales + row0 * kSrow + 16 * (c + kLPR * i));
        scv[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
    if (!h_early) {
      const half8_t* src = reinterpret_cast<const half8_t*>(p.hh + (int64_t)yrow * I + 32 * c);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = src[i];
    }
    gsc = bg[(uint32_t)e];
#pragma unroll
    for (int r = 0; r < kDcCols; ++r) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t>(bcodes + (row0 + r) * (I / 2) + 16 * c));
      q[r] = make_uint4(v.x, v.y, v.z, v.w);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kDcCols; ++r) q[r] = make_uint4(0u, 0u, 0u, 0u);
  }
  const float gate = shared && p.sh_gate ? p.sh_gate[t] : 1.0f;  // used at the end only
  if (j < 256 / kLPR) {
#pragma unroll
    for (int i = 0; i < kSPL; ++i)
      if (c + kLPR * i < kSPieces) *reinterpret_cast<uint4*>(&sct[j][16 * (c + kLPR * i)]) = scv[i];
    if (c == 0) wsh[j] = wj;
  }
  __syncthreads();
  uint32_t sc[kDcCols];
#pragma unroll
  for (int r = 0; r < kDcCols; ++r) sc[r] = *reinterpret_cast<const uint16_t*>(&sct[j < 256 / kLPR ? j : 0][r * kSrow + 2 * c]);
  // 3. the rows' dot products (the down kernel's chunks and reduction)
  float acc[16];
#pragma unroll
  for (int r = 0; r < kDcCols; ++r) {
    acc[r] = chunk32(q[r], sc[r], a);
    __builtin_amdgcn_sched_barrier(0);
  }
  ReduceScatter<kLPR, kDcCols>::run(acc, l);
  const float G = gsc * p.g_mid;
  constexpr int kKeep = kDcCols / kLPR > 1 ? kDcCols / kLPR : 1;
  const bool writer = live && (kLPR <= kDcCols || (l & (kLPR / kDcCols - 1)) == 0);
  if (writer) {
    const int jb = ReduceScatter<kLPR, kDcCols>::base(l);
#pragma unroll
    for (int i = 0; i < kKeep; ++i) {
      const int r = jb + i;
      const float y = shared && p.sh_gate ? (G * acc[i]) * gate : G * acc[i];
      if (shared)
        p.y_shared[(int64_t)t * H + n0 + r] = y;
      else
        p.y_rows[(int64_t)yrow * H + n0 + r] = y;
      ycomb[j][r] = y;
    }
  }
  __syncthreads();
  // 4. the combine of this workgroup's columns
  if (tid < kDcCols) {
    float o = 0.0f;
    for (int jj = 0; jj < k; ++jj) o = fmaf(wsh[jj], ycomb[jj][tid], o);
    if (p.has_shared) o += ycomb[k][tid];
    if (p.residual) o += bf16_to_f32(p.residual[(int64_t)t * H + n0 + tid]);
    p.out[(int64_t)t * H + n0 + tid] = f32_to_bf16_rne(o);
  }
}

// ---------------------------------------------------------------- launchers
bool down_combine_decode_supported(int H, int I, int k, int has_shared) {
  const int lpr = I / 32;
  return H % kDcCols == 0 && lpr >= 2 && lpr <= 64 && (lpr & (lpr - 1)) == 0 &&
         (k + (has_shared ? 1 : 0)) * lpr <= 256;
}

hipError_t launch_down_combine_decode(const FfnParams& p, hipStream_t s, hipEvent_t ev_before,
                                      hipEvent_t ev_after) {
  const int lpr = p.I / 32;
  const int threads = ((p.k + (p.has_shared ? 1 : 0)) * lpr + kWave - 1) / kWave * kWave;
  const dim3 grid((unsigned)(p.T * (p.H / kDcCols))), block((unsigned)threads);
  switch (lpr) {
    case 2: return launch_timed(k_down_combine_decode<2>, grid, block, 0, s, ev_before, ev_after, p);
    case 4: return launch_timed(k_down_combine_decode<4>, grid, block, 0, s, ev_before, ev_after, p);
    case 8: return launch_timed(k_down_combine_decode<8>, grid, block, 0, s, ev_before, ev_after, p);
    case 16: return launch_timed(k_down_combine_decode<16>, grid, block, 0, s, ev_before, ev_after, p);
    case 32: return launch_timed(k_down_combine_decode<32>, grid, block, 0, s, ev_before, ev_after, p);
    default: return launch_timed(k_down_combine_decode<64>, grid, block, 0, s, ev_before, ev_after, p);
  }
}

bool ffn_decode_supported(int H, int I, int64_t T) {
  const int lpr = I / 32;
  return T <= kDecMaxT && H <= 2048 && H % 32 == 0 && I % 32 == 0 && lpr >= 1 && lpr <= 64 &&
         (lpr & (lpr - 1)) == 0;
}

static int decode_slots(const FfnParams& p) {
  return p.n_routed_slots + (p.has_shared ? (p.shared_split ? p.T : 1) : 0);
}

hipError_t launch_gateup_decode(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const int slots = decode_slots(p);
  if (slots == 0) return record_idle(s, ev_before, ev_after);
  // the fused call's grid has one more workgroup: it publishes the routing
  const dim3 grid((unsigned)(slots * (p.I / kGuCols) + (p.slot_tab ? 1 : 0)));
  if (p.act8) {
    if (p.slot_tab && p.pair_rows)
      return launch_timed(k_gateup_decode<true, true, true>, grid, dim3(256), 0, s, ev_before, ev_after, p);
    if (p.slot_tab) return launch_timed(k_gateup_decode<true, true, false>, grid, dim3(256), 0, s, ev_before, ev_after, p);
    return launch_timed(k_gateup_decode<false, true, false>, grid, dim3(256), 0, s, ev_before, ev_after, p);
  }
  if (p.slot_tab && p.pair_rows)
    return launch_timed(k_gateup_decode<true, false, true>, grid, dim3(256), 0, s, ev_before, ev_after, p);
  if (p.slot_tab) return launch_timed(k_gateup_decode<true, false, false>, grid, dim3(256), 0, s, ev_before, ev_after, p);
  return launch_timed(k_gateup_decode<false, false, false>, grid, dim3(256), 0, s, ev_before, ev_after, p);
}

bool fused_decode_supported(int H, int I, int E, int k, int64_t T) {
  return ffn_decode_supported(H, I, T) && route_decode_supported(H, E, k, T);
}

template <bool kTable>
static hipError_t launch_down_lpr(const FfnParams& p, int lpr, dim3 grid, hipStream_t s, hipEvent_t e0,
                                  hipEvent_t e1) {
  switch (lpr) {
    case 1: return launch_timed(k_down_decode<1, kTable>, grid, dim3(256), 0, s, e0, e1, p);
    case 2: return launch_timed(k_down_decode<2, kTable>, grid, dim3(256), 0, s, e0, e1, p);
    case 4: return launch_timed(k_down_decode<4, kTable>, grid, dim3(256), 0, s, e0, e1, p);
    case 8: return launch_timed(k_down_decode<8, kTable>, grid, dim3(256), 0, s, e0, e1, p);
    case 16: return launch_timed(k_down_decode<16, kTable>, grid, dim3(256), 0, s, e0, e1, p);
    case 32: return launch_timed(k_down_decode<32, kTable>, grid, dim3(256), 0, s, e0, e1, p);
    default: return launch_timed(k_down_decode<64, kTable>, grid, dim3(256), 0, s, e0, e1, p);
  }
}

hipError_t launch_down_decode(const FfnParams& p, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  const int slots = decode_slots(p);
  const int lpr = p.I / 32;
  const int rows_wg = 4 * kDownLoads * (64 / lpr);
  const dim3 grid((unsigned)(slots * ((p.H + rows_wg - 1) / rows_wg)));
  if (slots == 0) return record_idle(s, ev_before, ev_after);
  if (p.slot_tab) return launch_down_lpr<true>(p, lpr, grid, s, ev_before, ev_after);
  return launch_down_lpr<false>(p, lpr, grid, s, ev_before, ev_after);
}

}  // namespace moe

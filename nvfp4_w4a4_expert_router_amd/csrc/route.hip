// Router: logits over the experts, top-k per token and softmax over the
// selected logits (512 experts, top-10 routed: capy-flash README v0.5.4,
// synthetic test-artifact script; Richland article, "What shipped").
//
// Changing the summation order of a logit can swap which of two almost equal
// experts makes the top k
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
#include "lds_ring.hpp"
#include "routing.hpp"

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

// ---------------------------------------------------------------- pass A on the matrix cores
// The same FP32 logits with a proven radius, from BF16 matrix-core products.
// Every FP32 router weight is the exact sum of three BF16 pieces (truncation
// leaves at most 16, then 8 significant bits: w = w1 + w2 + w3), and a BF16
// hidden state times a BF16 piece is exact in FP32, so the only errors are the
// FP32 additions.  Each K step of 32 sums the 3 pieces x 2 MFMAs (16 products
// each) into a fresh accumulator: at most 96 additions on any path, counting
// the MFMA's internal sum as sequential.  Step sums join a group sum (8 steps)
// and group sums the running sum: depth 96 + 8 + H/256.  The terms' absolute
// sum is at most (1 + 2^-7 + 2^-14) sum_h |x_h W_eh|; the radius takes unit
// roundoff 2^-23 (any rounding of the MFMA's FP32 adds, not only to nearest).
// The exact router's pass A takes only the first two pieces: the third is
// below 2^-14 |w| for every weight, which adds 2^-14 sum_h |x_h W_eh| to the
// radius (depth 64 + 8 + H/256 for the additions).  Only the candidates
// depend on the radius; the selection and the weights come from the FP64
// logits either way, and the radius stays far below the logits' spacing near
// the k-th value, so there are hardly more candidates for a third less work.
constexpr int RM_T = 256, RM_E = 128, RM_K = 32, RM_S = 3;  // tokens, experts, K step, ring stages

// W [E][H] FP32 -> Wp [3][E][H] BF16 pieces (truncation; exact split)
__global__ __launch_bounds__(256) void k_router_split(const float* __restrict__ W, int64_t n,
                                                      uint16_t* __restrict__ Wp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t u = __float_as_uint(W[i]);
  const float r1 = W[i] - __uint_as_float(u & 0xFFFF0000u);
  const uint32_t u2 = __float_as_uint(r1) & 0xFFFF0000u;
  const float r2 = r1 - __uint_as_float(u2);
  Wp[i] = (uint16_t)(u >> 16);
  Wp[n + i] = (uint16_t)(u2 >> 16);
  Wp[2 * n + i] = (uint16_t)(__float_as_uint(r2) >> 16);
}

// W [E][H] FP32 -> Wp [E][H] BF16, round to nearest even: the operand of the
// reduced-precision (BF16) router mode
__global__ __launch_bounds__(256) void k_router_round_bf16(const float* __restrict__ W, int64_t n,
                                                           uint16_t* __restrict__ Wp) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  Wp[i] = f32_to_bf16_rne(W[i]);
}

// LDS stage: 256 token rows and NP x 128 expert rows of a K step (64 B = 4
// chunks of 16 B per row; chunk c of row r sits in slot c ^ f(r), f(r) = bit 2
// of r plus twice (bit 1 xor bit 3), so the MFMA reads of 16 consecutive rows
// fall in 16 different 16-byte bank groups).  A ring of 3 stages (120 KB with
// 3 pieces, one workgroup per CU) filled by buffer loads that write LDS
// directly, two steps ahead.  The stages are separate LDS variables (so the
// compiler does not make the reads of one wait for the transfers into
// another) and the ring's barrier is ring_barrier.
template <int NP>
struct RouterStage {
  uint4 a[RM_T * 4];
  uint4 b[NP][RM_E * 4];
};
static_assert(RM_S == 3, "three stages, selected at compile time");

typedef short bf16x8_t __attribute__((ext_vector_type(8)));

// logits[t][e] for a 256-token x 128-expert tile; 8 waves, wave w owns tokens
// 32 w.. x all 128 experts as 4 MFMA tiles (each B fragment read from LDS feeds
// one MFMA per wave, each A fragment four).  K order inside a step is
// lane-contiguous (lanes 0..31 supply elements 8s.., lanes 32..63 16+8s.. in
// MFMA s), the same for both operands.
// NP: BF16 pieces per router row (3: the exact split; 2: its first two, the
// exact router's pass A; 1: a BF16 router).
template <int NP>
__global__ __launch_bounds__(512) void k_router_logits_mfma(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ Wp, int T, int H, int E,
                                                            float* __restrict__ logits) {
  static_assert(NP >= 1 && NP <= 3, "pieces");
  __shared__ __align__(16) RouterStage<NP> rs0, rs1, rs2;
  auto stage = [&](auto kc) -> RouterStage<NP>& {
    constexpr int k = decltype(kc)::value % RM_S;
    if constexpr (k == 0) return rs0;
    else if constexpr (k == 1) return rs1;
    else return rs2;
  };
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  // expert tile major within each XCD's run: one XCD keeps one expert tile's
  // router rows (3 pieces x 128 rows x H) in its L2 while token tiles stream by
  const int ntb = (int)gridDim.y;
  const int lt = xcd_tile((int)(blockIdx.y * gridDim.x + blockIdx.x), (int)(gridDim.x * gridDim.y));
  const int t0 = (lt % ntb) * RM_T, e0 = (lt / ntb) * RM_E;
  const int n = H / RM_K;
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x, (uint32_t)T * H * 2u);
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(Wp, (uint32_t)NP * E * H * 2u);
  // transfers: lane -> row (lane / 4) of a 16-row group, slot lane % 4
  auto swz_of = [](int r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); };
  const uint32_t sw = (uint32_t)(((lane & 3) ^ swz_of(lane >> 2)) * 16);
  uint32_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ta = t0 + 32 * wave + 16 * i + (lane >> 2);
    aoff[i] = (uint32_t)(ta < T ? ta : T - 1) * H * 2u + sw;  // rows past T repeat the last; dropped
  }
  const uint32_t boff = (uint32_t)(e0 + (lane >> 2)) * H * 2u + sw;
  // two A and NP B transfers per wave and step (steps past the last repeat it)
  auto dma = [&](int t, RouterStage<NP>& S) {
    const uint32_t k0 = (uint32_t)((t < n ? t : n - 1) * RM_K);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)&S.a[(32 * wave + 16 * i) * 4], 16, aoff[i], k0 * 2, 0,
                                               0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int q = NP * wave + i, pc = q >> 3, c = q & 7;  // piece, 16-row group
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)&S.b[pc][16 * c * 4], 16, boff,
                                               k0 * 2 + (uint32_t)(pc * E + 16 * c) * H * 2u, 0, 0);
    }
  };
  floatx16 fresh[4], grp[4], run[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    grp[j] = floatx16{};
    run[j] = floatx16{};
  }
  const int hk = lane >> 5, r32 = lane & 31;
  const int swz = swz_of(r32);
  // vmcnt(2 + NP): the newest step's transfers may be in flight, the one before
  // is complete (the barrier then publishes it)
  dma(0, rs0);
  dma(1, rs1);
  ring_barrier<2 + NP>();
  // step t (stage t % 3, a compile-time index): transfers for step t + 2 into
  // stage (t + 2) % 3, last read in step t - 1, before the barrier
  auto step = [&](auto pc, int t) {
    dma(t + 2, stage(IntC<decltype(pc)::value + 2>{}));
    RouterStage<NP>& S = stage(pc);
#pragma unroll
    for (int j = 0; j < 4; ++j) fresh[j] = floatx16{};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int slot = (2 * hk + s2) ^ swz;
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, S.a[(32 * wave + r32) * 4 + slot]);
#pragma unroll
      for (int pc2 = NP - 1; pc2 >= 0; --pc2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8_t b = __builtin_bit_cast(bf16x8_t, S.b[pc2][(32 * j + r32) * 4 + slot]);
          fresh[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, fresh[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) grp[j] += fresh[j];
    if ((t & 7) == 7 || t == n - 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        run[j] += grp[j];
        grp[j] = floatx16{};
      }
    }
    ring_barrier<2 + NP>();  // this wave's transfers for step t + 1 are complete
  };
  int t = 0;
  for (; t + 3 <= n; t += 3) static_for<0, 3>([&](auto pc) { step(pc, t + decltype(pc)::value); });
  const int rem = n - t;
  static_for<0, 2>([&](auto pc) {
    if (decltype(pc)::value < rem) step(pc, t + decltype(pc)::value);
  });
  __builtin_amdgcn_s_waitcnt(0xF70);  // no transfer into LDS outlives the loop
  // lane holds experts 32 j + lane % 32 of tokens 32 w + 8 (q / 4) + 4 (lane / 32) + q % 4
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 32 * j + r32;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int tt = t0 + 32 * wave + 8 * (q >> 2) + 4 * hk + (q & 3);
      if (tt < T) logits[(int64_t)tt * E + e] = run[j][q];
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
  if (H % 4 == 0) {  // 16-byte loads, contiguous across the wave
    for (int h = 4 * lane; h < H; h += 4 * kWave) {
      const float4 w = *reinterpret_cast<const float4*>(W + (int64_t)e * H + h);
      s = fmaf(w.x, w.x, s);
      s = fmaf(w.y, w.y, s);
      s = fmaf(w.z, w.z, s);
      s = fmaf(w.w, w.w, s);
    }
  } else {
    for (int h = lane; h < H; h += kWave) {
      const float w = W[(int64_t)e * H + h];
      s = fmaf(w, w, s);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  if (lane == 0) wnorm[e] = sqrtf(s);
}

// ---------------------------------------------------------------- decode: FP64 logits
// For a few tokens the router weights (E x H x 4 bytes) are streamed once and
// every logit is summed in FP64 from exact products (BF16 x FP32 fits in 53
// bits), so the selection needs no refinement pass.  A workgroup takes two
// experts, two waves each: lane L = 64 (wave & 1) + lane of an expert's pair
// owns elements 2048 j + 16 L .. + 16 (two FP64 partial sums per token, all
// loads issued before the arithmetic), then a butterfly over each wave and the
// sum of the two waves' totals.
//
// Fused variant (moe_layer_forward at T <= 4): the workgroups also write the
// A4 codes of x; the selection of the top k of every token, the softmax
// weights, the permutation and the slot table are then formed inside the
// gate/up kernel's workgroups (routing.hpp), each from the FP64 logits, so no
// separate one-workgroup kernel sits on the chain.  (A last-workgroup-done
// election inside the logits kernel needs a device-scope hand-off per
// workgroup, which measured slower than the kernel boundary.)
constexpr int kGemvMaxT = 8;
// kNorm (fused call with pre_norm, T <= 4, H <= 2048): x is first normed in the
// workgroup exactly as k_rms_norm norms it (each thread's 8 consecutive
// elements, FP64 sums of squares in the same order, the wave sums and the four
// wave totals in order, the product in FP64 rounded once to BF16), the normed
// rows are kept in LDS for the encoding and the FP64 sums, and workgroup 0
// writes them to q.xn.
template <bool kFused, bool kNorm>
__global__ __launch_bounds__(256) void k_route_decode(RouteDecodeParams q) {
  __shared__ double part[2][kGemvMaxT][2];
  __shared__ __align__(16) uint16_t xnl[kNorm ? 4 * 2048 : 8];
  __shared__ double nsum[kNorm ? 4 * 4 : 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int T = q.T, H = q.H, E = q.E;
  // 1. loads in dependency order: (kNorm) this thread's 8 elements of every row,
  // (fused) this lane's element of an A4 block of x (16 lanes per block, blocks
  // workgroup + grid * (tid / 16) + ..., so every workgroup encodes a few), then
  // the first router and x chunks; the encoding runs while the router rows are
  // in flight
  uint4 xr[kNorm ? 4 : 1];
  if (kNorm) {
#pragma unroll
    for (int t = 0; t < 4; ++t) xr[t] = (t < T && 8 * tid < H) ? *reinterpret_cast<const uint4*>(q.x + (int64_t)t * H + 8 * tid)
                                                               : make_uint4(0u, 0u, 0u, 0u);
  }
  const int64_t nb = kFused ? (int64_t)T * (H / 16) : 0;
  const int64_t b = (int64_t)(tid >> 4) * gridDim.x + blockIdx.x;
  const bool enc = b < nb;
  uint32_t xe = 0u;
  if (!kNorm && enc) xe = q.x[b * 16 + (tid & 15)];
  // logits of expert e: lane L of the expert's wave pair owns elements h0 .. h0 + 15
  const int e = 2 * blockIdx.x + (wave >> 1);
  const int L = kWave * (wave & 1) + lane;
  double acc[kGemvMaxT][2] = {};
  float4 wv[4];
  uint4 xv[kGemvMaxT][2];
  auto load_w = [&](int h0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = *reinterpret_cast<const float4*>(q.W + (int64_t)e * H + h0 + 4 * i);
  };
  auto load_x = [&](int h0) {
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t)
      if (t < T)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          xv[t][i] = kNorm ? *reinterpret_cast<const uint4*>(&xnl[t * H + h0 + 8 * i])
                           : *reinterpret_cast<const uint4*>(q.x + (int64_t)t * H + h0 + 8 * i);
  };
  auto fma_chunk = [&]() {
    const float wf[16] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w,
                          wv[2].x, wv[2].y, wv[2].z, wv[2].w, wv[3].x, wv[3].y, wv[3].z, wv[3].w};
#pragma unroll
    for (int t = 0; t < kGemvMaxT; ++t) {
      if (t < T) {
        const uint32_t xw[8] = {xv[t][0].x, xv[t][0].y, xv[t][0].z, xv[t][0].w,
                                xv[t][1].x, xv[t][1].y, xv[t][1].z, xv[t][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[t][0] = fma((double)__uint_as_float(xw[i] << 16), (double)wf[2 * i], acc[t][0]);
          acc[t][1] = fma((double)__uint_as_float(xw[i] & 0xFFFF0000u), (double)wf[2 * i + 1], acc[t][1]);
        }
      }
    }
  };
  const bool has = e < E && 16 * L < H;
  if (has) {
    load_w(16 * L);
    if (!kNorm) load_x(16 * L);
  }
  if (kNorm) {
    // the RMS norm of every row (k_rms_norm's arithmetic and order)
    double ss[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t w4[4] = {xr[t].x, xr[t].y, xr[t].z, xr[t].w};
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double lo = __uint_as_float(w4[i] << 16), hi = __uint_as_float(w4[i] & 0xFFFF0000u);
        a = fma(lo, lo, a);
        a = fma(hi, hi, a);
      }
      ss[t] = a;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < T) {
        const double sw = wave_sum_f64(ss[t]);
        if (lane == 0) nsum[t * 4 + wave] = sw;
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < T && 8 * tid < H) {
        double tot = 0.0;
#pragma unroll
        for (int w = 0; w < 4; ++w) tot += nsum[t * 4 + w];
        const double inv = 1.0 / sqrt(tot / (double)H + q.norm_eps);
        const uint32_t w4[4] = {xr[t].x, xr[t].y, xr[t].z, xr[t].w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = f64_to_bf16_rne((double)__uint_as_float(w4[i] << 16) * inv);
          const uint32_t hi = f64_to_bf16_rne((double)__uint_as_float(w4[i] & 0xFFFF0000u) * inv);
          o[i] = lo | (hi << 16);
        }
        const uint4 nv = make_uint4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<uint4*>(&xnl[t * H + 8 * tid]) = nv;
        if (blockIdx.x == 0) *reinterpret_cast<uint4*>(q.xn + (int64_t)t * H + 8 * tid) = nv;
      }
    }
    __syncthreads();
    if (enc) xe = xnl[b * 16 + (tid & 15)];
    if (has) load_x(16 * L);
  }
  // 2. A4 (or A8) codes of x (fused): each DPP row of 16 lanes encodes one block (block
  // maximum and code pairs by DPP; the even lanes store one byte of two codes),
  // blocks b, b + 16 * grid, ... (the first element loaded above).  A whole
  // row takes the same branch, so the row operations see all 16 lanes.
  if (kFused) {
    for (int64_t bb = b; bb < nb; bb += (int64_t)16 * gridDim.x) {
      if (bb != b) xe = kNorm ? xnl[bb * 16 + (tid & 15)] : q.x[bb * 16 + (tid & 15)];
      const float v = __uint_as_float(xe << 16);
      const float amax = row16_absmax(v);
      if (q.act8) {  // the W4A8 variant: UE4M3 scale from amax / (127 g), one INT8 code per element
        const uint32_t sc = scale_code(amax, 127.0f * q.g_in);
        q.xq[bb * 16 + (tid & 15)] = (uint8_t)(int8_code(v, sc ? ue4m3_value(sc) * q.g_in : __builtin_inff()) & 0xFF);
        if ((tid & 15) == 0) q.xs[bb] = (uint8_t)sc;
      } else {
        const uint32_t sc = scale_code(amax, 6.0f * q.g_in);
        const uint32_t c = elem_code_s(v, sc ? ue4m3_value(sc) * q.g_in : __builtin_inff());
        const uint32_t c2 = c | ((uint32_t)__builtin_amdgcn_mov_dpp((int)c, 0xB1, 0xF, 0xF, true) << 4);
        if ((tid & 1) == 0) q.xq[bb * 8 + ((tid & 15) >> 1)] = (uint8_t)c2;
        if ((tid & 15) == 0) q.xs[bb] = (uint8_t)sc;
      }
    }
  }
  // 3. the FP64 sums
  if (has) {
    fma_chunk();
    for (int h0 = 16 * L + 2048; h0 < H; h0 += 2048) {
      load_w(h0);
      load_x(h0);
      fma_chunk();
    }
  }
#pragma unroll
  for (int t = 0; t < kGemvMaxT; ++t) {
    if (t < T) {
      const double a = wave_sum_f64(acc[t][0] + acc[t][1]);
      if (lane == 0) part[wave >> 1][t][wave & 1] = a;
    }
  }
  __syncthreads();
  if ((wave & 1) == 0 && lane < T && e < E)
    q.logits[(int64_t)lane * E + e] = part[wave >> 1][lane][0] + part[wave >> 1][lane][1];
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
  // per wave: candidate values and ids, later the top-k scratch (same bytes)
  static_assert(sizeof(TopkScratch) <= kMaxCand * (sizeof(double) + sizeof(int)), "scratch fits");
  __shared__ __align__(16) unsigned char cbuf[4][kMaxCand * (sizeof(double) + sizeof(int))];
  double* const cvalw = reinterpret_cast<double*>(cbuf[threadIdx.x >> 6]);
  int* const cidw = reinterpret_cast<int*>(cbuf[threadIdx.x >> 6] + kMaxCand * sizeof(double));
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
      if (c) cidw[ncand + __popcll(m & ((1ull << lane) - 1ull))] = e;
      ncand += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const uint16_t* xr = p.x + t * H;
    for (int c = 0; c < ncand; c += 2) {
      const int e0 = cidw[c];
      const int e1 = c + 1 < ncand ? cidw[c + 1] : e0;
      double a0 = dot64_lane(xr, p.W + (int64_t)e0 * H, H, lane);
      double a1 = dot64_lane(xr, p.W + (int64_t)e1 * H, H, lane);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        a0 += __shfl_xor(a0, m);
        a1 += __shfl_xor(a1, m);
      }
      if (lane == 0) {
        cvalw[c] = a0;
        if (c + 1 < ncand) cvalw[c + 1] = a1;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // the candidates replace the per-lane values: lane owns candidates lane + 64 q
#pragma unroll
    for (int q = 0; q < kMaxPerLane; ++q) {
      const int c = lane + kWave * q;
      v[q] = c < ncand ? cvalw[c] : -INFINITY;
      vid[q] = c < ncand ? cidw[c] : 0x7FFFFFFF;
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
    wave_topk512(v8, id8, k, *reinterpret_cast<TopkScratch*>(cbuf[wave]), &my_v, &my_e);
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

// Pass B for E <= 512 (8 logits per lane), one wave per token.  The k-th largest
// lower end comes from the wave top-k on the lower ends; the candidates' FP64
// dot products run four at a time with every load of the four issued first;
// the final top k is the wave top-k on the candidates.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// FP64 dots of x_t with four router rows, summed over the wave (exact products:
// BF16 x FP32 fits in 53 bits).  Lane l takes elements 256 i + 4 l .. + 3, so
// every load instruction of the wave reads one contiguous run (1 KB of a router
// row, 512 B of x).
__device__ __forceinline__ void dot64x4(const uint16_t* __restrict__ xr, const float* __restrict__ W, int H,
                                        const int (&e)[4], int lane, double (&out)[4]) {
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  for (int h0 = lane * 4; h0 < H; h0 += kWave * 4 * 8) {
    uint2 xv[8];
    float4 w[4][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xv[i] = *reinterpret_cast<const uint2*>(xr + h0 + 256 * i);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) w[c][i] = *reinterpret_cast<const float4*>(W + (int64_t)e[c] * H + h0 + 256 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double x0 = (double)__uint_as_float(xv[i].x << 16), x1 = (double)__uint_as_float(xv[i].x & 0xFFFF0000u);
      const double x2 = (double)__uint_as_float(xv[i].y << 16), x3 = (double)__uint_as_float(xv[i].y & 0xFFFF0000u);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        a[c] = fma(x0, (double)w[c][i].x, a[c]);
        a[c] = fma(x1, (double)w[c][i].y, a[c]);
        a[c] = fma(x2, (double)w[c][i].z, a[c]);
        a[c] = fma(x3, (double)w[c][i].w, a[c]);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) out[c] = wave_sum_f64(a[c]);
}

__global__ __launch_bounds__(256) void k_route_select_refine(RouteB p) {
  __shared__ TopkScratch ts[4];  // per wave; between the two top-k passes it holds the candidates
  const int wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= p.T) return;
  const int lane = lane_id();
  const int E = p.E, H = p.H, k = p.k;
  const uint16_t* xr = p.x + t * H;
  // ||x_t||_2, inflated for its own rounding
  float sq = 0.0f;
  for (int h0 = lane * 8; h0 < H; h0 += kWave * 8) {
    const uint4 q = *reinterpret_cast<const uint4*>(xr + h0);
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(w4[j] << 16), hi = __uint_as_float(w4[j] & 0xFFFF0000u);
      sq = fmaf(lo, lo, sq);
      sq = fmaf(hi, hi, sq);
    }
  }
  const float xn = sqrtf((float)wave_sum_f64((double)sq)) * 1.001f;
  // lower ends of the intervals; k-th largest of them
  double v[8], lo[8];
  float rad[8];
  int id[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = lane + kWave * j;
    const bool ok = e < E;
    id[j] = ok ? e : 0x7FFFFFFF;
    v[j] = ok ? (double)p.l32[t * E + e] : -INFINITY;
    rad[j] = ok ? p.gamma * xn * (p.wnorm[e] * 1.001f) + 1e-30f : 0.0f;
    lo[j] = v[j] - (double)rad[j];
  }
  double my_lo = 0.0;
  int my_id = 0;
  wave_topk512(lo, id, k, ts[wave], &my_lo, &my_id);
  const double lk = readlane_f64(my_lo, k - 1);
  // candidates: upper end reaches lk; listed in lane order
  bool cand[8];
  int m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    cand[j] = id[j] != 0x7FFFFFFF && v[j] + (double)rad[j] >= lk;
    m += cand[j];
  }
  const int incl = wave_incl_scan_i32(m);
  const int nc = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - m;
  wave_sync_lds();  // the top-k scratch is read
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (cand[j]) ts[wave].key[pos++] = (uint64_t)id[j];
  wave_sync_lds();
  // FP64 logits of the candidates, four at a time
  for (int c0 = 0; c0 < nc; c0 += 4) {
    int e4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) e4[c] = (int)ts[wave].key[c0 + c < nc ? c0 + c : c0];
    double d4[4];
    dot64x4(xr, p.W, H, e4, lane, d4);
    if (lane < 4 && c0 + lane < nc)
      ts[wave].val[c0 + lane] = lane == 0 ? d4[0] : lane == 1 ? d4[1] : lane == 2 ? d4[2] : d4[3];
  }
  wave_sync_lds();
  // final top k among the candidates (lane owns candidates lane + 64 q)
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int c = lane + kWave * q;
    v[q] = c < nc ? ts[wave].val[c] : -INFINITY;
    id[q] = c < nc ? (int)ts[wave].key[c] : 0x7FFFFFFF;
  }
  wave_sync_lds();
  double my_v = 0.0;
  int my_e = 0;
  wave_topk512(v, id, k, ts[wave], &my_v, &my_e);
  const float wk = topk_softmax_weight(my_v, k);
  if (lane < k) {
    p.idx[t * k + lane] = my_e;
    p.w[t * k + lane] = wk;
  }
}

__global__ __launch_bounds__(256) void k_shared_gate(const uint16_t* __restrict__ x, const float* __restrict__ wg,
                                                     int64_t T, int H, float* __restrict__ gate) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float g = shared_gate_wave(x + t * H, wg, H);
  if (lane_id() == 0) gate[t] = g;
}

hipError_t launch_shared_gate(const uint16_t* x, const float* wg, int64_t T, int H, float* gate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  hipLaunchKernelGGL(k_shared_gate, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, x, wg, T, H, gate);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
bool route_decode_supported(int H, int E, int k, int64_t T) {
  return T >= 1 && T <= kRdMaxT && E <= kRdMaxE && k <= 32 && H % 32 == 0;
}

// the FP64 logits and the A4 codes of x; the selection runs in the gate/up
// kernel's workgroups (routing.hpp)
hipError_t launch_route_decode(const RouteDecodeParams& q, hipStream_t s, hipEvent_t ev_before, hipEvent_t ev_after) {
  if (q.pre_norm)
    return launch_timed(k_route_decode<true, true>, dim3((unsigned)((q.E + 1) / 2)), dim3(256), 0, s, ev_before,
                        ev_after, q);
  return launch_timed(k_route_decode<true, false>, dim3((unsigned)((q.E + 1) / 2)), dim3(256), 0, s, ev_before,
                      ev_after, q);
}

static float gamma_for_depth(int d) {
  const double u = 0x1p-24;
  return (float)(1.01 * d * u / (1.0 - d * u));
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

static bool router_mfma_shape(int H, int E) { return E % RM_E == 0 && H % RM_K == 0; }

static bool router_mfma_ok(int64_t T, int H, int E) { return T > kGemvMaxT && router_mfma_shape(H, E); }

bool route_mode_supported(int H, int E, int mode) { return mode == MOE_ROUTER_EXACT || router_mfma_shape(H, E); }

// logits (FP64 at decode, FP32 otherwise), ||W_e|| and, on the matrix-core
// path, the BF16 pieces of W (three; one in the BF16 mode)
size_t route_ws_bytes(int64_t T, int E, int H, int mode) {
  const bool mfma = mode != MOE_ROUTER_EXACT || router_mfma_ok(T, H, E);
  const size_t lg = (T <= kGemvMaxT && mode == MOE_ROUTER_EXACT) ? (size_t)(T * E) * sizeof(double)
                                                                   : (size_t)(T * E) * sizeof(float);
  const size_t pieces = mfma ? (mode == MOE_ROUTER_BF16 ? 1 : 3) * (size_t)E * H * sizeof(uint16_t) : 0;
  return align256(lg) + align256((size_t)E * sizeof(float)) + align256(pieces);
}

hipError_t launch_pack_router(const float* W, int E, int H, uint16_t* pieces, hipStream_t s) {
  const int64_t nw = (int64_t)E * H;
  hipLaunchKernelGGL(k_router_split, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, W, nw, pieces);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* x, const float* W, int64_t T, int H, int E, int k, const float* logits_in,
                        int32_t* idx, float* w, void* ws, int mode, const uint16_t* pieces, hipStream_t s) {
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
  } else if (T <= kGemvMaxT && mode == MOE_ROUTER_EXACT) {
    RouteDecodeParams q = {};
    q.x = x;
    q.W = W;
    q.T = (int)T;
    q.H = H;
    q.E = E;
    q.k = k;
    q.logits = static_cast<double*>(ws);
    hipLaunchKernelGGL((k_route_decode<false, false>), dim3((unsigned)((E + 1) / 2)), dim3(256), 0, s, q);
    p.l64 = q.logits;
    p.mode = kSelF64;
  } else {
    float* lg = static_cast<float*>(ws);
    char* after_lg = static_cast<char*>(ws) + align256((size_t)(T * E) * sizeof(float));
    float* wn = reinterpret_cast<float*>(after_lg);
    uint16_t* wp = reinterpret_cast<uint16_t*>(after_lg + align256((size_t)E * sizeof(float)));
    const int64_t nw = (int64_t)E * H;
    const dim3 grid((unsigned)(E / RM_E), (unsigned)((T + RM_T - 1) / RM_T));
    if (mode == MOE_ROUTER_BF16) {  // one BF16 pass on the rounded router, selection on its FP32 logits
      hipLaunchKernelGGL(k_router_round_bf16, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, W, nw, wp);
      hipLaunchKernelGGL(k_router_logits_mfma<1>, grid, dim3(512), 0, s, x, (const uint16_t*)wp, (int)T, H, E, lg);
      p.l32 = lg;
      p.mode = kSelF32;
    } else if (mode == MOE_ROUTER_SPLIT3_F32 || router_mfma_ok(T, H, E)) {
      if (!pieces) {
        hipLaunchKernelGGL(k_router_split, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s, W, nw, wp);
        pieces = wp;
      }
      if (mode == MOE_ROUTER_SPLIT3_F32) {
        hipLaunchKernelGGL(k_router_logits_mfma<3>, grid, dim3(512), 0, s, x, pieces, (int)T, H, E, lg);
        p.mode = kSelF32;
      } else {
        hipLaunchKernelGGL(k_router_logits_mfma<2>, grid, dim3(512), 0, s, x, pieces, (int)T, H, E, lg);
        // u = 2^-23 (twice the FP32 unit roundoff), the pieces' 1 + 2^-7, and
        // the dropped third piece's 2^-14; all inflated by 2^-6
        p.gamma = (2.0f * gamma_for_depth(2 * 2 * 16 + 8 + (H / RM_K + 7) / 8) * (1.0f + 0x1p-7f) + 0x1p-14f) *
                  (1.0f + 0x1p-6f);
        p.mode = kSelRefine;
      }
      p.l32 = lg;
    } else {
      const dim3 tgrid((unsigned)((E + RE - 1) / RE), (unsigned)((T + RT - 1) / RT));
      hipLaunchKernelGGL(k_router_logits_tiled, tgrid, dim3(256), 0, s, x, W, (int)T, H, E, lg);
      p.gamma = gamma_for_depth(RK + H / RK);
      p.l32 = lg;
      p.mode = kSelRefine;
    }
    if (p.mode == kSelRefine) {
      hipLaunchKernelGGL(k_router_norms, dim3((E + 3) / 4), dim3(256), 0, s, W, H, E, wn);
      p.wnorm = wn;
    }
  }
  if (p.mode == kSelRefine && E <= 512 && k <= 32 && H % 2048 == 0)
    hipLaunchKernelGGL(k_route_select_refine, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_route_select, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace moe

// Expert FFN for prefill chunks: grouped GEMM on the matrix cores.
//
// NVFP4 operands are decoded exactly to FP16 (Richland article, "What
// shipped": E2M1 codes times UE4M3 block scales): an E2M1 value times a UE4M3
// scale has at most 6 significant bits and lies in [2^-10, 2688], so it is an
// exact FP16 normal number.  The block scale therefore rides on the element and
// the product of two decoded operands is exact in FP32; the matrix core sums in
// FP32 (Richland article, "Why it matters": FP32 partials) and the per-expert
// FP32 scales multiply the result once.  The A4 activations are read already
// dequantized to FP16 (x from the A4 kernel, h from the gate/up epilogue): each
// is decoded once instead of once per column tile, and a 64-wide K step of an
// FP16 row is one 128-byte line, so 8 lanes load a row with full-line requests.
// The weights are read as codes and scales and decoded by the workgroup.
//
// Work decomposition: the rows of each expert segment (permuted-row order) are
// cut into 128-row tiles; a work item is (row tile, column tile).  A small
// kernel turns expert_off into the prefix of tile counts and a table of row
// tiles; each workgroup reads its row tile from the table.  Workgroups are
// dealt round robin to the 8 XCDs and each XCD takes one contiguous run of
// work items, so the column tiles of a row tile and the row tiles of an expert
// share one L2.
//
// G1 (gate/up): 128 rows x (128 gate + 128 up) columns, K = H in steps of 64;
// wave w computes all 128 rows and h columns 32 w .. 32 w + 31 for both gate
// and up, so SwiGLU pairs meet in the same lane; the epilogue forms h, encodes
// its 16-column blocks and stores the dequantized FP16 h.  G2 (down): 128 rows
// x 256 output columns, K = I; wave w computes columns 64 w .. 64 w + 63.
#include "common.hpp"
#include "lds_ring.hpp"

namespace moe {

namespace {

constexpr int kBM = 128, kBN = 256, kBK = 64;  // tile rows, tile B rows (columns), K step

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));


// In the workspace: tile_start ([E + 2] int32), the chained kernels' work
// counters (kCounters int32), then the tile table, 16-byte aligned.
constexpr int kCounters = 16;
__host__ __device__ inline int tile_tab_offset(int E) { return (E + 2 + kCounters + 3) / 4 * 4; }

}  // namespace

// tile_start[s] = number of 128-row tiles of segments < s; segments 0..E-1 are the
// routed experts, segment E the shared expert (T rows), tile_start[E+1] = total.
// tile_tab[mt] = (segment, first row of the tile in the segment, the segment's
// first row in the permuted order, the segment's rows) for every row tile mt <
// total, so that a GEMM workgroup finds its tile in one load instead of a
// binary search of dependent loads.
__global__ __launch_bounds__(1024) void k_tile_map(const int32_t* __restrict__ off, int E, int T, int has_shared,
                                                   int32_t* __restrict__ tile_start, int4* __restrict__ tile_tab) {
  __shared__ int part[1024];
  __shared__ int row0[1024], rows[1024];
  const int tid = threadIdx.x;
  const int r0 = tid < E ? off[tid] : 0;
  const int nr = tid < E ? off[tid + 1] - r0 : (tid == E && has_shared ? T : 0);
  part[tid] = (nr + kBM - 1) / kBM;
  row0[tid] = r0;
  rows[tid] = nr;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int add = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  if (tid <= E + 1) tile_start[tid] = tid > 0 ? part[tid - 1] : 0;
  if (tid < kCounters) tile_start[E + 2 + tid] = 0;  // the work counters start at zero
  const int total = part[E];
  for (int mt = tid; mt < total; mt += 1024) {
    int lo = 0, hi = E;  // first segment whose inclusive tile count exceeds mt
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (part[mid] > mt) hi = mid; else lo = mid + 1;
    }
    const int first = lo > 0 ? part[lo - 1] : 0;
    tile_tab[mt] = make_int4(lo, (mt - first) * kBM, row0[lo], rows[lo]);
  }
}

// LDS ring of kStages K steps (the down GEMM's; the gate/up ring holds only A,
// see StageA).  Each stage holds the tile's A rows (128 rows x 64
// FP16 = 128 B, as 8 chunks of 16 B; chunk c of row r sits in slot
// c ^ (r % 8) ^ (r / 8 % 2), so that the MFMA reads of 16 consecutive rows hit 16
// different 16-byte bank groups), the step's 32 B of codes of each of the 256 B
// rows (two 16-byte halves; half h of row r sits in slot h ^ (r / 4 % 2) ^
// (r / 8 % 2), for the same reason) and the step's four UE4M3 scales of each B
// row.  All of it arrives by buffer loads that write LDS directly (64 lanes x
// 16 B per transfer: 8 A rows or 32 B rows; 64 lanes x 4 B: 64 scale words), so
// the ring costs no registers and is filled 2 steps ahead.
constexpr int kStages = 3;
struct Stage {
  uint4 a[kBM * 8];
  uint4 b[kBN * 2];
  uint32_t s[kBN];
};
// The three stages are separate LDS variables, so the compiler can tell that
// the transfers into one stage and the reads of another do not overlap.  With
// one array it cannot, and it made every read wait for all transfers in flight
// (the two steps issued ahead included), which left the matrix cores waiting
// out a memory round trip every step.  For the same reason the ring's barrier
// is ring_barrier (lds_ring.hpp), not __syncthreads.
struct Ring {
  Stage& st0;
  Stage& st1;
  Stage& st2;
  template <int kS>
  __device__ __forceinline__ Stage& at() {
    if constexpr (kS % kStages == 0) return st0;
    else if constexpr (kS % kStages == 1) return st1;
    else return st2;
  }
};

// One operand set: buffer resources and per-lane byte offsets (a K step at
// element k0 adds 2 k0 for A, bmul k0 / 2 for B codes and bmul k0 / 16 for B
// scales as wave-uniform offsets).  adma[c] / bdma[c]: the row (and swizzled chunk) this lane moves in
// the wave's c-th A / B transfer; sdma: the B row whose scales this lane moves.
struct Operands {
  __amdgpu_buffer_rsrc_t a, bq, bs;
  __amdgpu_buffer_rsrc_t a0, bq0, bs0;  // the same with no bytes: every access out of range
  uint32_t adma[4], bdma[2], sdma;
  uint32_t bmul;  // B bytes per K step: 32 bmul of codes, 4 bmul of scales
};

// B rows (one expert's N x K NVFP4 matrix) are read either from the row-major
// bank (a row's K step: 32 code bytes at row K/2 + 32 s, bmul = 1) or from its
// K-step-major copy (32 bytes at (s N + row) 32, bmul = N), where the 32 rows
// of one wave transfer are one contiguous 1 KB run instead of 32 separate
// lines; the expert's block has the same size and offset in both.

// A (FP16 activation rows) x B (weight rows, NVFP4 codes decoded to FP16 in
// registers) over K = [k_begin, k_begin + K).  Every wave owns all 128 rows of
// the tile and 64 B rows as 4 x 2 MFMA tiles, so each B element a wave decodes
// feeds four MFMAs (the decode is the main loop's largest VALU cost).  K is
// taken in a lane-contiguous order: in MFMA s (0..3) of a step, lanes 0..31
// supply elements 8s..8s+7 and lanes 32..63 elements 32+8s..32+8s+7, for A and
// B alike, so a lane's B codes for the step are one 16-byte half-row (two whole
// 16-element blocks).  Each wave decodes the
// B codes it needs after reading them from the ring.  One barrier per step.
// bj(j): the ring's B row index of the wave's column block j (lane % 32 added).
// live_rows: rows of the tile inside the expert's segment; a tile with none
// skips the step.  kRB: 32-row blocks computed (the caller instantiates one
// variant per block count, so a segment's last tile runs only the blocks that
// hold its rows without a branch per MFMA; blocks past kRB keep their zeros).
// kTransposed: the MFMAs take B as their first operand, so acc[i][j] holds the
// transposed 32 x 32 block (lane l: tile row 32 i + l % 32, B rows
// 8 (q / 4) + 4 (l / 32) + q % 4 of block j in its entries q = 0..15).
// 32-row blocks holding a tile's live rows (1..4; 4 when the segment continues
// past the tile)
__device__ __forceinline__ int tile_blocks(int live_rows) {
  return live_rows >= kBM ? 4 : live_rows <= 32 ? 1 : (live_rows + 31) / 32;
}

// The wave's transfers of one K step (element k0) into a ring stage: 4 A, 2 B
// and 1 scale transfers.  real = false: the same transfers through resources
// of no bytes, which read nothing and write zeros into the stage (used where
// no later step reads it).  Issuing them keeps every step's transfers
// unconditional: around a conditional transfer the compiler cannot tell which
// stage is in flight and makes the next reads wait for all of them.
__device__ __forceinline__ void dma_step(const Operands& O, bool real, uint32_t k0, Stage& S) {
  const int wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t ra = real ? O.a : O.a0, rq = real ? O.bq : O.bq0, rs = real ? O.bs : O.bs0;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)&S.a[(32 * wave + 8 * c) * 8], 16, O.adma[c], k0 * 2, 0,
                                             0);
#pragma unroll
  for (int c = 0; c < 2; ++c)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_ptr_t)&S.b[(64 * wave + 32 * c) * 2], 16, O.bdma[c],
                                             k0 / 2 * O.bmul, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)&S.s[64 * wave], 4, O.sdma, k0 / 16 * O.bmul, 0, 0);
}

// The MFMAs of one K step from a ring stage (layout: see tile_mma).
template <bool kTransposed, int kRB, typename BRow>
__device__ __forceinline__ void mma_step(Stage& S, BRow bj, floatx16 (&acc)[4][2]) {
  const int lane = lane_id();
  const int hk = lane >> 5;
  uint4 bq[2];
  half2_t sv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = bj(j) + (lane & 31);
    bq[j] = S.b[r * 2 + (hk ^ (((r >> 2) ^ (r >> 3)) & 1))];
    sv[j] = ue4m3x2_to_half2(S.s[r] >> (16 * hk));
  }
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    half8_t a[4];
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const int row = 32 * i + (lane & 31);
      a[i] = __builtin_bit_cast(half8_t, S.a[row * 8 + ((4 * hk + s4) ^ (lane & 7) ^ ((lane >> 3) & 1))]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const half2_t S2 = half2_t{sv[j][s4 >> 1], sv[j][s4 >> 1]};
      const uint32_t w = s4 == 0 ? bq[j].x : s4 == 1 ? bq[j].y : s4 == 2 ? bq[j].z : bq[j].w;
      const half2_t c0 = fp4x2<0>(w) * S2, c1 = fp4x2<1>(w) * S2, c2 = fp4x2<2>(w) * S2, c3 = fp4x2<3>(w) * S2;
      const half8_t b = half8_t{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
#pragma unroll
      for (int i = 0; i < kRB; ++i) {  // rows past live_rows in a block are computed, never stored
        if (kTransposed)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a[i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b, acc[i][j], 0, 0, 0);
      }
    }
  }
}

template <bool kTransposed, int kRB, typename BRow>
__device__ __forceinline__ void tile_mma(const Operands& O, int k_begin, int K, int live_rows, Ring& ring, BRow bj,
                                         floatx16 (&acc)[4][2]) {
  const int n = K / kBK;
  const int nlive = __builtin_amdgcn_readfirstlane(live_rows > 0 ? 1 : 0);
  auto kof = [&](int t) { return (uint32_t)(k_begin + (t < n ? t : n - 1) * kBK); };  // n = 1: the prologue repeats step 0
  // step t into ring stage `stage` (real = false for the last two steps' transfers)
  auto dma = [&](int t, Stage& S, bool real) { dma_step(O, real, kof(t), S); };
  auto compute = [&](Stage& S) {
    if (nlive == 0) return;
    mma_step<kTransposed, kRB>(S, bj, acc);
  };

  // vmcnt(7): the wave's 7 newest transfers (the step issued last) may still be
  // in flight; the one before is complete, and the barrier then publishes it
  // to the other waves
  dma(0, ring.at<0>(), true);
  dma(1, ring.at<1>(), true);
  ring_barrier<7>();
  // step t: transfers for step t + 2 into stage (t + 2) % 3 (last read in step
  // t - 1, before the previous barrier), then the MFMAs of step t.  The last
  // two steps' transfers read nothing.
  auto phase = [&](auto pc, int t) {
    constexpr int P = decltype(pc)::value;  // t % 3
    dma(t + 2, ring.at<P + 2>(), t + 2 < n);
    __builtin_amdgcn_sched_barrier(0);
    compute(ring.at<P>());
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier<7>();
  };
  int t = 0;
  for (; t + 3 <= n; t += 3) static_for<0, 3>([&](auto pc) { phase(pc, t + decltype(pc)::value); });
  const int rem = n - t;
  static_for<0, 2>([&](auto pc) {
    if (decltype(pc)::value < rem) phase(pc, t + decltype(pc)::value);
  });
  __builtin_amdgcn_s_waitcnt(0);  // no transfer into LDS outlives the loop
}

// field-wise choice between two operand sets (values, so that both stay in
// registers)
__device__ __forceinline__ Operands pick(bool c, const Operands& A, const Operands& B) {
  Operands R;
  R.a = c ? A.a : B.a;
  R.bq = c ? A.bq : B.bq;
  R.bs = c ? A.bs : B.bs;
  R.a0 = A.a0;
  R.bq0 = A.bq0;
  R.bs0 = A.bs0;
#pragma unroll
  for (int i = 0; i < 4; ++i) R.adma[i] = c ? A.adma[i] : B.adma[i];
#pragma unroll
  for (int i = 0; i < 2; ++i) R.bdma[i] = c ? A.bdma[i] : B.bdma[i];
  R.sdma = c ? A.sdma : B.sdma;
  R.bmul = c ? A.bmul : B.bmul;
  return R;
}

// The K loop of one tile in a workgroup that runs several tiles with one ring:
// the tile's first two steps are already in flight (issued by the previous
// tile's last two steps, or by the workgroup's prologue), and its last two
// steps issue the next tile's first two.  make_on() returns the next tile's
// operands (resources of no bytes when there is none); it runs after the
// first step's barrier, so loads issued before this loop for it have
// completed by then.  kPh: the ring stage of step 0; kNm3 = n % 3, n >= 3
// steps from k_begin (the same K range for every tile).  No wait at the end:
// the next tile's transfers stay in flight through this tile's epilogue.
template <bool kTransposed, int kRB, int kPh, int kNm3, typename BRow, typename MakeOn>
__device__ __forceinline__ void tile_mma_chain(const Operands& O, MakeOn make_on, int k_begin, int n, Ring& ring,
                                               BRow bj, floatx16 (&acc)[4][2]) {
  // (an empty statement that differs per kRB: without it the compiler hoists
  // the identical first transfers of the kRB variants above the branch that
  // picks one, and then makes every variant but one wait for all transfers)
  asm volatile("; kRB %0" ::"n"(kRB));
  dma_step(O, true, (uint32_t)(k_begin + 2 * kBK), ring.at<kPh + 2>());
  __builtin_amdgcn_sched_barrier(0);
  mma_step<kTransposed, kRB>(ring.at<kPh>(), bj, acc);
  __builtin_amdgcn_sched_barrier(0);
  ring_barrier<7>();
  const Operands On = make_on();
  // steps t = 1 + 3 m + pc: stage (kPh + 1 + pc) % 3
  auto phase = [&](auto pc, int t) {
    constexpr int P = kPh + 1 + decltype(pc)::value;
    const bool own = t + 2 < n;
    const uint32_t k0 = (uint32_t)(k_begin + (own ? t + 2 : t + 2 - n) * kBK);
    dma_step(pick(own, O, On), true, k0, ring.at<P + 2>());
    __builtin_amdgcn_sched_barrier(0);
    mma_step<kTransposed, kRB>(ring.at<P>(), bj, acc);
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier<7>();
  };
  int t = 1;
  for (; t + 3 <= n; t += 3) static_for<0, 3>([&](auto pc) { phase(pc, t + decltype(pc)::value); });
  static_for<0, (kNm3 + 2) % 3>([&](auto pc) { phase(pc, t + decltype(pc)::value); });
}


// The gate/up GEMM's ring holds only A: each lane's B codes (16 B per column
// block) and scale words go straight from memory into registers, three
// register sets for the three steps in flight.  A wave's B rows are its own
// (no other wave reads them), so staging them in LDS only added LDS traffic
// (a fifth of the ring's writes and reads); the ring then takes 48 KB.
struct StageA {
  uint4 a[kBM * 8];
};
struct RingA {
  StageA& st0;
  StageA& st1;
  StageA& st2;
  template <int kS>
  __device__ __forceinline__ StageA& at() {
    if constexpr (kS % kStages == 0) return st0;
    else if constexpr (kS % kStages == 1) return st1;
    else return st2;
  }
};
struct OperandsR {
  __amdgpu_buffer_rsrc_t a, bq, bs;
  __amdgpu_buffer_rsrc_t a0, bq0, bs0;
  uint32_t adma[4];
  uint32_t boff[2], soff[2];  // the lane's B code and scale word offsets, column blocks j = 0, 1
  uint32_t bmul;
};

// mma_step with B from registers: bq[j] the lane's 16 code bytes of column
// block j, sc[j] the step's four scale codes of its B row
template <bool kTransposed, int kRB>
__device__ __forceinline__ void mma_step_r(StageA& S, const uint4 (&bq)[2], const uint32_t (&sc)[2],
                                           floatx16 (&acc)[4][2]) {
  const int lane = lane_id();
  const int hk = lane >> 5;
  half2_t sv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) sv[j] = ue4m3x2_to_half2(sc[j] >> (16 * hk));
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    half8_t a[4];
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const int row = 32 * i + (lane & 31);
      a[i] = __builtin_bit_cast(half8_t, S.a[row * 8 + ((4 * hk + s4) ^ (lane & 7) ^ ((lane >> 3) & 1))]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const half2_t S2 = half2_t{sv[j][s4 >> 1], sv[j][s4 >> 1]};
      const uint32_t w = s4 == 0 ? bq[j].x : s4 == 1 ? bq[j].y : s4 == 2 ? bq[j].z : bq[j].w;
      const half2_t c0 = fp4x2<0>(w) * S2, c1 = fp4x2<1>(w) * S2, c2 = fp4x2<2>(w) * S2, c3 = fp4x2<3>(w) * S2;
      const half8_t b = half8_t{c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
#pragma unroll
      for (int i = 0; i < kRB; ++i) {
        if (kTransposed)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a[i], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b, acc[i][j], 0, 0, 0);
      }
    }
  }
}

// tile_mma with the A-only ring: per step and wave 4 A transfers into LDS and
// 4 B loads into registers (the last two steps' through resources of no
// bytes, as in tile_mma), one barrier per step after the wave's 8 newest
// loads at most are left in flight.
template <bool kTransposed, int kRB>
__device__ __forceinline__ void tile_mma_r(const OperandsR& O, int k_begin, int K, RingA& ring,
                                           floatx16 (&acc)[4][2]) {
  const int n = K / kBK;
  const int wave = threadIdx.x >> 6;
  auto kof = [&](int t) { return (uint32_t)(k_begin + (t < n ? t : n - 1) * kBK); };
  uint4 bq[3][2];
  uint32_t sc[3][2];
  auto dma = [&](int t, StageA& S, bool real) {
    const uint32_t k0 = kof(t);
    const __amdgpu_buffer_rsrc_t ra = real ? O.a : O.a0;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)&S.a[(32 * wave + 8 * c) * 8], 16, O.adma[c], k0 * 2, 0,
                                               0);
  };
  auto loadb = [&](int t, uint4 (&q)[2], uint32_t (&s)[2], bool real) {
    const uint32_t k0 = kof(t);
    const __amdgpu_buffer_rsrc_t rq = real ? O.bq : O.bq0, rs = real ? O.bs : O.bs0;
#pragma unroll
    for (int j = 0; j < 2; ++j) q[j] = buffer_load16(rq, O.boff[j], k0 / 2 * O.bmul);
#pragma unroll
    for (int j = 0; j < 2; ++j) s[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, O.soff[j], k0 / 16 * O.bmul, 0);
  };
  dma(0, ring.at<0>(), true);
  loadb(0, bq[0], sc[0], true);
  dma(1, ring.at<1>(), true);
  loadb(1, bq[1], sc[1], true);
  ring_barrier<8>();
  auto phase = [&](auto pc, int t) {
    constexpr int P = decltype(pc)::value;
    dma(t + 2, ring.at<P + 2>(), t + 2 < n);
    loadb(t + 2, bq[(P + 2) % 3], sc[(P + 2) % 3], t + 2 < n);
    __builtin_amdgcn_sched_barrier(0);
    mma_step_r<kTransposed, kRB>(ring.at<P>(), bq[P], sc[P], acc);
    __builtin_amdgcn_sched_barrier(0);
    ring_barrier<8>();
  };
  int t = 0;
  for (; t + 3 <= n; t += 3) static_for<0, 3>([&](auto pc) { phase(pc, t + decltype(pc)::value); });
  const int rem = n - t;
  static_for<0, 2>([&](auto pc) {
    if (decltype(pc)::value < rem) phase(pc, t + decltype(pc)::value);
  });
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------- G1
// Tile: 128 rows x (128 gate + 128 up) columns; wave w holds h columns
// nt*128 + 32 w .. + 31 of all 128 rows as gate block j = 0 and up block j = 1,
// so SwiGLU pairs meet in the same lane.  Dequantized A4(h) of every row goes
// to hh (permuted rows, then shared rows); the down GEMM reads it back as its A
// operand.  Codes and scales are written only to the debug dumps.
__global__ __launch_bounds__(256, 2) void k_gateup_mfma(FfnParams p, const int32_t* __restrict__ tile_start,
                                                        const int4* __restrict__ tile_tab) {
  __shared__ __align__(16) StageA st0, st1, st2;
  RingA ring{st0, st1, st2};
  const int H = p.H, I = p.I, T = p.T, E = p.E;
  const int n_nt = I / 128;
  const int nseg = E + 1;
  const int n_tiles = tile_start[nseg] * n_nt;
  if ((int)blockIdx.x >= n_tiles) return;
  const int lt = xcd_tile((int)blockIdx.x, n_tiles);
  const int mt = lt / n_nt, nt = lt % n_nt;
  const int4 te = tile_tab[mt];
  const int seg = __builtin_amdgcn_readfirstlane(te.x), m0 = __builtin_amdgcn_readfirstlane(te.y);
  const int seg_row0 = __builtin_amdgcn_readfirstlane(te.z), seg_rows = __builtin_amdgcn_readfirstlane(te.w);
  const bool shared = seg == E;
  const moe_nvfp4_bank& bank = shared ? (p.sh13k.codes ? p.sh13k : p.sh13) : (p.w13k.codes ? p.w13k : p.w13);
  const bool km = shared ? p.sh13k.codes != nullptr : p.w13k.codes != nullptr;
  const int64_t erow = shared ? 0 : (int64_t)seg * 2 * I;  // the expert's first row in the bank
  const uint8_t* codes = bank.codes + erow * (H / 2);
  const uint8_t* scales = bank.scales + erow * (H / 16);
  const uint32_t qrow = km ? 32u : (uint32_t)(H / 2), srow = km ? 4u : (uint32_t)(H / 16);
  const float G = (shared ? p.sh13.gscale[0] : p.w13.gscale[seg]) * p.g_in;
  const int tid = threadIdx.x, wave = tid >> 6, lane = lane_id();
  const int wn = 32 * wave;
  // ring B row r: gate column nt*128 + r (r < 128), up column I + nt*128 + r - 128
  auto wrow = [&](int r) { return (uint32_t)(r < 128 ? nt * 128 + r : I + nt * 128 + (r - 128)); };
  auto bj = [&](int j) { return j == 0 ? wn : 128 + wn; };
  OperandsR O;
  O.a = buffer_rsrc(p.xh, (uint32_t)T * H * 2u);
  O.a0 = buffer_rsrc(p.xh, 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    // A row: the token of tile row 32 w + 8 c + lane / 8 (rows past the segment read token 0; dropped)
    const int m = 32 * wave + 8 * c + (lane >> 3);
    const int tok = m0 + m < seg_rows ? (shared ? m0 + m : p.row2pair[seg_row0 + m0 + m] / p.k) : 0;
    O.adma[c] = (uint32_t)tok * H * 2u + (uint32_t)((lane & 7) ^ (lane >> 3) ^ (c & 1)) * 16u;
  }
  O.bq = buffer_rsrc(codes, 2u * I * (H / 2));
  O.bs = buffer_rsrc(scales, 2u * I * (H / 16));
  O.bq0 = buffer_rsrc(codes, 0u);
  O.bs0 = buffer_rsrc(scales, 0u);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = bj(j) + (lane & 31);
    O.boff[j] = wrow(r) * qrow + (uint32_t)(lane >> 5) * 16u;
    O.soff[j] = wrow(r) * srow;
  }
  O.bmul = km ? 2u * I : 1u;
  floatx16 acc[4][2] = {};
  switch (tile_blocks(seg_rows - m0)) {
    case 1: tile_mma_r<true, 1>(O, 0, H, ring, acc); break;
    case 2: tile_mma_r<true, 2>(O, 0, H, ring, acc); break;
    case 3: tile_mma_r<true, 3>(O, 0, H, ring, acc); break;
    default: tile_mma_r<true, 4>(O, 0, H, ring, acc); break;
  }
  // Epilogue.  acc[i][j] is transposed: lane l holds row m = 32 i + l % 32
  // and h columns c(q) = nt*128 + wn + 8 (q / 4) + 4 (l / 32) + q % 4, so
  // the first 16-column A4 block of the 32 is entries q < 8 of lanes l and l ^ 32,
  // the second entries q >= 8.  Each lane takes the maxima of its halves, the
  // lane pair completes them, lane l < 32 computes the first block's scale code
  // and lane l + 32 the second's, and the pair exchanges the codes.  Codes of
  // adjacent columns (q, q + 1) are paired inside the lane, converted to FP16 and
  // scaled together; four consecutive columns go out as one 8-byte store.
  // Stores go through a buffer resource sized to the segment's rows in this
  // tile: rows past the segment are dropped by its range check.
  const float g6 = 6.0f * p.g_mid;
  const int64_t orow0 = (shared ? (int64_t)T * p.k : (int64_t)seg_row0) + m0;
  const int nrows = seg_rows - m0 < kBM ? seg_rows - m0 : kBM;
  const __amdgpu_buffer_rsrc_t hh_r = buffer_rsrc(p.hh + orow0 * I, (uint32_t)nrows * I * 2u);
  const int hi = lane >> 5;
  const float c_exp = -G * 1.4426950408889634f, inv_g2 = 1.0f / (G * G);
  // (the debug dumps and the A8 encoding of the W4A8 variant take separate
  // copies of the epilogue)
  auto epilogue = [&](auto dumps_c, auto a8_c) {
    constexpr bool kDumps = decltype(dumps_c)::value != 0;
    constexpr bool kA8 = decltype(a8_c)::value != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 32 * i + (lane & 31);  // tile row
      {
        const int col0 = nt * 128 + wn + 4 * hi;  // column of q = 0
        float hv[16];
        uint32_t p0 = 0u, p1 = 0u;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          hv[q] = swiglu_scaled(acc[i][0][q], acc[i][1][q], c_exp, inv_g2);
          const uint32_t a = __float_as_uint(hv[q]) & 0x7FFFFFFFu;
          if (q < 8) p0 = max(p0, a);
          else p1 = max(p1, a);
        }
        uint32_t x0, y0, x1, y1;
        lane_pair(p0, &x0, &y0);
        lane_pair(p1, &x1, &y1);
        const float amax = __uint_as_float(hi ? max(x1, y1) : max(x0, y0));
        const uint32_t mine = scale_code(amax, kA8 ? 127.0f * p.g_mid : g6) | ((uint32_t)hi << 8);
        uint32_t ca, cb;
        lane_pair(mine, &ca, &cb);
        const uint32_t sc0 = ((ca >> 8) == 0u ? ca : cb) & 0xFFu, sc1 = ((ca >> 8) == 0u ? cb : ca) & 0xFFu;
        const float u0 = ue4m3_value(sc0), u1 = ue4m3_value(sc1);  // 0 for code 0
        const E2M1Thresholds T0 = e2m1_thresholds(sc0 ? u0 * p.g_mid : __builtin_inff());
        const E2M1Thresholds T1 = e2m1_thresholds(sc1 ? u1 * p.g_mid : __builtin_inff());
        const half_t uh0 = (half_t)u0, uh1 = (half_t)u1;  // exact: UE4M3 values
        if (kDumps && p.hs_dbg && m < nrows)
          p.hs_dbg[(orow0 + m) * (I / 16) + (nt * 128 + wn) / 16 + hi] = (uint8_t)(hi ? sc1 : sc0);
        if (kA8) {  // INT8 codes; FP16 values q * scale (exact)
          const float s0 = sc0 ? u0 * p.g_mid : __builtin_inff(), s1 = sc1 ? u1 * p.g_mid : __builtin_inff();
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const float sg = g < 2 ? s0 : s1, ug = g < 2 ? u0 : u1;
            int qv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) qv[e] = int8_code(hv[4 * g + e], sg);
            const half2_t h01 = half2_t{(half_t)((float)qv[0] * ug), (half_t)((float)qv[1] * ug)};
            const half2_t h23 = half2_t{(half_t)((float)qv[2] * ug), (half_t)((float)qv[3] * ug)};
            const uint32_t voff = (uint32_t)(m * I + col0 + 8 * g) * 2u;
            buffer_store8(u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)}, hh_r, voff);
            if (kDumps && m < nrows) {
              const int64_t orow = orow0 + m;
              const int c = col0 + 8 * g;
              if (p.hq_dbg)
                *reinterpret_cast<uint32_t*>(p.hq_dbg + orow * I + c) =
                    (uint32_t)(qv[0] & 0xFF) | (uint32_t)(qv[1] & 0xFF) << 8 | (uint32_t)(qv[2] & 0xFF) << 16 |
                    (uint32_t)(qv[3] & 0xFF) << 24;
              if (p.h_dbg)
#pragma unroll
                for (int e = 0; e < 4; ++e) p.h_dbg[orow * I + c + e] = hv[4 * g + e];
            }
          }
          continue;
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {  // columns col0 + 8 g .. + 3: entries 4 g .. 4 g + 3
          const E2M1Thresholds& Tg = g < 2 ? T0 : T1;
          const half_t uh = g < 2 ? uh0 : uh1;
          uint32_t by[2];
          half2_t hd[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int q = 4 * g + 2 * e;
            by[e] = elem_code_t(hv[q], Tg) | elem_code_t(hv[q + 1], Tg) << 4;
            hd[e] = fp4x2<0>(by[e]) * half2_t{uh, uh};  // exact: <= 6 significant bits
          }
          const uint32_t voff = (uint32_t)(m * I + col0 + 8 * g) * 2u;
          buffer_store8(u32x2{__builtin_bit_cast(uint32_t, hd[0]), __builtin_bit_cast(uint32_t, hd[1])}, hh_r, voff);
          if (kDumps && m < nrows) {
            const int64_t orow = orow0 + m;
            const int c = col0 + 8 * g;
            if (p.hq_dbg)
              *reinterpret_cast<uint16_t*>(p.hq_dbg + orow * (I / 2) + c / 2) = (uint16_t)(by[0] | by[1] << 8);
            if (p.h_dbg)
#pragma unroll
              for (int e = 0; e < 4; ++e) p.h_dbg[orow * I + c + e] = hv[4 * g + e];
          }
        }
      }
    }
  };
  const bool dumps = p.h_dbg || p.hq_dbg || p.hs_dbg;
  if (p.act8) {
    if (dumps)
      epilogue(IntC<1>{}, IntC<1>{});
    else
      epilogue(IntC<0>{}, IntC<1>{});
  } else if (dumps) {
    epilogue(IntC<1>{}, IntC<0>{});
  } else {
    epilogue(IntC<0>{}, IntC<0>{});
  }
}

// ---------------------------------------------------------------- G2
// Tile: 128 rows x 256 output columns; wave w holds columns nt*256 + 64 w ..
// + 63 of all 128 rows as blocks j = 0, 1.
struct DownTile {
  Operands O;
  float* y;    // the tile's first output row (y_rows in permuted order, or y_shared)
  int nrows;   // rows of the segment in the tile (1..128)
  int m0;      // the tile's first row in its segment
  int nt;      // column tile
  bool shared;
};

__device__ __forceinline__ int down_bj(int j) { return 64 * (int)(threadIdx.x >> 6) + 32 * j; }

// Operands and output rows of the work item (row tile te = its tile table
// entry, column tile nt)
__device__ __forceinline__ DownTile down_tile(const FfnParams& p, int4 te, int nt) {
  const int H = p.H, I = p.I, T = p.T, E = p.E;
  const int seg = __builtin_amdgcn_readfirstlane(te.x), m0 = __builtin_amdgcn_readfirstlane(te.y);
  const int seg_row0 = __builtin_amdgcn_readfirstlane(te.z), seg_rows = __builtin_amdgcn_readfirstlane(te.w);
  const bool shared = seg == E;
  const moe_nvfp4_bank& bank = shared ? (p.sh2k.codes ? p.sh2k : p.sh2) : (p.w2k.codes ? p.w2k : p.w2);
  const bool km = shared ? p.sh2k.codes != nullptr : p.w2k.codes != nullptr;
  const int64_t erow = shared ? 0 : (int64_t)seg * H;  // the expert's first row in the bank
  const uint8_t* codes = bank.codes + erow * (I / 2);
  const uint8_t* scales = bank.scales + erow * (I / 16);
  const uint32_t qrow = km ? 32u : (uint32_t)(I / 2), srow = km ? 4u : (uint32_t)(I / 16);
  const int wave = threadIdx.x >> 6, lane = lane_id();
  DownTile d;
  // A rows: the tile's rows of hh; rows past the segment read zeros (range check)
  const int64_t row0 = (shared ? (int64_t)T * p.k : (int64_t)seg_row0) + m0;
  d.nrows = seg_rows - m0 < kBM ? seg_rows - m0 : kBM;
  d.O.a = buffer_rsrc(p.hh + row0 * I, (uint32_t)d.nrows * I * 2u);
  d.O.a0 = buffer_rsrc(p.hh + row0 * I, 0u);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    d.O.adma[c] = (uint32_t)(32 * wave + 8 * c + (lane >> 3)) * I * 2u +
                  (uint32_t)((lane & 7) ^ (lane >> 3) ^ (c & 1)) * 16u;
  d.O.bq = buffer_rsrc(codes, (uint32_t)H * (I / 2));
  d.O.bs = buffer_rsrc(scales, (uint32_t)H * (I / 16));
  d.O.bq0 = buffer_rsrc(codes, 0u);
  d.O.bs0 = buffer_rsrc(scales, 0u);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 64 * wave + 32 * c + (lane >> 1);
    d.O.bdma[c] = (uint32_t)(nt * kBN + r) * qrow + (uint32_t)((lane & 1) ^ (((r >> 2) ^ (r >> 3)) & 1)) * 16u;
  }
  d.O.sdma = (uint32_t)(nt * kBN + 64 * wave + lane) * srow;
  d.O.bmul = km ? (uint32_t)H : 1u;
  d.y = shared ? p.y_shared + (int64_t)m0 * H : p.y_rows + (int64_t)(seg_row0 + m0) * H;
  d.m0 = m0;
  d.nt = nt;
  d.shared = shared;
  return d;
}

// The tile's output rows through a resource sized to the segment's rows in it
// (non-temporal: the combine reads them after every tile is done).  G: the
// expert's FP32 scale times the activation scale.
__device__ __forceinline__ void down_store(const FfnParams& p, const DownTile& d, float G,
                                           const floatx16 (&acc)[4][2]) {
  // H through an empty asm statement: in a loop over tiles the compiler
  // would otherwise compute the 128 store offsets of every lane once, before
  // the loop, and keep them in registers it does not have
  int H = p.H;
  asm volatile("" : "+s"(H));
  const int T = p.T, lane = lane_id();
  const __amdgpu_buffer_rsrc_t y_r = buffer_rsrc(d.y, (uint32_t)d.nrows * H * 4u);
  const uint32_t voff0 = (uint32_t)(4 * (lane >> 5) * H) * 4u;
  if (d.shared && p.sh_gate) {
    // shared rows are tokens m0 + row: each scaled by its gate, the tile's 128
    // gates staged in LDS once (rows past the segment read the last token's and
    // are dropped by the store's range check)
    __shared__ float gsh[128];
    if (threadIdx.x < 128) gsh[threadIdx.x] = p.sh_gate[d.m0 + (int)threadIdx.x < T ? d.m0 + (int)threadIdx.x : T - 1];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int dm = 32 * i + 8 * (q >> 2) + (q & 3) + 4 * (lane >> 5);
        const float gr = gsh[dm];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = d.nt * kBN + down_bj(j) + (lane & 31);
          buffer_store4_nt(__float_as_uint((G * acc[i][j][q]) * gr), y_r,
                           voff0 + (uint32_t)((dm - 4 * (lane >> 5)) * H * 4) + (uint32_t)(n * 4));
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = d.nt * kBN + down_bj(j) + (lane & 31);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int dm = 32 * i + 8 * (q >> 2) + (q & 3);
        buffer_store4_nt(__float_as_uint(G * acc[i][j][q]), y_r, voff0 + (uint32_t)(dm * H * 4) + (uint32_t)(n * 4));
      }
    }
}

// One work item per workgroup (K ranges of one or two steps: K-split partials;
// banks in different layouts).
__global__ __launch_bounds__(256, 2) void k_down_mfma(FfnParams p, const int32_t* __restrict__ tile_start,
                                                      const int4* __restrict__ tile_tab) {
  __shared__ __align__(16) Stage st0, st1, st2;
  Ring ring{st0, st1, st2};
  const int n_nt = p.H / kBN;
  const int n_tiles = tile_start[p.E + 1] * n_nt;
  if ((int)blockIdx.x >= n_tiles) return;
  const int lt = xcd_tile((int)blockIdx.x, n_tiles);
  const int4 te = tile_tab[lt / n_nt];
  const DownTile d = down_tile(p, te, lt % n_nt);
  const int seg = __builtin_amdgcn_readfirstlane(te.x);
  const float G = (d.shared ? p.sh2.gscale[0] : p.w2.gscale[seg]) * p.g_mid;
  floatx16 acc[4][2] = {};
  // K range [kc0, kc1) of I (the full sum: 0, I)
  switch (tile_blocks(d.nrows)) {
    case 1: tile_mma<false, 1>(d.O, p.kc0, p.kc1 - p.kc0, d.nrows, ring, down_bj, acc); break;
    case 2: tile_mma<false, 2>(d.O, p.kc0, p.kc1 - p.kc0, d.nrows, ring, down_bj, acc); break;
    case 3: tile_mma<false, 3>(d.O, p.kc0, p.kc1 - p.kc0, d.nrows, ring, down_bj, acc); break;
    default: tile_mma<false, 4>(d.O, p.kc0, p.kc1 - p.kc0, d.nrows, ring, down_bj, acc); break;
  }
  down_store(p, d, G, acc);
}

// The same work items with a grid of two workgroups per CU (K ranges of at
// least three steps, routed and shared banks in the same layout).  XCD x
// (= blockIdx % 8) takes the same contiguous run of work items as in
// k_down_mfma; its gx workgroups start on the run's first 3 gx items (every
// gx-th), then take the next item of the run from the XCD's counter, so the
// items in flight on an XCD stay neighbours (shared A rows and weights in its
// L2) and a slow item delays only its own workgroup.
// The LDS ring runs on from one item into the next: an item's last two steps
// transfer the next item's first two, so the next item's first transfers and
// set-up overlap this item's last MFMAs and its row stores instead of
// following them.  The tile table entry and the expert scale of an item are
// read an item ahead by vector loads (a scalar load in flight would make every
// LDS read of the K loop wait for it: both count on one counter).  A lane's
// transfer offsets are the same for every item (the column tile moves the B
// resources' base), so an item adds only scalar state.  kNm3 = steps per item
// mod 3: the ring stage of an item's first step advances by it from item to
// item, so the item loop is unrolled three times and every stage index is a
// compile-time value.
struct ChainItem {
  __amdgpu_buffer_rsrc_t a, bq, bs;  // A rows, the column tile's B codes and scales
  float* y;                          // the item's first output row
  int nrows, m0, nt;
  bool shared;
};

template <int kNm3>
__global__ __launch_bounds__(256, 2) void k_down_mfma_chain(FfnParams p, const int32_t* __restrict__ tile_start,
                                                            const int4* __restrict__ tile_tab,
                                                            int32_t* __restrict__ counters) {
  __shared__ __align__(16) Stage st0, st1, st2;
  Ring ring{st0, st1, st2};
  const int H = p.H, I = p.I, E = p.E;
  const int n_nt = H / kBN;
  const int n_mt = tile_start[E + 1];
  const int n_tiles = n_mt * n_nt;
  const int x = (int)blockIdx.x & 7, gx = (int)gridDim.x >> 3;
  const int q = n_tiles >> 3, r = n_tiles & 7;
  const int run0 = x * q + (x < r ? x : r), end = run0 + q + (x < r ? 1 : 0);
  int lt = run0 + ((int)blockIdx.x >> 3);
  if (lt >= end) return;
  // a workgroup's first three items are lt, lt + gx, lt + 2 gx; after those
  // it takes the XCD's next item from a counter, so the items in flight stay
  // consecutive and a slow item delays only its own workgroup
  __shared__ int next_slot;
  int32_t* const ctr = counters + x;
  const int dyn0 = run0 + 3 * gx;
  const int n = (p.kc1 - p.kc0) / kBK;
  const bool km = p.w2k.codes != nullptr;  // the shared bank's layout is the same
  const uint8_t* const rq = km ? p.w2k.codes : p.w2.codes;
  const uint8_t* const rs = km ? p.w2k.scales : p.w2.scales;
  const uint8_t* const sq = km ? p.sh2k.codes : p.sh2.codes;
  const uint8_t* const ss = km ? p.sh2k.scales : p.sh2.scales;
  const uint32_t qrow = km ? 32u : (uint32_t)(I / 2), srow = km ? 4u : (uint32_t)(I / 16);
  const uint32_t bmul = km ? (uint32_t)H : 1u;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  // the lane's transfer offsets (every item)
  Operands L;
#pragma unroll
  for (int c = 0; c < 4; ++c)
    L.adma[c] = (uint32_t)(32 * wave + 8 * c + (lane >> 3)) * I * 2u + (uint32_t)((lane & 7) ^ (lane >> 3) ^ (c & 1)) * 16u;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int rr = 64 * wave + 32 * c + (lane >> 1);
    L.bdma[c] = (uint32_t)rr * qrow + (uint32_t)((lane & 1) ^ (((rr >> 2) ^ (rr >> 3)) & 1)) * 16u;
  }
  L.sdma = (uint32_t)(64 * wave + lane) * srow;
  L.bmul = bmul;
  const __amdgpu_buffer_rsrc_t null_r = buffer_rsrc(p.hh, 0u);
  L.a0 = null_r;
  L.bq0 = null_r;
  L.bs0 = null_r;
  const __amdgpu_buffer_rsrc_t tt_r = buffer_rsrc(tile_tab, (uint32_t)n_mt * 16u);
  const __amdgpu_buffer_rsrc_t gw_r = buffer_rsrc(p.w2.gscale, (uint32_t)E * 4u);
  const __amdgpu_buffer_rsrc_t gs_r = buffer_rsrc(p.sh2.gscale, 4u);
  // item l's resources and output rows from its table entry te (uniform)
  auto make_item = [&](int4 te, int l) {
    const int seg = te.x, m0 = te.y, seg_row0 = te.z, seg_rows = te.w, nt = l % n_nt;
    ChainItem it;
    it.shared = seg == E;
    it.m0 = m0;
    it.nt = nt;
    it.nrows = seg_rows - m0 < kBM ? seg_rows - m0 : kBM;
    const int64_t row0 = (it.shared ? (int64_t)p.T * p.k : (int64_t)seg_row0) + m0;
    it.a = buffer_rsrc(p.hh + row0 * I, (uint32_t)it.nrows * I * 2u);
    const int64_t erow = it.shared ? 0 : (int64_t)seg * H;  // the expert's first row in the bank
    const uint32_t cq = (uint32_t)(nt * kBN) * qrow, cs = (uint32_t)(nt * kBN) * srow;
    it.bq = buffer_rsrc((it.shared ? sq : rq) + erow * (I / 2) + cq, (uint32_t)H * (I / 2) - cq);
    it.bs = buffer_rsrc((it.shared ? ss : rs) + erow * (I / 16) + cs, (uint32_t)H * (I / 16) - cs);
    it.y = it.shared ? p.y_shared + (int64_t)m0 * H : p.y_rows + (int64_t)(seg_row0 + m0) * H;
    return it;
  };
  auto with = [&](const ChainItem& it) {
    Operands O = L;
    O.a = it.a;
    O.bq = it.bq;
    O.bs = it.bs;
    return O;
  };
  // the table entry of item l (l < end) by a vector load; uniform() reads it
  // out where it is used, so that no wait follows the load
  auto entry = [&](int l) { return __builtin_amdgcn_raw_buffer_load_b128(tt_r, 0u, (uint32_t)(l / n_nt) * 16u, 0); };
  auto uniform = [](u32x4 v) {
    return make_int4(__builtin_amdgcn_readfirstlane((int)v.x), __builtin_amdgcn_readfirstlane((int)v.y),
                     __builtin_amdgcn_readfirstlane((int)v.z), __builtin_amdgcn_readfirstlane((int)v.w));
  };
  // the FP32 scale of the segment of table entry te (uniform), by a vector load
  auto gscale = [&](int4 te) {
    const bool sh = te.x == E;
    return __builtin_amdgcn_raw_buffer_load_b32(sh ? gs_r : gw_r, 0u, sh ? 0u : (uint32_t)te.x * 4u, 0);
  };
  const int4 te0 = uniform(entry(lt));
  ChainItem cur = make_item(te0, lt);
  float G = __uint_as_float(__builtin_amdgcn_readfirstlane(gscale(te0))) * p.g_mid;
  int lt1 = lt + gx, lt2 = lt1 + gx;
  int4 te1 = uniform(entry(lt1 < end ? lt1 : lt));
  // a zero the compiler cannot see through: with a uniform address it would
  // widen the one-lane atomic below to a wave-wide one whose result it waits
  // for at once
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  dma_step(with(cur), true, (uint32_t)p.kc0, ring.at<0>());
  dma_step(with(cur), true, (uint32_t)(p.kc0 + kBK), ring.at<1>());
  ring_barrier<7>();
  // one item at ring phase kPh; false when it was the workgroup's last
  auto item = [&](auto ph) -> bool {
    constexpr int kPh = decltype(ph)::value;
    const bool has1 = lt1 < end;
    const int4 t1 = te1;
    // loads for the next items, issued before this item's first transfers
    // (its first barrier then covers them), and the item after them from the
    // counter (one lane; the value goes to the other waves through LDS).  All
    // three are read out after the first step's barrier (make_on), where the
    // compiler knows that they have completed.
    const u32x4 te2v = entry(lt2 < end ? lt2 : lt);
    const uint32_t g1v = gscale(t1);
    int got;  // set and read by thread 0 only (no merge that would wait for the atomic here)
    if (threadIdx.x == 0) got = __hip_atomic_fetch_add(ctr + zero, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_sched_barrier(0);
    const ChainItem nxt = make_item(t1, lt1);
    int4 te2;
    float g1;
    auto make_on = [&] {
      if (threadIdx.x == 0) next_slot = dyn0 + got;  // read after the next barriers, at the item's end
      te2 = uniform(te2v);
      g1 = __uint_as_float(__builtin_amdgcn_readfirstlane(g1v));
      Operands On = with(nxt);
      if (!has1) {
        On.a = null_r;
        On.bq = null_r;
        On.bs = null_r;
      }
      return On;
    };
    const Operands O = with(cur);
    floatx16 acc[4][2] = {};
    switch (tile_blocks(cur.nrows)) {
      case 1: tile_mma_chain<false, 1, kPh, kNm3>(O, make_on, p.kc0, n, ring, down_bj, acc); break;
      case 2: tile_mma_chain<false, 2, kPh, kNm3>(O, make_on, p.kc0, n, ring, down_bj, acc); break;
      case 3: tile_mma_chain<false, 3, kPh, kNm3>(O, make_on, p.kc0, n, ring, down_bj, acc); break;
      default: tile_mma_chain<false, 4, kPh, kNm3>(O, make_on, p.kc0, n, ring, down_bj, acc); break;
    }
    DownTile d;
    d.y = cur.y;
    d.nrows = cur.nrows;
    d.m0 = cur.m0;
    d.nt = cur.nt;
    d.shared = cur.shared;
    down_store(p, d, G, acc);
    cur = nxt;
    G = g1 * p.g_mid;
    lt = lt1;
    lt1 = lt2;
    lt2 = __builtin_amdgcn_readfirstlane(next_slot);
    te1 = te2;
    return has1;
  };
  for (;;) {
    if (!item(IntC<0>{})) break;
    if (!item(IntC<kNm3>{})) break;
    if (!item(IntC<(2 * kNm3) % 3>{})) break;
  }
  __builtin_amdgcn_s_waitcnt(0);  // no transfer into LDS outlives the workgroup
}

// ---------------------------------------------------------------- launchers
// Buffer resources address at most 2^32 bytes: the FP16 rows of x (gathered by
// token) and one expert's weights must stay below 2^31 (h and output rows are
// addressed per 128-row tile).
bool ffn_mfma_supported(int H, int I, int E, int64_t T, int k) {
  const int64_t lim = (int64_t)1 << 31;
  return H % kBN == 0 && H % kBK == 0 && I % 128 == 0 && I % kBK == 0 && E <= 1000 && T * H * 2 < lim &&
         (int64_t)I * H < lim;
}

static int64_t mfma_max_tiles(int64_t T, int k, int E, int has_shared) {
  const int64_t P = T * k;
  return (P + kBM - 1) / kBM + (P < E ? P : E) + (has_shared ? (T + kBM - 1) / kBM : 0);
}

size_t ffn_mfma_ws_bytes(int E, int64_t T, int k, int has_shared) {
  return (size_t)tile_tab_offset(E) * sizeof(int32_t) + (size_t)mfma_max_tiles(T, k, E, has_shared) * sizeof(int4);
}

// K-step-major copy of a bank: thread i moves 16 code bytes (half of one row's
// K step) or, for i < n_exp S N, one row's 4 scale bytes of a step; both
// written in output order (contiguous), read as 16- and 4-byte pieces.
__global__ __launch_bounds__(256) void k_pack_kmajor(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int64_t n_rows_steps, int N,
                                                     int K, uint8_t* __restrict__ codes_out,
                                                     uint8_t* __restrict__ scales_out) {
  const int S = K / 64;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n_rows_steps; i += (int64_t)gridDim.x * 256) {
    const int64_t q = i >> 1;  // (e, s, n) in output order
    const int half = (int)(i & 1);
    const int n = (int)(q % N);
    const int64_t es = q / N;
    const int st = (int)(es % S);
    const int64_t e = es / S;
    const int64_t row = e * N + n;
    *reinterpret_cast<uint4*>(codes_out + i * 16) =
        *reinterpret_cast<const uint4*>(codes + row * (K / 2) + st * 32 + half * 16);
    if (half == 0)
      *reinterpret_cast<uint32_t*>(scales_out + q * 4) =
          *reinterpret_cast<const uint32_t*>(scales + row * (K / 16) + st * 4);
  }
}

hipError_t launch_pack_kmajor(const uint8_t* codes, const uint8_t* scales, int n_exp, int N, int K, uint8_t* codes_out,
                              uint8_t* scales_out, hipStream_t s) {
  const int64_t n = (int64_t)n_exp * (K / 64) * N;
  const int64_t blocks = (2 * n + 255) / 256;
  hipLaunchKernelGGL(k_pack_kmajor, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s, codes, scales,
                     n, N, K, codes_out, scales_out);
  return hipGetLastError();
}

// Workgroups of a chained kernel: two per CU (what its LDS ring allows), at
// most one per work item, a multiple of 8 (the XCDs take workgroups in turn).
static int chain_grid(int64_t items) {
  static int cus[16] = {};  // per device; every thread that fills it writes the same value
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int c = dev < 16 ? cus[dev] : 0;
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
    if (dev < 16) cus[dev] = c;
  }
  const int64_t g = items < 2 * (int64_t)c ? items : 2 * (int64_t)c;
  return (int)((g + 7) / 8 * 8);
}

hipError_t launch_ffn_mfma(const FfnParams& p, int32_t* tile_start, hipStream_t s, hipEvent_t* ev) {
  const int64_t max_tiles = mfma_max_tiles(p.T, p.k, p.E, p.has_shared);
  int4* tile_tab = reinterpret_cast<int4*>(tile_start + tile_tab_offset(p.E));
  hipLaunchKernelGGL(k_tile_map, dim3(1), dim3(1024), 0, s, p.off, p.E, p.T, p.has_shared, tile_start, tile_tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_timed(k_gateup_mfma, dim3((unsigned)(max_tiles * (p.I / 128))), dim3(256), 0, s, ev ? ev[2] : nullptr,
                   ev ? ev[3] : nullptr, p, (const int32_t*)tile_start, (const int4*)tile_tab);
  if (e != hipSuccess) return e;
  const int64_t items = max_tiles * (p.H / kBN);
  const int n = (p.kc1 - p.kc0) / kBK;
  // the chained kernel: at least three K steps per item, both banks in one layout
  if (n < 3 || (p.w2k.codes != nullptr) != (p.sh2k.codes != nullptr))
    return launch_timed(k_down_mfma, dim3((unsigned)items), dim3(256), 0, s, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr,
                        p, (const int32_t*)tile_start, (const int4*)tile_tab);
  const dim3 g((unsigned)chain_grid(items));
  auto k = n % 3 == 0 ? k_down_mfma_chain<0> : n % 3 == 1 ? k_down_mfma_chain<1> : k_down_mfma_chain<2>;
  return launch_timed(k, g, dim3(256), 0, s, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr, p,
                      (const int32_t*)tile_start, (const int4*)tile_tab, tile_start + p.E + 2);
}

}  // namespace moe

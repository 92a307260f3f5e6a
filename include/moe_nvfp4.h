/*
 * moe_nvfp4.h -- C ABI of the routed NVFP4 W4A4 mixture-of-experts layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (pages cited by title and section):
 *   - router logits over E experts, top-k routed experts plus one always-on
 *     shared expert (capy-flash README v0.5.4, synthetic test-artifact script:
 *     "512 NVFP4 experts top-10 + shared"; Richland article, "What shipped");
 *   - expert weights in NVFP4: E2M1 codes, UE4M3 block scales, an FP32
 *     per-expert scale, taken from the checkpoint unchanged (Richland
 *     article, "What shipped");
 *   - activations quantized the same way (W4A4) wherever an expert runs
 *     (capy-flash README v0.5.4, "What it does" and "Serve");
 *   - FP32 accumulation of partials (Richland article, "Why it matters");
 *   - every selected expert is computed and combined with its router weight
 *     (none is skipped; capy-flash README v0.7.7, "Benchmarks").
 * Readings where the pages are silent: 16-element blocks, block scale =
 * RNE(amax/6) on the UE4M3 grid, element codes RNE onto E2M1 with
 * saturation, SwiGLU (h = silu(gate) * up), softmax over the k selected
 * logits, shared-expert weight 1, element 2i in the low nibble of byte i.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer, including the workspace; the library never allocates or
 *     frees device memory and keeps no mutable global state.
 *   - Calls are asynchronous on `stream`; none synchronizes the host, so a
 *     sequence of calls may be captured into a HIP graph.
 *   - Arguments are validated on the host only; a kernel fault surfaces at
 *     the caller's next synchronization.
 *   - All device pointers must be 16-byte aligned (MOE_EINVAL otherwise).
 *   - T == 0 is a successful no-op.
 *   - Results are deterministic run to run (no floating-point atomics).
 *   - Return value: MOE_OK (0) or a negative MOE_E* code; moe_strerror()
 *     names it.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* null required pointer, misaligned pointer, bad dtype   */
  MOE_ESHAPE = -2,     /* H or I not a multiple of 32, k outside [1, min(E,32)],
                          E outside [1, 1024], H > 16384, I > 4096, or a token
                          count T outside 0 <= T, T*H*2 < 2^31, T*(k+1) < 2^31
                          (32-bit row offsets and int32 pair ids; at H = 2048:
                          T < 524,288)                                         */
  MOE_EWORKSPACE = -3, /* workspace smaller than moe_workspace_bytes()          */
  MOE_ELAUNCH = -4     /* a kernel launch failed (hipGetLastError)              */
};

/* One bank of NVFP4 matrices, n_exp matrices of N rows by K columns:
 *   codes  [n_exp][N][K/2]  E2M1 codes, element 2i of a row in the low nibble
 *                           of byte i, element 2i+1 in the high nibble
 *   scales [n_exp][N][K/16] UE4M3 scale per 16 consecutive elements of a row
 *                           (bit 7 must be 0; 0x7F is never used)
 *   gscale [n_exp]          FP32 per-matrix scale
 * A weight's value is e2m1(code) * ue4m3(scale) * gscale.                    */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
} moe_nvfp4_bank;

/* One MoE layer.  Host struct; the pointers inside are device pointers.
 *   w13 : routed experts, n_exp = E, N = 2I, K = H; rows 0..I-1 are the gate
 *         projection, rows I..2I-1 the up projection
 *   w2  : routed experts, n_exp = E, N = H, K = I (down projection)
 *   sh13, sh2 : the shared expert (n_exp = 1), same shapes; ignored when
 *         has_shared == 0
 *   router_w : [E][H] FP32 router weights
 *   a_gscale_in, a_gscale_mid : global scales of the activation encodings of
 *         x and of h; powers of two (1.0 by default)
 *   w13k, w2k, sh13k, sh2k : optional K-step-major copies (moe_pack_kmajor) of
 *         the codes and scales of w13, w2, sh13, sh2 (their gscale is not
 *         read).  Where a copy's codes pointer is non-null, the matrix-core
 *         kernels (prompt chunks) read the copy, whose K steps are contiguous
 *         runs; otherwise they read the row-major bank.  Results are identical
 *         either way; the decode and weight-streaming kernels always read the
 *         row-major banks.  Zero-initialise the struct to leave them unset.
 *   shared_gate_w : optional [H] FP32 gate vector of the shared expert (null:
 *         no gate, the shared expert's weight is 1).  With it, the shared
 *         expert's output row of token t is multiplied by
 *         g_t = fl32(sigmoid(sum_h x[t][h] * shared_gate_w[h])), the sum in FP64
 *         over exact products and the sigmoid in FP64 (y_shared holds the gated
 *         rows).  The pages print no gate on the shared expert; this is the
 *         plainest form an optional gate takes (a streamed-prefill hand-off
 *         with such a gate is what the pages' model family runs).
 *   router_pieces : optional [3][E][H] BF16 pieces of router_w written once by
 *         moe_pack_router; where set, the matrix-core router reads them
 *         instead of splitting router_w on every call (identical results).
 *   router_mode : MOE_ROUTER_EXACT (0, the default), MOE_ROUTER_SPLIT3_F32 or
 *         MOE_ROUTER_BF16; see moe_route.
 *   act_bits : activation encoding of x and h: 0 or 4 = A4 (W4A4, the
 *         default); 8 = A8, the W4A8 variant (the pages' older host path,
 *         capy-flash README v0.5.4, "Serve"; its format is not given there):
 *         the same 16-element blocks and UE4M3 block scale, chosen as
 *         RNE(amax / (127 g)), with INT8 element codes q = RNE(x / (s g))
 *         saturating at +-127.  A power-of-two activation global scale below 1
 *         (e.g. 2^-4 for N(0,1) hidden states) keeps its block scales in UE4M3's
 *         normal range.  Other values are MOE_ESHAPE.
 *   pre_norm, pre_norm_eps : moe_layer_forward only.  pre_norm = 1: the layer's
 *         input is moe_rms_norm(x, pre_norm_eps) instead of x (the stack's
 *         composition in one call; the residual argument is still added as
 *         given), with results identical to the two calls; 0 (the default):
 *         x as given.  The separate calls ignore these fields.  Other values,
 *         or pre_norm_eps outside [0, 1], are MOE_EINVAL.                     */
typedef struct {
  int32_t H, I, E, k, has_shared;
  const float* router_w;
  moe_nvfp4_bank w13, w2, sh13, sh2;
  float a_gscale_in, a_gscale_mid;
  moe_nvfp4_bank w13k, w2k, sh13k, sh2k;
  const float* shared_gate_w;
  const uint16_t* router_pieces;
  int32_t router_mode;
  int32_t act_bits;
  int32_t pre_norm;
  double pre_norm_eps;
} moe_layer;

enum { MOE_ROUTER_EXACT = 0, MOE_ROUTER_SPLIT3_F32 = 1, MOE_ROUTER_BF16 = 2 };

/* Optional dumps of intermediate values (all nullable, device pointers).
 *   xq [T][H/2], xs [T][H/16] : A4 encoding of x (codes, UE4M3 scales);
 *                               A8 layers: xq [T][H] INT8 codes
 *   h  [R][I] FP32            : h = silu(gate) * up before its encoding
 *   hq [R][I/2], hs [R][I/16] : A4 encoding of h; A8 layers: hq [R][I] INT8
 * R = T*k routed rows in permuted-row order, followed by T shared-expert rows
 * (token order) when has_shared.
 *   events (host array, nullable): 2*MOE_FFN_KERNELS created HIP events (a null
 *   entry is MOE_EINVAL); events[2i] and events[2i+1] take the start and end
 *   timestamps of kernel i of moe_expert_ffn itself (0: A4(x), 1: gate/up +
 *   SwiGLU + A4(h), 2: down projection), so hipEventElapsedTime gives that
 *   kernel's execution time; a kernel that a path does not run has both events
 *   recorded at the same point.  The kernels are the same with or without dumps
 *   and events.                                                              */
#define MOE_FFN_KERNELS 3
typedef struct {
  uint8_t* xq;
  uint8_t* xs;
  float* h;
  uint8_t* hq;
  uint8_t* hs;
  hipEvent_t* events;
} moe_debug;

int moe_abi_version(void);
const char* moe_strerror(int code);

/* Bytes of workspace that moe_route, moe_permute, moe_expert_ffn and
 * moe_layer_forward need for up to T_max tokens of layer L (one workspace may
 * serve all of them, not concurrently).  Returns 0 if L or T_max is invalid
 * (including a T_max beyond the token bound of MOE_ESHAPE).
 * Host call.  The workspace is scratch: nothing is kept between calls.       */
size_t moe_workspace_bytes(const moe_layer* L, int64_t T_max);

/* Router: logits l[t][e] = sum_h x[t][h] * router_w[e][h], the k largest per
 * token in descending order (equal logits: lower expert id first), and
 * w[t][j] = softmax over the k selected logits (FP64, rounded to FP32).
 * Precision (L->router_mode):
 *   MOE_ROUTER_EXACT      the selection is taken on FP64 sums of the exact
 *                         products, so it does not depend on summation order
 *                         (see route.hip)
 *   MOE_ROUTER_SPLIT3_F32 FP32 logits from BF16 matrix-core products of x with
 *                         the three exact BF16 pieces of router_w (FP32 sums),
 *                         selected as they are: a reordered FP32 sum, which may
 *                         resolve a near tie either way
 *   MOE_ROUTER_BF16       router_w rounded to BF16 (nearest, ties to even),
 *                         one BF16 matrix-core pass with FP32 sums, selected as
 *                         is: a reduced-precision router, which also moves
 *                         the logits by the rounding of the weights
 * The two reduced modes need E % 128 == 0 and H % 32 == 0 (MOE_ESHAPE
 * otherwise) and take the matrix cores at every T.
 *   x        [T][H] BF16 hidden states (bit patterns)
 *   logits_in [T][E] FP32, nullable: when given, these logits are used as is
 *             (test hook for tie-breaking rules; the mode is then ignored)
 *   topk_idx [T][k] int32 out; topk_w [T][k] FP32 out
 * Pages: capy-flash README v0.5.4, "Measured" footnote (router on tensor cores
 * for prompt chunks; reordered sums may pick another of two tied experts).   */
int moe_route(const moe_layer* L, const uint16_t* x, int64_t T, const float* logits_in, int32_t* topk_idx,
              float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream);

/* Permutation: groups the T*k (token, slot) pairs by expert, expert id
 * ascending and token ascending within an expert (pair id p = t*k + j).
 *   topk_idx   [T][k] int32 in (each row: k distinct ids in [0, E))
 *   expert_off [E+1] int32 out: exclusive prefix sum of per-expert counts
 *   row2pair   [T*k] int32 out: pair id held by permuted row r
 *   pair2row   [T*k] int32 out: inverse of row2pair
 * Pages: capy-flash README v0.5.4, "What it does" (experts partitioned by id). */
int moe_permute(const moe_layer* L, const int32_t* topk_idx, int64_t T, int32_t* expert_off, int32_t* row2pair,
                int32_t* pair2row, void* ws, size_t ws_bytes, hipStream_t stream);

/* Expert FFN, routed and shared:
 *   (xq, xs) = A4(x) per 16-element block of H with a_gscale_in
 *   for permuted row r (pair p = row2pair[r], token t = p / k, expert e):
 *     gate_i, up_i = W13_e . dequant(xq, xs) in FP32, h_i = silu(gate_i)*up_i
 *     (hq, hs) = A4(h) per 16-block of I with a_gscale_mid
 *     y_rows[r][n] = W2_e[n] . dequant(hq, hs) in FP32
 *   y_shared[t][n]: the same with the shared expert for every token (times
 *     the token's gate g_t when L->shared_gate_w is set)
 *   expert_off, row2pair as produced by moe_permute
 *   y_rows [T*k][H] FP32 out (permuted-row order)
 *   y_shared [T][H] FP32 out; nullable iff has_shared == 0
 *   dbg nullable (see moe_debug)
 * Pages: Richland article, "What shipped" (NVFP4 format) and "Why it matters"
 * (FP32 accumulation); capy-flash README v0.5.4, "Serve" (W4A4).              */
int moe_expert_ffn(const moe_layer* L, const uint16_t* x, int64_t T, const int32_t* expert_off,
                   const int32_t* row2pair, float* y_rows, float* y_shared, const moe_debug* dbg, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/* moe_expert_ffn with the down projection summed over the 16-element blocks
 * [kb0, kb1) of I only: y_rows / y_shared receive that K-split partial (the
 * gate/up, SwiGLU and A4(h) steps are the full ones).  Two calls with
 * [0, I/32) and [I/32, I/16) give the two partial products that a
 * two-way split of the down projection would exchange (Richland article, "Why
 * it matters": partial sums exchanged in BF16 lose accuracy, FP16 with a 2^-k
 * shift keeps it).  kb0 < kb1 <= I/16, both even; a partial range runs on the
 * matrix-core kernels (T >= 32, kb0 and kb1 multiples of 4) or the generic
 * ones.  Errors as moe_expert_ffn, MOE_ESHAPE for a bad range.               */
int moe_expert_ffn_krange(const moe_layer* L, const uint16_t* x, int64_t T, const int32_t* expert_off,
                          const int32_t* row2pair, int32_t kb0, int32_t kb1, float* y_rows, float* y_shared,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* The un-rounded FP32 output of the combine without residual:
 *   out[t] = sum_j topk_w[t][j] * y_rows[pair2row[t*k+j]] + y_shared[t]
 * summed exactly as moe_combine sums before its rounding (j ascending, then
 * the shared row).  out [T][H] FP32 device.                                  */
int moe_combine_f32(const moe_layer* L, int64_t T, const float* y_rows, const float* y_shared,
                    const int32_t* pair2row, const float* topk_w, float* out, hipStream_t stream);

/* Combine: out[t] = RNE_BF16( sum_j topk_w[t][j] * y_rows[pair2row[t*k+j]]
 *                             + y_shared[t] + residual[t] ), summed in FP32 in
 * that order (j ascending).  y_shared nullable iff has_shared == 0; residual
 * [T][H] BF16 nullable; out [T][H] BF16.  Needs no workspace.
 * Pages: capy-flash README v0.7.7, "Benchmarks" (every selected expert is
 * computed); Richland article, "Why it matters" (FP32 partials).             */
int moe_combine(const moe_layer* L, int64_t T, const float* y_rows, const float* y_shared, const int32_t* pair2row,
                const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t stream);

/* The whole layer in one call: route -> permute -> expert FFN -> combine, with
 * every output of the four calls above written exactly as they write it
 * (topk_idx, topk_w [T][k]; expert_off [E+1]; row2pair, pair2row [T*k];
 * y_rows [T*k][H]; y_shared [T][H] (nullable iff !has_shared); out [T][H];
 * residual nullable).  For decode batches (T <= 4, H <= 2048, E <= 512, no
 * dumps requested, the exact router; A4 or A8 activations; events allowed) it
 * runs fused in three kernels: router (FP64 logits and the codes of x; events 0/1
 * of moe_debug), gate/up (events 2/3; each workgroup selects the top k of the
 * batch, the softmax weights, the permutation and its expert from the FP64
 * logits, and one extra workgroup writes them out), down projection with the
 * combine (events 4/5; one workgroup per token and 4 output columns, when
 * (k + has_shared) * I / 32 <= 256, else a down kernel and the combine
 * kernel).  Otherwise it runs the four calls in order.  Results are identical
 * either way.  ws must hold moe_workspace_bytes(L, T_max) bytes with
 * T <= T_max.
 * Pages: capy-flash README v0.5.4, "What it does" (a routed layer computed
 * per expert id with the W4A4 quantization).                                */
int moe_layer_forward(const moe_layer* L, const uint16_t* x, int64_t T, const uint16_t* residual,
                      int32_t* topk_idx, float* topk_w, int32_t* expert_off, int32_t* row2pair, int32_t* pair2row,
                      float* y_rows, float* y_shared, uint16_t* out, const moe_debug* dbg, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a device array inside
 * the library of moe_noalloc_scratch_bytes() bytes (64 MiB), one per GPU the
 * library runs on, held until the process ends; this call allocates nothing.
 * Arguments, outputs and results are those of moe_layer_forward (same
 * kernels).  MOE_EWORKSPACE when moe_workspace_bytes(L, T) exceeds the array
 * (at hidden 2048, 512 experts, top 10 + shared, intermediate 512: more than
 * 3,391 tokens); the size is checked before anything else touches the GPU.  The array of the current device is used (the stream
 * must belong to it).  Every call on a GPU shares that GPU's array and leaves
 * its contents behind (no call needs it cleared); calls that overlap in time
 * on one GPU race.                                                            */
size_t moe_noalloc_scratch_bytes(void);
int moe_layer_forward_noalloc(const moe_layer* L, const uint16_t* x, int64_t T, const uint16_t* residual,
                              int32_t* topk_idx, float* topk_w, int32_t* expert_off, int32_t* row2pair,
                              int32_t* pair2row, float* y_rows, float* y_shared, uint16_t* out,
                              const moe_debug* dbg, hipStream_t stream);

/* Parameter-free RMS norm of BF16 rows, the composition that chains layers
 * into a stack (the pages run 48 MoE layers, Richland article, "What
 * shipped"; the block structure around them is not printed):
 *   out[t][h] = RNE_BF16( x[t][h] / sqrt(mean_h x[t][h]^2 + eps) )
 * with the sum of squares, the scale and the product in FP64.
 *   x, out [T][H] BF16 device (16-byte aligned); 0 <= eps <= 1.
 * Errors: MOE_ESHAPE (T < 0, H <= 0), MOE_EINVAL (pointers, eps).            */
int moe_rms_norm(const uint16_t* x, int64_t T, int32_t H, double eps, uint16_t* out, hipStream_t stream);

/* A4 encoding of a row-major [rows][cols] matrix (cols % 16 == 0):
 *   dtype MOE_DTYPE_BF16 (x is uint16 BF16 patterns) or MOE_DTYPE_F32
 *   gscale: power-of-two global scale (host)
 *   codes [rows][cols/2], scales [rows][cols/16] out
 * Per 16-element block: scale = RNE(amax/(6*gscale)) on the UE4M3 grid,
 * saturating at 448; codes = RNE(|x|/(scale*gscale)) on the E2M1 grid,
 * saturating at 6, sign bit = sign of x.  Exact (decided by comparisons).
 * Pages: capy-flash README v0.5.4, "Serve" (the GPU's W4A4 quantization).    */
enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 };
int moe_quantize_act(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, uint8_t* codes,
                     uint8_t* scales, hipStream_t stream);

/* The three BF16 pieces of a router (written once per layer, named in
 * moe_layer.router_pieces): router_w[e][h] = p1 + p2 + p3 exactly, p1 = the
 * upper 16 bits of the FP32 value, p2 those of the remainder, p3 those of the
 * last remainder (truncation; FP32 keeps at most 24 significant bits, so three
 * 8-bit pieces hold it exactly).  pieces_out [3][E][H] BF16.  This is the
 * operand of the matrix-core router pass (capy-flash README v0.5.4, "Measured":
 * the prompt router on tensor cores).
 * Errors: MOE_ESHAPE (E < 1, H < 1), MOE_EINVAL (null or misaligned pointer). */
int moe_pack_router(const float* router_w, int32_t E, int32_t H, uint16_t* pieces_out, hipStream_t stream);

/* A8 encoding (the W4A8 variant's, see moe_layer.act_bits) of a row-major
 * [rows][cols] matrix (cols % 16 == 0): codes [rows][cols] INT8 out, scales
 * [rows][cols/16] out.  Per 16-element block: scale = RNE(amax/(127*gscale))
 * on the UE4M3 grid, saturating at 448; codes = RNE(x/(scale*gscale)) on the
 * integers, saturating at +-127.  Exact (decided by comparisons with exact
 * thresholds).  Errors and dtype as moe_quantize_act.
 * Pages: capy-flash README v0.5.4, "Serve" (the older W4A8 host path).      */
int moe_quantize_act8(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, int8_t* codes,
                      uint8_t* scales, hipStream_t stream);

/* K-step-major copy of one NVFP4 bank (the format of moe_nvfp4_bank: the
 * pages' 16-element E2M1 blocks with UE4M3 scales, Richland article, "What
 * shipped"), for the matrix-core kernels.  With S = K/64 steps of 64 elements:
 *   codes_out  [n_exp][S][N][32] : bytes 32s .. 32s+31 of row n (its elements
 *                                  64s .. 64s+63, same nibble order)
 *   scales_out [n_exp][S][N][4]  : scales 4s .. 4s+3 of row n
 * so that one K step of consecutive rows is one contiguous run of memory.
 *   codes, scales : the row-major bank (device, 16- and 4-byte aligned)
 *   codes_out [n_exp*N*K/2], scales_out [n_exp*N*K/16] : device, caller-owned,
 *                   16- and 4-byte aligned, not overlapping the inputs
 * A pure permutation of bytes; run once per layer, before the copies are
 * named in a moe_layer.
 * Errors: MOE_EINVAL (null or misaligned pointer), MOE_ESHAPE (n_exp < 1,
 * N < 1, K < 64 or K % 64 != 0).                                             */
int moe_pack_kmajor(const uint8_t* codes, const uint8_t* scales, int32_t n_exp, int32_t N, int32_t K,
                    uint8_t* codes_out, uint8_t* scales_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */

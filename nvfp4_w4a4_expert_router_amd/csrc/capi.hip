// C ABI of the NVFP4 W4A4 MoE layer: host-side validation, workspace layout
// and kernel dispatch.  Declarations and the full contract are in
// include/moe_nvfp4.h.
#include <math.h>
#include <stdint.h>

#include "common.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }

inline bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }

// the A4 comparisons are exact only for power-of-two global scales
inline bool pow2_scale(float g) {
  if (!(g > 0.0f) || g > 1e30f || g < 1e-30f) return false;
  int e;
  return frexpf(g, &e) == 0.5f;
}

int check_bank(const moe_nvfp4_bank& b) {
  return (ptr_ok(b.codes) && ptr_ok(b.scales) && ptr_ok(b.gscale)) ? MOE_OK : MOE_EINVAL;
}

int check_shape(const moe_layer* L) {
  if (!L) return MOE_EINVAL;
  if (L->H <= 0 || L->I <= 0 || L->H % 32 || L->I % 32 || L->H > 16384 || L->I > 4096) return MOE_ESHAPE;
  if (L->E < 1 || L->E > 1024) return MOE_ESHAPE;
  if (L->k < 1 || L->k > 32 || L->k > L->E) return MOE_ESHAPE;
  if (L->has_shared != 0 && L->has_shared != 1) return MOE_ESHAPE;
  if (L->router_mode < MOE_ROUTER_EXACT || L->router_mode > MOE_ROUTER_BF16) return MOE_ESHAPE;
  if (L->act_bits != 0 && L->act_bits != 4 && L->act_bits != 8) return MOE_ESHAPE;
  return MOE_OK;
}

// A8 (the W4A8 variant): one code byte per element instead of two per byte
inline bool act8(const moe_layer* L) { return L->act_bits == 8; }

// the shared expert's gate is applied only when the layer has a shared expert
inline const float* shared_gate(const moe_layer* L) { return L->has_shared ? L->shared_gate_w : nullptr; }

// Token counts: the router's and the matrix-core kernels' buffer resources
// address a call's [T][H] BF16 rows with 32-bit offsets, and pair ids and
// permuted rows are int32, so T * H * 2 and T * (k + 1) stay below 2^31.
inline bool tokens_ok(const moe_layer* L, int64_t T) {
  const int64_t lim = (int64_t)1 << 31;
  return T >= 0 && T < lim / (2 * (int64_t)L->H) && T < lim / ((int64_t)L->k + 1);
}

// an optional K-step-major copy: absent (null codes) or codes and scales
// aligned, with K a whole number of 64-element steps
int check_kmajor(const moe_nvfp4_bank& b, int K) {
  if (!b.codes) return MOE_OK;
  if (!aligned16(b.codes) || !b.scales || reinterpret_cast<uintptr_t>(b.scales) % 4) return MOE_EINVAL;
  return K % 64 ? MOE_ESHAPE : MOE_OK;
}

int check_layer(const moe_layer* L, bool need_router, bool need_experts) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (need_router) {
    if (!ptr_ok(L->router_w) || !opt_ok(L->router_pieces)) return MOE_EINVAL;
    if (!route_mode_supported(L->H, L->E, L->router_mode)) return MOE_ESHAPE;
  }
  if (need_experts) {
    if ((rc = check_bank(L->w13)) || (rc = check_bank(L->w2))) return rc;
    if (L->has_shared && ((rc = check_bank(L->sh13)) || (rc = check_bank(L->sh2)))) return rc;
    if ((rc = check_kmajor(L->w13k, L->H)) || (rc = check_kmajor(L->w2k, L->I))) return rc;
    if (L->has_shared && ((rc = check_kmajor(L->sh13k, L->H)) || (rc = check_kmajor(L->sh2k, L->I)))) return rc;
    if (!pow2_scale(L->a_gscale_in) || !pow2_scale(L->a_gscale_mid)) return MOE_EINVAL;
    if (!opt_ok(L->shared_gate_w)) return MOE_EINVAL;
  }
  return MOE_OK;
}

// workspace of each call, laid out from offset 0 (calls never overlap in time)

size_t route_ws(const moe_layer* L, int64_t T) { return align_up(route_ws_bytes(T, L->E, L->H, L->router_mode)); }

size_t permute_ws(const moe_layer* L, int64_t T) { return align_up(permute_ws_bytes(T, L->E)); }

struct FfnWs {
  size_t xq, xs, xh, hh, hq, hs, tiles, gate, end;
};

FfnWs ffn_ws(const moe_layer* L, int64_t T) {
  FfnWs w;
  const int64_t R = T * L->k + (L->has_shared ? T : 0);
  size_t o = 0;
  w.xq = o;
  o = align_up(o + (size_t)T * (act8(L) ? L->H : L->H / 2));
  w.xs = o;
  o = align_up(o + (size_t)T * (L->H / 16));
  w.xh = o;
  o = align_up(o + (size_t)T * L->H * sizeof(half_t));
  w.hh = o;
  o = align_up(o + (size_t)R * L->I * sizeof(half_t));
  w.hq = o;
  o = align_up(o + (size_t)R * (act8(L) ? L->I : L->I / 2));
  w.hs = o;
  o = align_up(o + (size_t)R * (L->I / 16));
  w.tiles = o;
  o = align_up(o + ffn_mfma_ws_bytes(L->E, T, L->k, L->has_shared));
  w.gate = o;  // the shared expert's per-token gate, when the layer has one
  o = align_up(o + (shared_gate(L) ? (size_t)T * sizeof(float) : 0));
  w.end = o;
  return w;
}

inline int launch_rc(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null or misaligned pointer, bad dtype or scale)";
    case MOE_ESHAPE:
      return "unsupported shape (H, I multiples of 32; 1 <= k <= min(E, 32); E <= 1024; 0 <= T, T*H*2 < 2^31, "
             "T*(k+1) < 2^31)";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_ELAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

// FP64 logits and the slot table of the fused decode path sit before the
// expert-FFN workspace
// fused decode path: FP64 logits, slot table, token-major copy of the routed output rows
size_t fused_logits_ws(const moe_layer* L, int64_t T) {
  const int64_t t = T < 4 ? T : 4;
  return align_up((size_t)t * L->E * sizeof(double)) + align_up((size_t)t * L->k * sizeof(int4)) +
         align_up((size_t)t * L->k * L->H * sizeof(float)) +
         align_up(shared_gate(L) ? (size_t)t * sizeof(float) : 0);
}

size_t moe_workspace_bytes(const moe_layer* L, int64_t T_max) {
  if (check_shape(L) != MOE_OK || !tokens_ok(L, T_max)) return 0;
  size_t need = route_ws(L, T_max);
  if (permute_ws(L, T_max) > need) need = permute_ws(L, T_max);
  if (ffn_ws(L, T_max).end > need) need = ffn_ws(L, T_max).end;
  need += fused_logits_ws(L, T_max);
  if (L->pre_norm == 1) need += align_up((size_t)T_max * L->H * sizeof(uint16_t));  // the normed input
  return need < kAlign ? kAlign : need;
}

int moe_route(const moe_layer* L, const uint16_t* x, int64_t T, const float* logits_in, int32_t* topk_idx,
              float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!tokens_ok(L, T)) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ptr_ok(topk_idx) || !ptr_ok(topk_w)) return MOE_EINVAL;
  if (!logits_in) {
    if ((rc = check_layer(L, true, false))) return rc;
    if (!ptr_ok(x) || !ptr_ok(ws)) return MOE_EINVAL;
    if (ws_bytes < route_ws(L, T)) return MOE_EWORKSPACE;
  } else if (!aligned16(logits_in)) {
    return MOE_EINVAL;
  }
  return launch_rc(launch_route(x, L->router_w, T, L->H, L->E, L->k, logits_in, topk_idx, topk_w,
                                logits_in ? nullptr : ws, L->router_mode, L->router_pieces, stream));
}

int moe_permute(const moe_layer* L, const int32_t* topk_idx, int64_t T, int32_t* expert_off, int32_t* row2pair,
                int32_t* pair2row, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!tokens_ok(L, T)) return MOE_ESHAPE;
  if (!ptr_ok(expert_off)) return MOE_EINVAL;
  if (T > 0 && (!ptr_ok(topk_idx) || !ptr_ok(row2pair) || !ptr_ok(pair2row) || !ptr_ok(ws))) return MOE_EINVAL;
  if (T > 0 && ws_bytes < permute_ws(L, T)) return MOE_EWORKSPACE;
  if (T == 0) return MOE_OK;
  return launch_rc(launch_permute(topk_idx, T, L->k, L->E, expert_off, row2pair, pair2row, ws, stream));
}

// dumps aligned or null; when an event array is given, every entry is a created event
static bool debug_ok(const moe_debug* d) {
  if (!d) return true;
  if (!opt_ok(d->xq) || !opt_ok(d->xs) || !opt_ok(d->h) || !opt_ok(d->hq) || !opt_ok(d->hs)) return false;
  if (d->events)
    for (int i = 0; i < 2 * MOE_FFN_KERNELS; ++i)
      if (!d->events[i]) return false;
  return true;
}

}  // extern "C"

// moe_expert_ffn with the down projection restricted to the I-blocks [kb0, kb1)
static int expert_ffn(const moe_layer* L, const uint16_t* x, int64_t T, const int32_t* expert_off,
                      const int32_t* row2pair, int kb0, int kb1, float* y_rows, float* y_shared,
                      const moe_debug* dbg, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_layer(L, false, true);
  if (rc) return rc;
  if (!tokens_ok(L, T)) return MOE_ESHAPE;
  const bool partial = kb0 != 0 || kb1 != L->I / 16;
  if (partial && (kb0 < 0 || kb1 > L->I / 16 || kb0 >= kb1 || kb0 % 2 || kb1 % 2)) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ptr_ok(x) || !ptr_ok(expert_off) || !ptr_ok(row2pair) || !ptr_ok(y_rows) || !ptr_ok(ws)) return MOE_EINVAL;
  if (L->has_shared && !ptr_ok(y_shared)) return MOE_EINVAL;
  if (!debug_ok(dbg)) return MOE_EINVAL;
  const FfnWs lay = ffn_ws(L, T);
  if (ws_bytes < lay.end) return MOE_EWORKSPACE;
  char* base = static_cast<char*>(ws);
  uint8_t* xq = reinterpret_cast<uint8_t*>(base + lay.xq);
  uint8_t* xs = reinterpret_cast<uint8_t*>(base + lay.xs);
  half_t* xh = reinterpret_cast<half_t*>(base + lay.xh);
  hipEvent_t* ev = dbg ? dbg->events : nullptr;
  // path by batch size: decode kernels (T <= 4), matrix cores (T >= 32), weight
  // streaming in between; generic kernels for shapes the others do not cover
  // (a K-split partial runs on the matrix cores or the generic kernels)
  const bool decode_path = !partial && ffn_decode_supported(L->H, L->I, T);
  const bool mfma_path = !decode_path && T >= 32 && ffn_mfma_supported(L->H, L->I, L->E, T, L->k) && kb0 % 4 == 0 &&
                         kb1 % 4 == 0;
  const bool stream_path = !partial && !decode_path && !mfma_path && ffn_stream_supported(L->H, L->I);
  const bool self_encoding = stream_path;  // these kernels encode x themselves
  const bool want_xdump = dbg && (dbg->xq || dbg->xs);
  // kernel 0: A4(x) codes into the workspace (plus a dequantized FP16 copy for
  // the generic kernels)
  if (!self_encoding || want_xdump) {
    if ((rc = launch_rc(launch_quant_act(x, MOE_DTYPE_BF16, T, L->H, L->a_gscale_in, xq, xs,
                                         self_encoding || decode_path ? nullptr : xh, stream,
                                         ev ? ev[0] : nullptr,
                                         ev ? ev[1] : nullptr, act8(L) ? 8 : 4))))
      return rc;
  } else if (ev && record_idle(stream, ev[0], ev[1]) != hipSuccess) {
    return MOE_ELAUNCH;
  }
  if (dbg && dbg->xq)
    if (hipMemcpyAsync(dbg->xq, xq, (size_t)T * (act8(L) ? L->H : L->H / 2), hipMemcpyDeviceToDevice, stream) !=
        hipSuccess)
      return MOE_ELAUNCH;
  if (dbg && dbg->xs)
    if (hipMemcpyAsync(dbg->xs, xs, (size_t)T * (L->H / 16), hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return MOE_ELAUNCH;
  FfnParams p = {};
  p.H = L->H;
  p.I = L->I;
  p.E = L->E;
  p.k = L->k;
  p.T = (int)T;
  p.has_shared = L->has_shared;
  const int64_t P = T * L->k;
  p.n_routed_slots = (int)(P < L->E ? P : L->E);
  p.off = expert_off;
  p.row2pair = row2pair;
  p.x = x;
  p.xh = xh;
  p.xq = xq;
  p.xs = xs;
  p.w13 = L->w13;
  p.w2 = L->w2;
  p.sh13 = L->sh13;
  p.sh2 = L->sh2;
  p.w13k = L->w13k;
  p.w2k = L->w2k;
  p.sh13k = L->has_shared ? L->sh13k : moe_nvfp4_bank{};
  p.sh2k = L->has_shared ? L->sh2k : moe_nvfp4_bank{};
  p.g_in = L->a_gscale_in;
  p.g_mid = L->a_gscale_mid;
  p.hh = reinterpret_cast<half_t*>(base + lay.hh);
  p.h_dbg = dbg ? dbg->h : nullptr;
  p.hq_dbg = dbg ? dbg->hq : nullptr;
  p.hs_dbg = dbg ? dbg->hs : nullptr;
  p.y_rows = y_rows;
  p.y_shared = L->has_shared ? y_shared : nullptr;
  p.kc0 = 16 * kb0;
  p.kc1 = 16 * kb1;
  p.act8 = act8(L) ? 1 : 0;
  if (shared_gate(L)) {  // the shared expert's per-token gate, read by the down kernels
    float* gate = reinterpret_cast<float*>(base + lay.gate);
    if ((rc = launch_rc(launch_shared_gate(x, L->shared_gate_w, T, L->H, gate, stream)))) return rc;
    p.sh_gate = gate;
  }
  if (mfma_path)
    return launch_rc(launch_ffn_mfma(p, reinterpret_cast<int32_t*>(base + lay.tiles), stream, ev));
  if (decode_path) {
    p.shared_split = 1;
    if ((rc = launch_rc(launch_gateup_decode(p, stream, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr)))) return rc;
    return launch_rc(launch_down_decode(p, stream, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr));
  }
  if (stream_path) {
    if ((rc = launch_rc(launch_gateup_stream(p, stream, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr)))) return rc;
    return launch_rc(launch_down_stream(p, stream, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr));
  }
  if ((rc = launch_rc(launch_ffn_gateup(p, stream, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr)))) return rc;
  return launch_rc(launch_ffn_down(p, stream, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr));
}

extern "C" {

int moe_expert_ffn(const moe_layer* L, const uint16_t* x, int64_t T, const int32_t* expert_off,
                   const int32_t* row2pair, float* y_rows, float* y_shared, const moe_debug* dbg, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  if (check_shape(L) != MOE_OK) return check_shape(L);
  return expert_ffn(L, x, T, expert_off, row2pair, 0, L->I / 16, y_rows, y_shared, dbg, ws, ws_bytes, stream);
}

int moe_expert_ffn_krange(const moe_layer* L, const uint16_t* x, int64_t T, const int32_t* expert_off,
                          const int32_t* row2pair, int32_t kb0, int32_t kb1, float* y_rows, float* y_shared,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  if (check_shape(L) != MOE_OK) return check_shape(L);
  return expert_ffn(L, x, T, expert_off, row2pair, kb0, kb1, y_rows, y_shared, nullptr, ws, ws_bytes, stream);
}

int moe_combine_f32(const moe_layer* L, int64_t T, const float* y_rows, const float* y_shared,
                    const int32_t* pair2row, const float* topk_w, float* out, hipStream_t stream) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!tokens_ok(L, T)) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ptr_ok(y_rows) || !ptr_ok(pair2row) || !ptr_ok(topk_w) || !ptr_ok(out)) return MOE_EINVAL;
  if (L->has_shared && !ptr_ok(y_shared)) return MOE_EINVAL;
  return launch_rc(launch_combine_f32(T, L->H, L->k, y_rows, L->has_shared ? y_shared : nullptr, pair2row, topk_w,
                                      out, stream));
}

int moe_combine(const moe_layer* L, int64_t T, const float* y_rows, const float* y_shared, const int32_t* pair2row,
                const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t stream) {
  int rc = check_shape(L);
  if (rc) return rc;
  if (!tokens_ok(L, T)) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ptr_ok(y_rows) || !ptr_ok(pair2row) || !ptr_ok(topk_w) || !ptr_ok(out) || !opt_ok(residual))
    return MOE_EINVAL;
  if (L->has_shared && !ptr_ok(y_shared)) return MOE_EINVAL;
  return launch_rc(launch_combine(T, L->H, L->k, y_rows, L->has_shared ? y_shared : nullptr, pair2row, topk_w,
                                  residual, out, stream));
}

int moe_layer_forward(const moe_layer* L, const uint16_t* x, int64_t T, const uint16_t* residual,
                      int32_t* topk_idx, float* topk_w, int32_t* expert_off, int32_t* row2pair, int32_t* pair2row,
                      float* y_rows, float* y_shared, uint16_t* out, const moe_debug* dbg, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  int rc = check_layer(L, true, true);
  if (rc) return rc;
  if (!tokens_ok(L, T)) return MOE_ESHAPE;
  if (T == 0) return MOE_OK;
  if (!ptr_ok(x) || !ptr_ok(topk_idx) || !ptr_ok(topk_w) || !ptr_ok(expert_off) || !ptr_ok(row2pair) ||
      !ptr_ok(pair2row) || !ptr_ok(y_rows) || !ptr_ok(out) || !ptr_ok(ws) || !opt_ok(residual))
    return MOE_EINVAL;
  if (L->has_shared && !ptr_ok(y_shared)) return MOE_EINVAL;
  if (!debug_ok(dbg)) return MOE_EINVAL;
  if (L->pre_norm != 0 && L->pre_norm != 1) return MOE_EINVAL;
  if (L->pre_norm && !(L->pre_norm_eps >= 0.0 && L->pre_norm_eps <= 1.0)) return MOE_EINVAL;
  // pre_norm: the normed input [T][H] BF16 at the start of the workspace, the rest after it
  uint16_t* xn = nullptr;
  if (L->pre_norm) {
    const size_t xn_bytes = align_up((size_t)T * L->H * sizeof(uint16_t));
    if (ws_bytes < xn_bytes) return MOE_EWORKSPACE;
    xn = static_cast<uint16_t*>(ws);
    ws = static_cast<char*>(ws) + xn_bytes;
    ws_bytes -= xn_bytes;
  }
  const bool dumps = dbg && (dbg->xq || dbg->xs || dbg->h || dbg->hq || dbg->hs);
  if (!fused_decode_supported(L->H, L->I, L->E, L->k, T) || dumps || L->router_mode != MOE_ROUTER_EXACT) {
    if (xn) {
      if ((rc = launch_rc(launch_rms_norm(x, T, L->H, L->pre_norm_eps, xn, stream)))) return rc;
      x = xn;
    }
    if ((rc = moe_route(L, x, T, nullptr, topk_idx, topk_w, ws, ws_bytes, stream))) return rc;
    if ((rc = moe_permute(L, topk_idx, T, expert_off, row2pair, pair2row, ws, ws_bytes, stream))) return rc;
    if ((rc = moe_expert_ffn(L, x, T, expert_off, row2pair, y_rows, y_shared, dbg, ws, ws_bytes, stream))) return rc;
    return moe_combine(L, T, y_rows, y_shared, pair2row, topk_w, residual, out, stream);
  }
  // pre_norm in the fused call: the router kernel norms x itself up to 2 tokens
  // (every router workgroup recomputes the norm of every row: at 1 token it saves
  // the norm kernel and its boundary, at 4 it costs more than it saves); from 3
  // tokens on the norm kernel runs first
  if (xn && T > 2) {
    if ((rc = launch_rc(launch_rms_norm(x, T, L->H, L->pre_norm_eps, xn, stream)))) return rc;
    x = xn;
    xn = nullptr;
  }
  const size_t lg_bytes = fused_logits_ws(L, T);
  const FfnWs lay = ffn_ws(L, T);
  if (ws_bytes < lg_bytes + lay.end) return MOE_EWORKSPACE;
  char* base = static_cast<char*>(ws);
  char* fbase = base + lg_bytes;
  hipEvent_t* ev = dbg ? dbg->events : nullptr;
  // kernel 1: FP64 logits + A4(x); the routing itself is selected inside the
  // gate/up kernel (kernel 2), whose last workgroup writes it out
  RouteDecodeParams q = {};
  q.x = x;
  q.W = L->router_w;
  q.T = (int)T;
  q.H = L->H;
  q.E = L->E;
  q.k = L->k;
  q.g_in = L->a_gscale_in;
  q.act8 = act8(L) ? 1 : 0;
  q.pre_norm = xn ? 1 : 0;  // the router kernel norms x itself and writes the normed rows to xn
  q.norm_eps = L->pre_norm_eps;
  q.xn = xn;
  q.logits = reinterpret_cast<double*>(base);
  q.slot_tab = reinterpret_cast<int4*>(base + align_up((size_t)T * L->E * sizeof(double)));
  q.xq = reinterpret_cast<uint8_t*>(fbase + lay.xq);
  q.xs = reinterpret_cast<uint8_t*>(fbase + lay.xs);
  q.idx = topk_idx;
  q.w = topk_w;
  q.off = expert_off;
  q.r2p = row2pair;
  q.p2r = pair2row;
  float* gate = nullptr;
  if (shared_gate(L)) {  // computed by the routing workgroup, read by the down kernel
    gate = reinterpret_cast<float*>(base + align_up((size_t)T * L->E * sizeof(double)) +
                                    align_up((size_t)T * L->k * sizeof(int4)) +
                                    align_up((size_t)T * L->k * L->H * sizeof(float)));
    q.wg = L->shared_gate_w;
    q.gate = gate;
  }
  if ((rc = launch_rc(launch_route_decode(q, stream, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr)))) return rc;
  if (xn) q.x = xn;  // the layer's input from here on (the publisher's shared-expert gate)
  // kernels 2, 3: gate/up (with the routing) and down over the slot table;
  // kernel 4: combine
  FfnParams p = {};
  p.H = L->H;
  p.I = L->I;
  p.E = L->E;
  p.k = L->k;
  p.T = (int)T;
  p.has_shared = L->has_shared;
  const int64_t P = T * L->k;
  const bool fused_down = down_combine_decode_supported(L->H, L->I, L->k, L->has_shared);
  p.pair_rows = fused_down ? 1 : 0;  // one routed slot per (token, rank)
  p.n_routed_slots = (int)(fused_down || P < L->E ? P : L->E);
  p.off = expert_off;
  p.row2pair = row2pair;
  p.x = x;
  p.xq = q.xq;
  p.xs = q.xs;
  p.slot_tab = q.slot_tab;
  p.w13 = L->w13;
  p.w2 = L->w2;
  p.sh13 = L->sh13;
  p.sh2 = L->sh2;
  p.w13k = L->w13k;
  p.w2k = L->w2k;
  p.sh13k = L->has_shared ? L->sh13k : moe_nvfp4_bank{};
  p.sh2k = L->has_shared ? L->sh2k : moe_nvfp4_bank{};
  p.g_in = L->a_gscale_in;
  p.g_mid = L->a_gscale_mid;
  p.act8 = q.act8;
  p.hh = reinterpret_cast<half_t*>(fbase + lay.hh);
  p.y_rows = y_rows;
  p.y_shared = L->has_shared ? y_shared : nullptr;
  p.shared_split = 1;
  p.kc0 = 0;
  p.kc1 = L->I;
  p.sh_gate = gate;
  p.rq = q;  // the gate/up workgroups select the routing from q.logits
  // the down kernel also writes the routed rows in token-major order, so the
  // combine reads them without the dependent pair2row load (same values)
  p.y_tok = reinterpret_cast<float*>(base + align_up((size_t)T * L->E * sizeof(double)) +
                                     align_up((size_t)T * L->k * sizeof(int4)));
  if ((rc = launch_rc(launch_gateup_decode(p, stream, ev ? ev[2] : nullptr, ev ? ev[3] : nullptr)))) return rc;
  if (fused_down) {
    // kernel 3 also combines: one workgroup per (token, 4 output columns)
    p.residual = residual;
    p.out = out;
    return launch_rc(launch_down_combine_decode(p, stream, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr));
  }
  if ((rc = launch_rc(launch_down_decode(p, stream, ev ? ev[4] : nullptr, ev ? ev[5] : nullptr)))) return rc;
  return launch_rc(launch_combine(T, L->H, L->k, p.y_tok, p.y_shared, nullptr, topk_w, residual, out, stream));
}

int moe_rms_norm(const uint16_t* x, int64_t T, int32_t H, double eps, uint16_t* out, hipStream_t stream) {
  if (T < 0 || H <= 0) return MOE_ESHAPE;
  if (!(eps >= 0.0) || eps > 1.0) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!ptr_ok(x) || !ptr_ok(out)) return MOE_EINVAL;
  return launch_rc(launch_rms_norm(x, T, H, eps, out, stream));
}

int moe_pack_router(const float* router_w, int32_t E, int32_t H, uint16_t* pieces_out, hipStream_t stream) {
  if (E < 1 || H < 1) return MOE_ESHAPE;
  if (!ptr_ok(router_w) || !ptr_ok(pieces_out)) return MOE_EINVAL;
  return launch_rc(launch_pack_router(router_w, E, H, pieces_out, stream));
}

int moe_pack_kmajor(const uint8_t* codes, const uint8_t* scales, int32_t n_exp, int32_t N, int32_t K,
                    uint8_t* codes_out, uint8_t* scales_out, hipStream_t stream) {
  if (n_exp < 1 || N < 1 || K < 64 || K % 64) return MOE_ESHAPE;
  if (!ptr_ok(codes) || !ptr_ok(codes_out) || !scales || !scales_out) return MOE_EINVAL;
  if (reinterpret_cast<uintptr_t>(scales) % 4 || reinterpret_cast<uintptr_t>(scales_out) % 4) return MOE_EINVAL;
  return launch_rc(launch_pack_kmajor(codes, scales, n_exp, N, K, codes_out, scales_out, stream));
}

int moe_quantize_act8(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, int8_t* codes,
                      uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 16) return MOE_ESHAPE;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32) return MOE_EINVAL;
  if (!pow2_scale(gscale)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!ptr_ok(x) || !ptr_ok(codes) || !ptr_ok(scales)) return MOE_EINVAL;
  return launch_rc(launch_quant_act(x, dtype, rows, cols, gscale, reinterpret_cast<uint8_t*>(codes), scales, nullptr,
                                    stream, nullptr, nullptr, 8));
}

int moe_quantize_act(const void* x, int dtype, int64_t rows, int32_t cols, float gscale, uint8_t* codes,
                     uint8_t* scales, hipStream_t stream) {
  if (rows < 0 || cols <= 0 || cols % 16) return MOE_ESHAPE;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_F32) return MOE_EINVAL;
  if (!pow2_scale(gscale)) return MOE_EINVAL;
  if (rows == 0) return MOE_OK;
  if (!ptr_ok(x) || !ptr_ok(codes) || !ptr_ok(scales)) return MOE_EINVAL;
  return launch_rc(launch_quant_act(x, dtype, rows, cols, gscale, codes, scales, nullptr, stream));
}

}  // extern "C"

"""FP64 CPU oracle for the routed NVFP4 W4A4 MoE layer (ctypes over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check and
by the benchmark's CPU-baseline leg, never by the product path.  It shares no
code with the HIP library.

Definitions followed (pages cited by title and section):
  * capy-flash README v0.5.4, "What it does" and "Serve": W4A4 activation
    quantization identical wherever an expert runs.
  * Richland article, "What shipped": 512 experts, 10 routed + 1 shared; E2M1
    codes, UE4M3 block scales, FP32 per-expert scale.
  * Richland article, "Why it matters": partials accumulate in FP32; BF16 vs
    FP16-with-2^-k-shift exchange payloads (the split-K check).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        i64, dbl, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        L.orc_e2m1.argtypes, L.orc_e2m1.restype = [ci], dbl
        L.orc_ue4m3.argtypes, L.orc_ue4m3.restype = [ci], dbl
        L.orc_scale_code.argtypes, L.orc_scale_code.restype = [dbl, dbl], ci
        L.orc_elem_code.argtypes, L.orc_elem_code.restype = [dbl, dbl], ci
        L.orc_quant_rows.argtypes = [vp, i64, i64, dbl, vp, vp]
        L.orc_bf16_to_f64.argtypes = [vp, i64, vp]
        L.orc_round_bf16.argtypes, L.orc_round_bf16.restype = [dbl], ctypes.c_uint16
        L.orc_round_f16_sat.argtypes, L.orc_round_f16_sat.restype = [dbl], dbl
        L.orc_router_logits.argtypes = [vp, vp, i64, i64, i64, vp]
        L.orc_topk_softmax.argtypes = [vp, i64, i64, ci, vp, vp]
        L.orc_permute.argtypes = [vp, i64, ci, i64, vp, vp, vp]
        L.orc_expert_rows.argtypes = [i64, vp, vp, vp, vp, dbl, vp, vp, vp, vp, vp, vp, i64, i64, dbl, i64, i64,
                                      vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_combine.argtypes = [i64, ci, i64, vp, vp, vp, vp, vp, vp]
        L.orc_rms_norm.argtypes = [vp, i64, i64, dbl, vp]
        L.orc_shared_gate.argtypes = [vp, vp, i64, i64, vp]
        L.orc_scale_code8.argtypes, L.orc_scale_code8.restype = [dbl, dbl], ci
        L.orc_int8_code.argtypes, L.orc_int8_code.restype = [dbl, dbl], ci
        L.orc_quant8_rows.argtypes = [vp, i64, i64, dbl, vp, vp]
        L.orc_expert_rows_a8.argtypes = [i64, vp, vp, vp, vp, dbl, vp, vp, vp, vp, vp, vp, i64, i64, dbl, i64, i64,
                                         vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_round_bf16_array.argtypes = [vp, i64, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# ---------------------------------------------------------------- formats
def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def ue4m3(code: int) -> float:
    return lib().orc_ue4m3(code)


def scale_code(amax: float, g: float = 1.0) -> int:
    return lib().orc_scale_code(amax, g)


def elem_code(v: float, s: float) -> int:
    return lib().orc_elem_code(v, s)


def quantize(v: np.ndarray, g: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """A4 encoding of a [rows][cols] FP64 matrix -> (codes [rows][cols/2], scales [rows][cols/16])."""
    v = _c(v, np.float64)
    rows, cols = v.shape
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    lib().orc_quant_rows(_p(v), rows, cols, g, _p(codes), _p(scales))
    return codes, scales


def scale_code8(amax: float, g: float = 1.0) -> int:
    """A8 block scale code: RNE of amax / (127 g) on the UE4M3 grid."""
    return lib().orc_scale_code8(amax, g)


def int8_code(v: float, s: float) -> int:
    """A8 element code: RNE(|v| / s) on 0..127 with the sign of v."""
    return lib().orc_int8_code(v, s)


def quantize8(v: np.ndarray, g: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """A8 encoding of a [rows][cols] FP64 matrix -> (int8 codes [rows][cols], scales [rows][cols/16])."""
    v = _c(v, np.float64)
    rows, cols = v.shape
    codes = np.empty((rows, cols), np.int8)
    scales = np.empty((rows, cols // 16), np.uint8)
    lib().orc_quant8_rows(_p(v), rows, cols, g, _p(codes), _p(scales))
    return codes, scales


def encode(v: np.ndarray, g: float = 1.0, act_bits: int = 4):
    """The activation encoding of a layer: A4 (act_bits 4) or A8 (8)."""
    return quantize8(v, g) if act_bits == 8 else quantize(v, g)


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    out = np.empty(x.shape, np.float64)
    lib().orc_bf16_to_f64(_p(x), x.size, _p(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest BF16 (ties to even) of FP64 values, as bit patterns."""
    a = _c(v, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().orc_round_bf16_array(_p(a), a.size, _p(out))
    return out


def round_f16_sat(v: float) -> float:
    return lib().orc_round_f16_sat(v)


# ---------------------------------------------------------------- router, permute
def router_logits(x_bf16: np.ndarray, wr: np.ndarray) -> np.ndarray:
    x_bf16, wr = _c(x_bf16, np.uint16), _c(wr, np.float32)
    T, H = x_bf16.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float64)
    lib().orc_router_logits(_p(x_bf16), _p(wr), T, H, E, _p(out))
    return out


def topk_softmax(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    logits = _c(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_topk_softmax(_p(logits), T, E, k, _p(idx), _p(w))
    return idx, w


def permute(idx: np.ndarray, E: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    idx = _c(idx, np.int32)
    T, k = idx.shape
    off = np.empty(E + 1, np.int32)
    r2p = np.empty(T * k, np.int32)
    p2r = np.empty(T * k, np.int32)
    lib().orc_permute(_p(idx), T, k, E, _p(off), _p(r2p), _p(p2r))
    return off, r2p, p2r


def shared_gate(x_bf16: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """Per-token gate of the shared expert (a reading; the pages print none):
    fl32(sigmoid(x_t . wg)), the dot in FP64 over exact products -> [T] FP32."""
    x_bf16, wg = _c(x_bf16, np.uint16), _c(wg, np.float32)
    T, H = x_bf16.shape
    g = np.empty(T, np.float32)
    lib().orc_shared_gate(_p(x_bf16), _p(wg), T, H, _p(g))
    return g


# ---------------------------------------------------------------- experts, combine
def expert_rows(a_row, a_exp, xq, xs, bank13, bank2, H, I, g_in=1.0, g_mid=1.0, kb=None, hq_in=None, hs_in=None,
                want_gu=False, act_bits=4):
    """Expert FFN for rows (token a_row[r], expert a_exp[r] of the banks).

    Returns dict with y [n][H] (FP64), h [n][I] (FP32), hq, hs, and optionally g, u.
    kb = (b0, b1) restricts the down projection to I-blocks [b0, b1).  act_bits 8:
    the W4A8 variant (xq int8 [T][H] from quantize8; hq int8 [n][I]).
    """
    a8 = act_bits == 8
    cdt = np.int8 if a8 else np.uint8
    cw = I if a8 else I // 2
    a_row, a_exp = _c(a_row, np.int32), _c(a_exp, np.int32)
    n = a_row.shape[0]
    xq, xs = _c(xq, cdt), _c(xs, np.uint8)
    q13, s13, g13 = _c(bank13["codes"], np.uint8), _c(bank13["scales"], np.uint8), _c(bank13["gscale"], np.float32)
    q2, s2, g2 = _c(bank2["codes"], np.uint8), _c(bank2["scales"], np.uint8), _c(bank2["gscale"], np.float32)
    b0, b1 = kb if kb is not None else (0, I // 16)
    hq_in = None if hq_in is None else _c(hq_in, cdt)
    hs_in = None if hs_in is None else _c(hs_in, np.uint8)
    g = np.empty((n, I), np.float64) if want_gu else None
    u = np.empty((n, I), np.float64) if want_gu else None
    h = np.empty((n, I), np.float32)
    hq = np.empty((n, cw), cdt)
    hs = np.empty((n, I // 16), np.uint8)
    y = np.empty((n, H), np.float64)
    if n:
        f = lib().orc_expert_rows_a8 if a8 else lib().orc_expert_rows
        f(n, _p(a_row), _p(a_exp), _p(xq), _p(xs), g_in, _p(q13), _p(s13), _p(g13), _p(q2), _p(s2), _p(g2), H, I,
          g_mid, b0, b1, _p(hq_in), _p(hs_in), _p(g), _p(u), _p(h), _p(hq), _p(hs), _p(y))
    out = {"y": y, "h": h, "hq": hq, "hs": hs}
    if want_gu:
        out["g"], out["u"] = g, u
    return out


def combine(y, w, ysh=None, residual=None):
    """y [n][k][H] FP64, w [n][k] FP32, ysh [n][H] FP64, residual [n][H] BF16 -> (out_f64, out_bf16)."""
    y = _c(y, np.float64)
    n, k, H = y.shape
    w = _c(w, np.float32)
    ysh = None if ysh is None else _c(ysh, np.float64)
    residual = None if residual is None else _c(residual, np.uint16)
    o64 = np.empty((n, H), np.float64)
    o16 = np.empty((n, H), np.uint16)
    lib().orc_combine(n, k, H, _p(y), _p(w), _p(ysh), _p(residual), _p(o64), _p(o16))
    return o64, o16


def rms_norm(x_bf16, eps=1e-6):
    """Parameter-free RMS norm of BF16 rows, rounded to BF16 (the stack's
    composition between MoE layers)."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    out = np.empty_like(x)
    lib().orc_rms_norm(_p(x), T, H, float(eps), _p(out))
    return out


# ---------------------------------------------------------------- whole layer
def layer(L, x_bf16, tokens=None, residual=None, kb=None, want_gu=False):
    """Reference forward of one MoE layer on the tokens listed (default: all).

    L: gen.Layer-like object (router_w, w13, w2, sh13, sh2, shape, a_gscale_in/mid,
    optional shared_gate_w and act_bits); sh13 None: a layer without the shared expert;
    act_bits 8: the W4A8 variant (A8 encodings of x and h);
    shared_gate_w [H] FP32 (absent or None: no gate): the shared expert's rows
    scaled per token by shared_gate().
    residual: [T][H] BF16 added before the rounding.  kb = (b0, b1): the down projections over I-blocks [b0, b1) only.
    Returns a dict of every intermediate.
    """
    sh = L.shape
    x_bf16 = _c(x_bf16, np.uint16)
    T = x_bf16.shape[0]
    tok = np.arange(T, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    res = {}
    lg = router_logits(x_bf16[tok], L.router_w)
    idx_t, w_s = topk_softmax(lg, sh.k)
    w_t = w_s.astype(np.float32)  # the combine takes the FP32 router weights
    res["logits"] = lg
    res["idx"], res["w"] = idx_t, w_t
    bits = getattr(L, "act_bits", 4)
    xf = bf16_to_f64(x_bf16[tok])
    xq, xs = encode(xf, L.a_gscale_in, bits)
    res["xq"], res["xs"] = xq, xs
    n = tok.shape[0]
    a_row = np.repeat(np.arange(n, dtype=np.int32), sh.k)
    a_exp = idx_t.reshape(-1).astype(np.int32)
    r = expert_rows(a_row, a_exp, xq, xs, L.w13, L.w2, sh.H, sh.I, L.a_gscale_in, L.a_gscale_mid, kb,
                    want_gu=want_gu, act_bits=bits)
    s = None
    if L.sh13 is not None:  # the shared expert runs on every token (weight 1)
        s = expert_rows(np.arange(n, dtype=np.int32), np.zeros(n, np.int32), xq, xs, L.sh13, L.sh2, sh.H, sh.I,
                        L.a_gscale_in, L.a_gscale_mid, kb, want_gu=want_gu, act_bits=bits)
    ysh = None if s is None else s["y"]
    wg = getattr(L, "shared_gate_w", None)
    if s is not None and wg is not None:  # optional gate: the shared row scaled by its FP32 gate value
        gate = shared_gate(x_bf16[tok], wg)
        res["shared_gate"] = gate
        ysh = ysh * gate.astype(np.float64)[:, None]
    res["routed"], res["shared"], res["y_shared"] = r, s, ysh
    resid = None if residual is None else _c(residual, np.uint16)[tok]
    o64, o16 = combine(r["y"].reshape(n, sh.k, sh.H), w_t, ysh, resid)
    res["out_f64"], res["out_bf16"] = o64, o16
    res["tokens"] = tok
    return res

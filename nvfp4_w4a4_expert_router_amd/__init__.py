"""Routed NVFP4 W4A4 mixture-of-experts layer for AMD MI355X (gfx950).

Thin ctypes binding over ``libnvfp4moe.so`` (the C ABI in include/moe_nvfp4.h).
Argument marshalling only: every step of the layer runs in the library's HIP
kernels; PyTorch supplies device memory and the stream.  There is no CPU
fallback: importing this package without the built library raises.

Steps (same names as the C ABI): ``moe_route`` -> ``moe_permute`` ->
``moe_expert_ffn`` -> ``moe_combine``; ``moe_quantize_act`` exposes the A4
activation encoding alone.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4moe.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EWORKSPACE, MOE_ELAUNCH = 0, -1, -2, -3, -4
MOE_DTYPE_BF16, MOE_DTYPE_F32 = 0, 1


class MoEError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s: %s (%d)" % (where, strerror(code), code))
        self.code = code


class Bank(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("gscale", ctypes.c_void_p)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("has_shared", ctypes.c_int32), ("router_w", ctypes.c_void_p), ("w13", Bank), ("w2", Bank),
                ("sh13", Bank), ("sh2", Bank), ("a_gscale_in", ctypes.c_float), ("a_gscale_mid", ctypes.c_float),
                ("w13k", Bank), ("w2k", Bank), ("sh13k", Bank), ("sh2k", Bank), ("shared_gate_w", ctypes.c_void_p),
                ("router_pieces", ctypes.c_void_p), ("router_mode", ctypes.c_int32), ("act_bits", ctypes.c_int32),
                ("pre_norm", ctypes.c_int32), ("pre_norm_eps", ctypes.c_double)]


MOE_ROUTER_EXACT, MOE_ROUTER_SPLIT3_F32, MOE_ROUTER_BF16 = 0, 1, 2


FFN_KERNELS = 3  # A4(x), gate/up + SwiGLU + A4(h), down


class Debug(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("xs", ctypes.c_void_p), ("h", ctypes.c_void_p), ("hq", ctypes.c_void_p),
                ("hs", ctypes.c_void_p), ("events", ctypes.POINTER(ctypes.c_void_p))]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnvfp4moe.so is not built (run __graft_entry__.build() or "
                          "python nvfp4_w4a4_expert_router_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
    pl = ctypes.POINTER(LayerDesc)
    L.moe_abi_version.restype = ci
    L.moe_strerror.argtypes, L.moe_strerror.restype = [ci], ctypes.c_char_p
    L.moe_workspace_bytes.argtypes, L.moe_workspace_bytes.restype = [pl, i64], sz
    L.moe_route.argtypes = [pl, vp, i64, vp, vp, vp, vp, sz, vp]
    L.moe_permute.argtypes = [pl, vp, i64, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn.argtypes = [pl, vp, i64, vp, vp, vp, vp, ctypes.POINTER(Debug), vp, sz, vp]
    L.moe_combine.argtypes = [pl, i64, vp, vp, vp, vp, vp, vp, vp]
    L.moe_quantize_act.argtypes = [vp, ci, i64, ctypes.c_int32, ctypes.c_float, vp, vp, vp]
    L.moe_quantize_act8.argtypes = [vp, ci, i64, ctypes.c_int32, ctypes.c_float, vp, vp, vp]
    L.moe_layer_forward.argtypes = [pl, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Debug), vp, sz,
                                    vp]
    L.moe_rms_norm.argtypes = [vp, i64, ctypes.c_int32, ctypes.c_double, vp, vp]
    L.moe_expert_ffn_krange.argtypes = [pl, vp, i64, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, sz, vp]
    L.moe_combine_f32.argtypes = [pl, i64, vp, vp, vp, vp, vp, vp]
    L.moe_noalloc_scratch_bytes.restype = sz
    L.moe_layer_forward_noalloc.argtypes = [pl, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.POINTER(Debug),
                                            vp]
    i32 = ctypes.c_int32
    L.moe_pack_router.argtypes = [vp, i32, i32, vp, vp]
    L.moe_pack_kmajor.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp]
    for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_quantize_act", "moe_layer_forward",
              "moe_rms_norm", "moe_expert_ffn_krange", "moe_combine_f32", "moe_pack_kmajor",
              "moe_layer_forward_noalloc", "moe_pack_router", "moe_quantize_act8"):
        getattr(L, f).restype = ci
    return L


lib = _load()
EXPORTS = ("moe_abi_version", "moe_strerror", "moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_ffn",
           "moe_combine", "moe_quantize_act", "moe_layer_forward", "moe_rms_norm", "moe_expert_ffn_krange",
           "moe_combine_f32", "moe_pack_kmajor", "moe_noalloc_scratch_bytes", "moe_layer_forward_noalloc",
           "moe_pack_router", "moe_quantize_act8")


def strerror(code: int) -> str:
    return lib.moe_strerror(code).decode()


def _check(rc: int, where: str):
    if rc != MOE_OK:
        raise MoEError(rc, where)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class MoELayer:
    """Device-resident layer parameters plus the C descriptor that points at them.

    router_w [E][H] float32; banks are dicts of uint8 codes / uint8 scales / float32
    gscale tensors in the layouts of include/moe_nvfp4.h; shared_gate_w [H] float32
    (optional gate of the shared expert); router_mode MOE_ROUTER_*; act_bits 4 (W4A4)
    or 8 (the W4A8 variant).
    Tensors are kept alive here.  pack_kmajor() adds the K-step-major copies that the
    matrix-core kernels read, pack_router() the router's BF16 pieces.
    """

    def __init__(self, H, I, E, k, router_w, w13, w2, sh13=None, sh2=None, a_gscale_in=1.0, a_gscale_mid=1.0,
                 shared_gate_w=None, router_mode=MOE_ROUTER_EXACT, act_bits=4):
        self.H, self.I, self.E, self.k = H, I, E, k
        self.has_shared = int(sh13 is not None)
        self.router_w, self.w13, self.w2, self.sh13, self.sh2 = router_w, w13, w2, sh13, sh2
        self.shared_gate_w = shared_gate_w

        def bank(b):
            return Bank() if b is None else Bank(_ptr(b["codes"]), _ptr(b["scales"]), _ptr(b["gscale"]))

        self.desc = LayerDesc(H, I, E, k, self.has_shared, _ptr(router_w), bank(w13), bank(w2), bank(sh13), bank(sh2),
                              a_gscale_in, a_gscale_mid)
        self.desc.shared_gate_w = _ptr(shared_gate_w)
        self.desc.router_mode = router_mode
        self.desc.act_bits = act_bits
        self.a_gscale_in, self.a_gscale_mid = a_gscale_in, a_gscale_mid
        self.router_mode, self.act_bits = router_mode, act_bits

    def pack_router(self, stream=None):
        """Write the router's three BF16 pieces once (moe_pack_router) and name them in
        the descriptor; returns self."""
        self.router_pieces = torch.empty((3, self.E, self.H), dtype=torch.int16, device=self.router_w.device)
        _check(lib.moe_pack_router(_ptr(self.router_w), self.E, self.H, _ptr(self.router_pieces), _stream(stream)),
               "moe_pack_router")
        self.desc.router_pieces = _ptr(self.router_pieces)
        return self

    def with_router_mode(self, mode):
        """The same layer (same device tensors) with another router precision mode."""
        other = MoELayer.__new__(MoELayer)
        other.__dict__.update(self.__dict__)
        other.desc = LayerDesc.from_buffer_copy(self.desc)
        other.desc.router_mode = mode
        other.router_mode = mode
        return other

    def with_act_bits(self, bits):
        """The same layer (same device tensors) with another activation encoding (4 or 8)."""
        other = self.with_router_mode(self.router_mode)
        other.desc.act_bits = bits
        other.act_bits = bits
        return other

    def with_pre_norm(self, eps=1e-6):
        """The same layer whose moe_layer_forward takes RMSNorm(x) (moe_rms_norm with eps)
        as its input: the stack's norm and layer in one call."""
        other = self.with_router_mode(self.router_mode)
        other.desc.pre_norm = 1
        other.desc.pre_norm_eps = float(eps)
        return other

    def with_shared_gate(self, shared_gate_w):
        """The same layer (same device tensors) with the shared expert's gate vector
        shared_gate_w ([H] float32 on the device; None: no gate)."""
        other = self.with_router_mode(self.router_mode)
        other.shared_gate_w = shared_gate_w
        other.desc.shared_gate_w = _ptr(shared_gate_w)
        return other

    def pack_kmajor(self, stream=None):
        """Write K-step-major copies of every bank (moe_pack_kmajor) and name them in
        the descriptor; returns self.  Needs H and I to be multiples of 64."""
        banks = [("w13k", self.w13, self.E, 2 * self.I, self.H), ("w2k", self.w2, self.E, self.H, self.I)]
        if self.has_shared:
            banks += [("sh13k", self.sh13, 1, 2 * self.I, self.H), ("sh2k", self.sh2, 1, self.H, self.I)]
        self.kmajor = {}
        for name, b, n_exp, N, K in banks:
            c, s = torch.empty_like(b["codes"]), torch.empty_like(b["scales"])
            moe_pack_kmajor(b["codes"], b["scales"], n_exp, N, K, c, s, stream=stream)
            self.kmajor[name] = (c, s)
            setattr(self.desc, name, Bank(_ptr(c), _ptr(s), None))
        return self

    def workspace_bytes(self, T_max: int) -> int:
        return int(lib.moe_workspace_bytes(ctypes.byref(self.desc), T_max))

    def workspace(self, T_max: int, device=None) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(T_max), dtype=torch.uint8, device=device or self.router_w.device)


def moe_route(layer: MoELayer, x, topk_idx, topk_w, ws, logits_in=None, T=None, stream=None):
    T = x.shape[0] if T is None else T
    _check(lib.moe_route(ctypes.byref(layer.desc), _ptr(x), T, _ptr(logits_in), _ptr(topk_idx), _ptr(topk_w),
                         _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "moe_route")


def moe_permute(layer: MoELayer, topk_idx, expert_off, row2pair, pair2row, ws, T=None, stream=None):
    T = topk_idx.shape[0] if T is None else T
    _check(lib.moe_permute(ctypes.byref(layer.desc), _ptr(topk_idx), T, _ptr(expert_off), _ptr(row2pair),
                           _ptr(pair2row), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "moe_permute")


def _debug(debug):
    """moe_debug from a dict of optional device tensors and/or 2 * FFN_KERNELS recorded events."""
    if debug is None:
        return None
    evs = debug.get("events")  # sequence of 2 * FFN_KERNELS recorded torch.cuda.Event
    ev_arr = None
    if evs is not None:
        if len(evs) != 2 * FFN_KERNELS:
            raise ValueError("debug['events'] takes %d events" % (2 * FFN_KERNELS))
        handles = [e.cuda_event for e in evs]
        if not all(handles):
            raise ValueError("record every event once (event.record()) before passing it: "
                             "torch creates the HIP event on first use")
        ev_arr = (ctypes.c_void_p * len(evs))(*handles)
    dbg = Debug(_ptr(debug.get("xq")), _ptr(debug.get("xs")), _ptr(debug.get("h")), _ptr(debug.get("hq")),
                _ptr(debug.get("hs")), ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p)) if evs else None)
    dbg._keep = ev_arr
    return dbg


def moe_expert_ffn(layer: MoELayer, x, expert_off, row2pair, y_rows, y_shared, ws, debug=None, T=None,
                   stream=None):
    T = x.shape[0] if T is None else T
    dbg = _debug(debug)
    _check(lib.moe_expert_ffn(ctypes.byref(layer.desc), _ptr(x), T, _ptr(expert_off), _ptr(row2pair), _ptr(y_rows),
                              _ptr(y_shared), None if dbg is None else ctypes.byref(dbg), _ptr(ws),
                              0 if ws is None else ws.numel(), _stream(stream)), "moe_expert_ffn")


def moe_combine(layer: MoELayer, y_rows, y_shared, pair2row, topk_w, out, residual=None, T=None, stream=None):
    T = out.shape[0] if T is None else T
    _check(lib.moe_combine(ctypes.byref(layer.desc), T, _ptr(y_rows), _ptr(y_shared), _ptr(pair2row), _ptr(topk_w),
                           _ptr(residual), _ptr(out), _stream(stream)), "moe_combine")


def moe_pack_kmajor(codes, scales, n_exp, N, K, codes_out, scales_out, stream=None):
    """K-step-major copy of one NVFP4 bank (include/moe_nvfp4.h)."""
    _check(lib.moe_pack_kmajor(_ptr(codes), _ptr(scales), n_exp, N, K, _ptr(codes_out), _ptr(scales_out),
                               _stream(stream)), "moe_pack_kmajor")


def moe_quantize_act(x, codes, scales, gscale=1.0, stream=None):
    dtype = {torch.bfloat16: MOE_DTYPE_BF16, torch.int16: MOE_DTYPE_BF16, torch.uint16: MOE_DTYPE_BF16,
             torch.float32: MOE_DTYPE_F32}[x.dtype]
    rows, cols = x.shape
    _check(lib.moe_quantize_act(_ptr(x), dtype, rows, cols, gscale, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_act")


def moe_quantize_act8(x, codes, scales, gscale=1.0, stream=None):
    """A8 encoding (the W4A8 variant's): codes int8 [rows][cols], scales [rows][cols/16]."""
    dtype = {torch.bfloat16: MOE_DTYPE_BF16, torch.int16: MOE_DTYPE_BF16, torch.uint16: MOE_DTYPE_BF16,
             torch.float32: MOE_DTYPE_F32}[x.dtype]
    rows, cols = x.shape
    _check(lib.moe_quantize_act8(_ptr(x), dtype, rows, cols, gscale, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_act8")


def moe_expert_ffn_krange(layer: MoELayer, x, expert_off, row2pair, kb0, kb1, y_rows, y_shared, ws, T=None,
                          stream=None):
    """moe_expert_ffn with the down projection over the I-blocks [kb0, kb1) only."""
    T = x.shape[0] if T is None else T
    _check(lib.moe_expert_ffn_krange(ctypes.byref(layer.desc), _ptr(x), T, _ptr(expert_off), _ptr(row2pair), kb0,
                                     kb1, _ptr(y_rows), _ptr(y_shared), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_expert_ffn_krange")


def moe_combine_f32(layer: MoELayer, y_rows, y_shared, pair2row, topk_w, out, T=None, stream=None):
    """FP32 combine without residual or rounding: out [T][H] float32."""
    T = out.shape[0] if T is None else T
    _check(lib.moe_combine_f32(ctypes.byref(layer.desc), T, _ptr(y_rows), _ptr(y_shared), _ptr(pair2row),
                               _ptr(topk_w), _ptr(out), _stream(stream)), "moe_combine_f32")


def moe_rms_norm(x, out, eps=1e-6, stream=None):
    """out = RNE_BF16(x / sqrt(mean(x^2) + eps)) row by row ([T][H] BF16 as int16)."""
    T, H = x.shape
    _check(lib.moe_rms_norm(_ptr(x), T, H, float(eps), _ptr(out), _stream(stream)), "moe_rms_norm")


class Buffers:
    """Outputs and workspace of one layer call for up to T tokens (device tensors)."""

    def __init__(self, layer: MoELayer, T: int, device):
        k, H = layer.k, layer.H
        self.T = T
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.expert_off = torch.empty(layer.E + 1, dtype=torch.int32, device=device)
        self.row2pair = torch.empty(T * k, dtype=torch.int32, device=device)
        self.pair2row = torch.empty(T * k, dtype=torch.int32, device=device)
        self.y_rows = torch.empty((T * k, H), dtype=torch.float32, device=device)
        self.y_shared = torch.empty((T, H), dtype=torch.float32, device=device) if layer.has_shared else None
        self.out = torch.empty((T, H), dtype=torch.int16, device=device)
        self.ws = layer.workspace(T, device)


def moe_layer_forward(layer: MoELayer, x, buf: Buffers, residual=None, T=None, debug=None, topk=None,
                      stream=None):
    """The whole layer in one library call (fused kernels for decode batches); returns buf.out.

    topk: optional (topk_idx, topk_w) tensors to write the routing into instead of buf's."""
    T = x.shape[0] if T is None else T
    idx, w = (buf.topk_idx, buf.topk_w) if topk is None else topk
    dbg = _debug(debug)
    _check(lib.moe_layer_forward(ctypes.byref(layer.desc), _ptr(x), T, _ptr(residual), _ptr(idx), _ptr(w),
                                 _ptr(buf.expert_off), _ptr(buf.row2pair), _ptr(buf.pair2row), _ptr(buf.y_rows),
                                 _ptr(buf.y_shared), _ptr(buf.out), None if dbg is None else ctypes.byref(dbg),
                                 _ptr(buf.ws), buf.ws.numel(), _stream(stream)), "moe_layer_forward")
    return buf.out


def moe_layer_forward_noalloc(layer: MoELayer, x, buf: Buffers, residual=None, T=None, debug=None, topk=None,
                              stream=None):
    """moe_layer_forward with the library's own device scratch array as workspace
    (buf.ws is not used; nothing is allocated); returns buf.out."""
    T = x.shape[0] if T is None else T
    idx, w = (buf.topk_idx, buf.topk_w) if topk is None else topk
    dbg = _debug(debug)
    _check(lib.moe_layer_forward_noalloc(ctypes.byref(layer.desc), _ptr(x), T, _ptr(residual), _ptr(idx), _ptr(w),
                                         _ptr(buf.expert_off), _ptr(buf.row2pair), _ptr(buf.pair2row),
                                         _ptr(buf.y_rows), _ptr(buf.y_shared), _ptr(buf.out),
                                         None if dbg is None else ctypes.byref(dbg), _stream(stream)),
           "moe_layer_forward_noalloc")
    return buf.out


def moe_forward(layer: MoELayer, x, buf: Buffers, residual=None, debug=None, stream=None):
    """route -> permute -> expert FFN -> combine on one stream; returns buf.out (BF16 bits as int16)."""
    T = x.shape[0]
    moe_route(layer, x, buf.topk_idx, buf.topk_w, buf.ws, T=T, stream=stream)
    moe_permute(layer, buf.topk_idx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=T, stream=stream)
    moe_expert_ffn(layer, x, buf.expert_off, buf.row2pair, buf.y_rows, buf.y_shared, buf.ws, debug=debug, T=T,
                   stream=stream)
    moe_combine(layer, buf.y_rows, buf.y_shared, buf.pair2row, buf.topk_w, buf.out, residual=residual, T=T,
                stream=stream)
    return buf.out

"""Helpers for the GPU parity tests: upload a generated layer, run the HIP path
through the C ABI, and check every step against the oracle (teacher-forced
where the checker accepts a near-tie or near-threshold difference)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import checker
import oracle
import nvfp4_w4a4_expert_router_amd as moe

DEV = "cuda:0"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bank_to_dev(b):
    if b is None:  # no shared expert
        return None
    return {"codes": to_dev(b["codes"]), "scales": to_dev(b["scales"]), "gscale": to_dev(b["gscale"])}


def device_layer(L, router_w=None, kmajor=True) -> moe.MoELayer:
    """The layer on the device; kmajor: also the K-step-major weight copies that the
    matrix-core kernels read (the product configuration)."""
    sh = L.shape
    rw = L.router_w if router_w is None else router_w
    wg = getattr(L, "shared_gate_w", None)
    DL = moe.MoELayer(sh.H, sh.I, sh.E, sh.k, to_dev(rw), bank_to_dev(L.w13), bank_to_dev(L.w2),
                      bank_to_dev(L.sh13), bank_to_dev(L.sh2), L.a_gscale_in, L.a_gscale_mid,
                      shared_gate_w=None if wg is None else to_dev(wg), act_bits=getattr(L, "act_bits", 4))
    if kmajor and sh.H % 64 == 0 and sh.I % 64 == 0:
        DL.pack_kmajor()
    return DL


def run_layer(DL: moe.MoELayer, x: np.ndarray, residual=None, dump=("xq", "xs", "hq", "hs"), logits_in=None):
    """Run route -> permute -> ffn -> combine; returns numpy copies of every output and dump."""
    T = x.shape[0]
    H, I, k = DL.H, DL.I, DL.k
    R = T * k + (T if DL.has_shared else 0)
    a8 = DL.act_bits == 8  # one code byte per element
    xd = to_dev(x.view(np.int16))
    buf = moe.Buffers(DL, T, DEV)
    dbg = {}
    if "xq" in dump:
        dbg["xq"] = torch.empty((T, H if a8 else H // 2), dtype=torch.uint8, device=DEV)
    if "xs" in dump:
        dbg["xs"] = torch.empty((T, H // 16), dtype=torch.uint8, device=DEV)
    if "h" in dump:
        dbg["h"] = torch.empty((R, I), dtype=torch.float32, device=DEV)
    if "hq" in dump:
        dbg["hq"] = torch.empty((R, I if a8 else I // 2), dtype=torch.uint8, device=DEV)
    if "hs" in dump:
        dbg["hs"] = torch.empty((R, I // 16), dtype=torch.uint8, device=DEV)
    res = None if residual is None else to_dev(residual.view(np.int16))
    lg = None if logits_in is None else to_dev(logits_in.astype(np.float32))
    moe.moe_route(DL, xd, buf.topk_idx, buf.topk_w, buf.ws, logits_in=lg, T=T)
    moe.moe_permute(DL, buf.topk_idx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=T)
    moe.moe_expert_ffn(DL, xd, buf.expert_off, buf.row2pair, buf.y_rows, buf.y_shared, buf.ws, debug=dbg, T=T)
    moe.moe_combine(DL, buf.y_rows, buf.y_shared, buf.pair2row, buf.topk_w, buf.out, residual=res, T=T)
    # the FP32 sum before the rounding (without the residual, which the checker adds in FP32)
    out32 = torch.empty((T, H), dtype=torch.float32, device=DEV)
    moe.moe_combine_f32(DL, buf.y_rows, buf.y_shared, buf.pair2row, buf.topk_w, out32, T=T)
    torch.cuda.synchronize()
    out = {"idx": buf.topk_idx.cpu().numpy(), "w": buf.topk_w.cpu().numpy(), "off": buf.expert_off.cpu().numpy(),
           "r2p": buf.row2pair.cpu().numpy(), "p2r": buf.pair2row.cpu().numpy(),
           "y_rows": buf.y_rows.cpu().numpy(), "out": buf.out.cpu().numpy().view(np.uint16),
           "out_f32": out32.cpu().numpy()}
    if buf.y_shared is not None:
        out["y_shared"] = buf.y_shared.cpu().numpy()
    for key, t in dbg.items():
        out[key] = t.cpu().numpy()
        if a8 and key in ("xq", "hq"):
            out[key] = out[key].view(np.int8)
    return out


def check_layer(L, x, g, tokens=None, residual=None, logits64=None, rep=None):
    """Check GPU results g (from run_layer) against the oracle on `tokens` (default all)."""
    rep = checker.Report() if rep is None else rep
    sh = L.shape
    T = x.shape[0]
    t0 = time.time()
    if logits64 is None:
        logits64 = oracle.router_logits(x, L.router_w)
    idx_ad, w_ad = checker.check_topk(g["idx"], g["w"], logits64, sh.k, rep)
    checker.check_permutation(idx_ad, sh.E, g["off"], g["r2p"], g["p2r"])
    bits = getattr(L, "act_bits", 4)
    xq_o, xs_o = oracle.encode(oracle.bf16_to_f64(x), L.a_gscale_in, bits)
    assert np.array_equal(g["xq"], xq_o), "A%d(x) codes differ" % bits
    assert np.array_equal(g["xs"], xs_o), "A%d(x) scales differ" % bits
    hcheck = checker.check_h_codes8 if bits == 8 else checker.check_h_codes
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, dtype=np.int32)
    n = tok.shape[0]
    a_row = np.repeat(tok, sh.k).astype(np.int32)
    a_exp = idx_ad[tok].reshape(-1).astype(np.int32)
    rows = g["p2r"][(tok[:, None] * sh.k + np.arange(sh.k)[None, :]).reshape(-1)]
    srows = T * sh.k + tok
    r_o = oracle.expert_rows(a_row, a_exp, xq_o, xs_o, L.w13, L.w2, sh.H, sh.I, L.a_gscale_in, L.a_gscale_mid,
                             act_bits=bits)
    shared = L.sh13 is not None
    if shared:
        s_o = oracle.expert_rows(tok, np.zeros(n, np.int32), xq_o, xs_o, L.sh13, L.sh2, sh.H, sh.I, L.a_gscale_in,
                                 L.a_gscale_mid, act_bits=bits)
    hq_r, hs_r = hcheck(r_o["h"], r_o["hq"], r_o["hs"], g["hq"][rows], g["hs"][rows], L.a_gscale_mid, rep, "h")
    if shared:
        hq_s, hs_s = hcheck(s_o["h"], s_o["hq"], s_o["hs"], g["hq"][srows], g["hs"][srows], L.a_gscale_mid, rep,
                            "hsh")
    if "h" in g:
        hr = g["h"][rows].astype(np.float64)
        d = np.abs(hr - r_o["h"]) / (np.abs(r_o["h"]).max() + 1e-30)
        rep["h_fp32_maxrel"] = float(d.max()) if d.size else 0.0
    # down projection on the oracle's own h codes, accepted band decisions taken on
    # their other side (identical to the oracle's codes when nothing flipped)
    r_t = oracle.expert_rows(a_row, a_exp, xq_o, xs_o, L.w13, L.w2, sh.H, sh.I, L.a_gscale_in, L.a_gscale_mid,
                             hq_in=hq_r, hs_in=hs_r, act_bits=bits)
    y_sh = None
    if shared:
        s_t = oracle.expert_rows(tok, np.zeros(n, np.int32), xq_o, xs_o, L.sh13, L.sh2, sh.H, sh.I, L.a_gscale_in,
                                 L.a_gscale_mid, hq_in=hq_s, hs_in=hs_s, act_bits=bits)
        y_sh = s_t["y"]
        wg = getattr(L, "shared_gate_w", None)
        if wg is not None:  # the shared expert's rows times the token's gate
            y_sh = y_sh * oracle.shared_gate(x[tok], wg).astype(np.float64)[:, None]
        checker.check_fp32_rows(g["y_shared"][tok], y_sh, rep, "y_shared")
    checker.check_fp32_rows(g["y_rows"][rows], r_t["y"], rep, "y_rows")
    resid = None if residual is None else residual[tok]
    o64, o16 = oracle.combine(r_t["y"].reshape(n, sh.k, sh.H), w_ad[tok], y_sh, resid)
    v32 = None
    if "out_f32" in g:  # the kernel's FP32 sum before rounding; the residual is its last FP32 addition
        v32 = g["out_f32"][tok].astype(np.float32)
        if resid is not None:
            v32 = v32 + checker.bf16_bits_to_f64(resid).astype(np.float32)
    checker.check_output(g["out"][tok], o64, o16, rep, v32=v32)
    rep["oracle_s"] = round(time.time() - t0, 2)
    rep["checked_tokens"] = n
    return rep


def run_krange(DL: moe.MoELayer, x: np.ndarray, kb0: int, kb1: int):
    """route -> permute -> moe_expert_ffn_krange over the I-blocks [kb0, kb1) ->
    moe_combine_f32; returns numpy copies of the partial rows and output."""
    T = x.shape[0]
    xd = to_dev(x.view(np.int16))
    buf = moe.Buffers(DL, T, DEV)
    moe.moe_route(DL, xd, buf.topk_idx, buf.topk_w, buf.ws, T=T)
    moe.moe_permute(DL, buf.topk_idx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=T)
    moe.moe_expert_ffn_krange(DL, xd, buf.expert_off, buf.row2pair, kb0, kb1, buf.y_rows, buf.y_shared, buf.ws, T=T)
    o32 = torch.empty((T, DL.H), dtype=torch.float32, device=DEV)
    moe.moe_combine_f32(DL, buf.y_rows, buf.y_shared, buf.pair2row, buf.topk_w, o32, T=T)
    torch.cuda.synchronize()
    out = {"idx": buf.topk_idx.cpu().numpy(), "p2r": buf.pair2row.cpu().numpy(), "y_rows": buf.y_rows.cpu().numpy(),
           "out_f32": o32.cpu().numpy()}
    if buf.y_shared is not None:
        out["y_shared"] = buf.y_shared.cpu().numpy()
    return out


def check_krange(L, x, g, part, kb0, kb1, rep=None):
    """A K-split partial (from run_krange) against the oracle's partial over the same
    I-blocks, on the h codes the full call g (run_layer with hq/hs dumps) produced,
    accepted by the checker (identical to the oracle's when nothing flipped)."""
    rep = checker.Report() if rep is None else rep
    sh = L.shape
    T = x.shape[0]
    assert np.array_equal(part["idx"], g["idx"]) and np.array_equal(part["p2r"], g["p2r"])
    logits64 = oracle.router_logits(x, L.router_w)
    idx_ad, w_ad = checker.check_topk(g["idx"], g["w"], logits64, sh.k, rep)
    xq, xs = oracle.quantize(oracle.bf16_to_f64(x), L.a_gscale_in)
    tok = np.arange(T, dtype=np.int32)
    a_row = np.repeat(tok, sh.k).astype(np.int32)
    a_exp = idx_ad.reshape(-1).astype(np.int32)
    rows = g["p2r"]
    args = (xq, xs, L.w13, L.w2, sh.H, sh.I, L.a_gscale_in, L.a_gscale_mid)
    r_o = oracle.expert_rows(a_row, a_exp, *args)
    hq, hs = checker.check_h_codes(r_o["h"], r_o["hq"], r_o["hs"], g["hq"][rows], g["hs"][rows], L.a_gscale_mid,
                                   rep, "h")
    r_t = oracle.expert_rows(a_row, a_exp, *args, kb=(kb0, kb1), hq_in=hq, hs_in=hs)
    checker.check_fp32_rows(part["y_rows"][rows], r_t["y"], rep, "y_rows_part")
    y_sh = None
    if L.sh13 is not None:
        sargs = (xq, xs, L.sh13, L.sh2, sh.H, sh.I, L.a_gscale_in, L.a_gscale_mid)
        s_o = oracle.expert_rows(tok, np.zeros(T, np.int32), *sargs)
        srows = T * sh.k + tok
        hq_s, hs_s = checker.check_h_codes(s_o["h"], s_o["hq"], s_o["hs"], g["hq"][srows], g["hs"][srows],
                                           L.a_gscale_mid, rep, "hsh")
        y_sh = oracle.expert_rows(tok, np.zeros(T, np.int32), *sargs, kb=(kb0, kb1), hq_in=hq_s, hs_in=hs_s)["y"]
        wg = getattr(L, "shared_gate_w", None)
        if wg is not None:
            y_sh = y_sh * oracle.shared_gate(x, wg).astype(np.float64)[:, None]
        checker.check_fp32_rows(part["y_shared"], y_sh, rep, "y_shared_part")
    o64, _ = oracle.combine(r_t["y"].reshape(T, sh.k, sh.H), w_ad, y_sh)
    rms = float(np.sqrt(np.mean(o64 ** 2)))
    d = np.abs(part["out_f32"].astype(np.float64) - o64)
    rep["part_fp32_maxabs_over_rms"] = float(d.max() / rms)
    assert d.max() <= 1e-2 * rms, "partial output: max-abs %.3g > 1e-2 * RMS" % d.max()
    rel = float(np.linalg.norm(part["out_f32"] - o64) / np.linalg.norm(o64))
    rep["part_rel_l2"] = rel
    assert rel <= 2e-3
    return rep

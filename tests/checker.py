"""Comparison of the HIP path against the FP64 oracle, step by step.

Rules (where floating point may legitimately change an integer decision):
  * top-k ids are bit-exact, except where the oracle's FP64 logits of the two
    experts involved differ by less than 1e-6 (and are not exactly equal): a
    reordered sum may then pick the other one (capy-flash README v0.5.4,
    "Measured", footnote on the tensor-core router).  Exactly equal logits are
    decided by the tie rule (lower id first), with no exemption.  For an
    accepted token the oracle continues with that valid alternative selection
    (its own weights for it, from its own logits).
  * A4(x) codes and scales are bit-exact (x is BF16, both sides exact).
  * the permutation is bit-exact (recomputed by the oracle from the adopted ids).
  * A4(h) codes may differ only where the oracle's h lies within the FP32
    rounding band of a decision threshold (the GPU's h is an FP32 sum in
    another order); for the down projection the oracle then encodes its own h
    with the decision taken on the other side of that threshold.
Every expected value is computed by the oracle; a GPU result only says which of
the oracle's valid alternatives (above) to continue with.
  * the BF16 output meets rel-L2 <= 2e-3 against the oracle's BF16 output; the
    kernel's FP32 sum before its rounding is within 1e-2 * RMS of the oracle's FP64
    value with no exemption; the BF16 output is the rounding of that FP32 sum; and a
    BF16 element further than 1e-2 * RMS from the oracle's is accepted only as a
    verified one-ulp straddle of a rounding midpoint.
"""
from __future__ import annotations

import numpy as np

import oracle

NEAR_TIE = 1e-6
BAND_REL = 2.0 ** -12
E2M1_MAG = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])


def bf16_bits_to_f64(b):
    return (np.asarray(b).astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class Report(dict):
    def line(self):
        return ", ".join("%s=%s" % (k, v) for k, v in self.items())


# ---------------------------------------------------------------- routing
def check_topk(idx_g, w_g, logits64, k, rep: Report):
    """Returns (idx_adopted, w_expected) after checking the GPU's routing."""
    idx_o, w_o = oracle.topk_softmax(logits64, k)
    T, E = logits64.shape
    idx_ad = idx_o.copy()
    bad = np.where((idx_g != idx_o).any(axis=1))[0]
    n_exempt = 0
    for t in bad:
        l = logits64[t]
        sg, so = set(idx_g[t].tolist()), set(idx_o[t].tolist())
        assert len(sg) == k and all(0 <= e < E for e in sg), "token %d: invalid ids %s" % (t, idx_g[t])
        for x_ in sg - so:  # GPU picked x_, oracle picked some y instead
            for y in so - sg:
                d = l[y] - l[x_]
                assert 0 < d < NEAR_TIE, "token %d: GPU chose %d over %d, FP64 margin %.3g" % (t, x_, y, d)
        # slot order: descending within the near-tie tolerance, exact ties by id
        seq = idx_g[t]
        for j in range(k - 1):
            a, b = seq[j], seq[j + 1]
            if l[a] == l[b]:
                assert a < b, "token %d: exact tie order %d,%d" % (t, a, b)
            else:
                assert l[a] > l[b] - NEAR_TIE, "token %d: slot order %d,%d margin %.3g" % (t, a, b, l[b] - l[a])
        idx_ad[t] = seq
        n_exempt += 1
    rep["topk_exempt"] = n_exempt
    # router weights for the adopted selection, in its order
    sel = np.take_along_axis(logits64, idx_ad.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w_ad = ex / ex.sum(axis=1, keepdims=True)
    err = np.abs(w_g.astype(np.float64) - w_ad)
    tol = 1e-6 * np.maximum(w_ad, 1e-3) + 1e-7
    assert np.all(err <= tol), "router weights: worst %.3g (tol %.3g)" % (err.max(), tol[np.unravel_index(
        np.argmax(err - tol), err.shape)])
    s = w_g.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= 16 * 2.0 ** -24), "router weights do not sum to 1: %g" % np.abs(s - 1).max()
    rep["w_maxerr"] = float(err.max()) if err.size else 0.0
    return idx_ad.astype(np.int32), w_ad.astype(np.float32)


def check_topk_radius(idx_g, w_g, logits64, radius, k, rep: Report):
    """A reduced-precision router against the oracle's top k on that router's own
    FP64 logits: every difference must lie within the kernel's FP32 error radius
    (radius[t][e] bounds |l32 - l64| for each logit), since FP32 sums in another
    order may resolve a near tie either way (capy-flash README v0.5.4, "Measured",
    footnote on the tensor-core router).  The weights are the softmax of FP32
    logits, so they may move by the same radius.  Returns the number of tokens
    whose selected set differs from the oracle's on these logits."""
    idx_o, _ = oracle.topk_softmax(logits64, k)
    T, E = logits64.shape
    flips = 0
    for t in np.where((idx_g != idx_o).any(axis=1))[0]:
        l, r = logits64[t], radius[t]
        sg, so = set(idx_g[t].tolist()), set(idx_o[t].tolist())
        assert len(sg) == k and all(0 <= e < E for e in sg), "token %d: invalid ids %s" % (t, idx_g[t])
        for a in sg - so:
            for b in so - sg:
                assert l[b] - l[a] <= r[a] + r[b], "token %d: chose %d over %d, margin %.3g > radius %.3g" % (
                    t, a, b, l[b] - l[a], r[a] + r[b])
        seq = idx_g[t]
        for j in range(k - 1):
            a, b = seq[j], seq[j + 1]
            assert l[a] >= l[b] - (r[a] + r[b]), "token %d: slot order %d,%d" % (t, a, b)
        flips += sg != so
    sel = np.take_along_axis(logits64, idx_g.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w_o = ex / ex.sum(axis=1, keepdims=True)
    rmax = np.take_along_axis(radius, idx_g.astype(np.int64), axis=1).max(axis=1, keepdims=True)
    err = np.abs(w_g.astype(np.float64) - w_o)
    tol = 2.0 * w_o * (2.0 * rmax) + 1e-6 * w_o + 1e-7
    assert np.all(err <= tol), "router weights beyond the radius: worst %.3g" % (err - tol).max()
    s = w_g.astype(np.float64).sum(axis=1)
    assert np.all(np.abs(s - 1.0) <= 16 * 2.0 ** -24)
    rep["set_flips_within_radius"] = int(flips)
    return flips


def check_permutation(idx_ad, E, off_g, r2p_g, p2r_g):
    off, r2p, p2r = oracle.permute(idx_ad, E)
    assert np.array_equal(off_g, off), "expert_off differs"
    assert np.array_equal(r2p_g, r2p), "row2pair differs"
    assert np.array_equal(p2r_g, p2r), "pair2row differs"
    return off, r2p, p2r


# ---------------------------------------------------------------- A4(h)
def _unpack(codes):
    c = np.asarray(codes)
    return np.stack([c & 15, c >> 4], -1).reshape(*c.shape[:-1], -1)


def check_h_codes(h_o, hq_o, hs_o, hq_g, hs_g, g_mid, rep: Report, prefix="h"):
    """Compare GPU A4(h) codes with the oracle's; accept flips inside the rounding band.

    h_o: oracle h (FP32 values), [n][I].  Returns the oracle's codes (hq, hs) with
    every accepted decision taken on the other side of its threshold: a block scale
    moved to the neighbouring code (and the block's elements re-encoded from the
    oracle's h under it), an element code moved to the neighbouring magnitude."""
    n, I = h_o.shape
    h = h_o.astype(np.float64)
    blocks = h.reshape(n, I // 16, 16)
    amax = np.abs(blocks).max(-1)
    flips = 0
    # block scales
    sd = np.argwhere(hs_o != hs_g)
    for r, b in sd:
        a, c = int(hs_o[r, b]), int(hs_g[r, b])
        assert abs(a - c) == 1, "row %d block %d: scale codes %d vs %d" % (r, b, a, c)
        lo = min(a, c)
        thr = 6.0 * g_mid * 0.5 * (oracle.ue4m3(lo) + oracle.ue4m3(lo + 1))
        assert abs(amax[r, b] - thr) <= BAND_REL * thr, "row %d block %d: scale flip outside band" % (r, b)
        flips += 1
    # element codes, judged with the GPU's scale
    qo, qg = _unpack(hq_o), _unpack(hq_g)
    ed = np.argwhere(qo != qg)
    for r, i in ed:
        b = i // 16
        if hs_o[r, b] != hs_g[r, b]:
            continue  # whole block re-encoded with the other scale: judged below
        co, cg = int(qo[r, i]), int(qg[r, i])
        if (co & 7) == 0 and (cg & 7) == 0:
            continue  # +0 vs -0
        assert (co & 8) == (cg & 8) and abs((co & 7) - (cg & 7)) == 1, "row %d col %d: codes %d vs %d" % (r, i, co,
                                                                                                          cg)
        s = oracle.ue4m3(int(hs_g[r, b])) * g_mid
        m = min(co & 7, cg & 7)
        thr = 0.5 * (E2M1_MAG[m] + E2M1_MAG[m + 1]) * s
        assert abs(abs(h[r, i]) - thr) <= BAND_REL * thr, "row %d col %d: code flip outside band (%.9g vs %.9g)" % (
            r, i, abs(h[r, i]), thr)
        flips += 1
    # blocks whose scale flipped: every code must be the A4 code of h under the GPU's scale, within the band
    for r, b in sd:
        s = oracle.ue4m3(int(hs_g[r, b])) * g_mid
        for i in range(16):
            col = b * 16 + i
            want = oracle.elem_code(float(h[r, col]), s)
            got = int(qg[r, col])
            if want == got or ((want & 7) == 0 and (got & 7) == 0):
                continue
            m = min(want & 7, got & 7)
            thr = 0.5 * (E2M1_MAG[m] + E2M1_MAG[m + 1]) * s
            assert abs(abs(h[r, col]) - thr) <= BAND_REL * thr, "row %d col %d: code under flipped scale" % (r, col)
    rep[prefix + "_flips"] = flips
    assert flips <= max(1, 1e-4 * n * I), "%d A4(h) flips exceed 1e-4 of %d elements" % (flips, n * I)
    # the oracle's codes with the accepted decisions on their other side
    hs_ad = np.array(hs_o, copy=True)
    q_ad = qo.copy()
    for r, b in sd:
        hs_ad[r, b] = int(hs_o[r, b]) + (1 if hs_g[r, b] > hs_o[r, b] else -1)
        s = oracle.ue4m3(int(hs_ad[r, b])) * g_mid
        for i in range(16):
            col = b * 16 + i
            q_ad[r, col] = oracle.elem_code(float(h[r, col]), s)
    for r, i in np.argwhere(q_ad != qg):  # element decisions in the band (validated above)
        co = int(q_ad[r, i])
        if (co & 7) == 0 and (int(qg[r, i]) & 7) == 0:
            continue
        q_ad[r, i] = co + (1 if (int(qg[r, i]) & 7) > (co & 7) else -1)
    assert np.array_equal(q_ad & 7, qg & 7) and np.array_equal(hs_ad, hs_g)
    hq_ad = (q_ad[..., 0::2] | (q_ad[..., 1::2] << 4)).astype(np.uint8)
    return hq_ad, hs_ad


def check_h_codes8(h_o, hq_o, hs_o, hq_g, hs_g, g_mid, rep: Report, prefix="h"):
    """check_h_codes for the A8 encoding of the W4A8 variant (INT8 codes, scale from
    amax / 127): a block scale may be the neighbouring code, and an element code the
    neighbouring integer, only where the oracle's h lies within the FP32 rounding
    band of that decision's threshold.  Returns the oracle's codes with every
    accepted decision taken on the other side."""
    n, I = h_o.shape
    h = h_o.astype(np.float64)
    amax = np.abs(h.reshape(n, I // 16, 16)).max(-1)
    flips = 0
    sd = np.argwhere(hs_o != hs_g)
    for r, b in sd:
        a, c = int(hs_o[r, b]), int(hs_g[r, b])
        assert abs(a - c) == 1, "row %d block %d: scale codes %d vs %d" % (r, b, a, c)
        lo = min(a, c)
        thr = 127.0 * g_mid * 0.5 * (oracle.ue4m3(lo) + oracle.ue4m3(lo + 1))
        assert abs(amax[r, b] - thr) <= BAND_REL * thr, "row %d block %d: scale flip outside band" % (r, b)
        flips += 1
    qo, qg = np.asarray(hq_o, np.int64), np.asarray(hq_g, np.int8).astype(np.int64)
    q_ad = qo.copy()
    hs_ad = np.array(hs_o, copy=True)
    for r, b in sd:  # the block re-encoded under the GPU's scale
        hs_ad[r, b] = hs_g[r, b]
        s = oracle.ue4m3(int(hs_g[r, b])) * g_mid
        for i in range(16):
            q_ad[r, b * 16 + i] = oracle.int8_code(float(h[r, b * 16 + i]), s)
    for r, i in np.argwhere(q_ad != qg):
        co, cg = int(q_ad[r, i]), int(qg[r, i])
        assert abs(co - cg) == 1 and (co * cg >= 0), "row %d col %d: codes %d vs %d" % (r, i, co, cg)
        s = oracle.ue4m3(int(hs_g[r, i // 16])) * g_mid
        thr = (min(abs(co), abs(cg)) + 0.5) * s
        assert abs(abs(h[r, i]) - thr) <= BAND_REL * thr, "row %d col %d: code flip outside band (%.9g vs %.9g)" % (
            r, i, abs(h[r, i]), thr)
        q_ad[r, i] = cg
        flips += 1
    rep[prefix + "_flips"] = flips
    assert flips <= max(1, 1e-4 * n * I), "%d A8(h) flips exceed 1e-4 of %d elements" % (flips, n * I)
    assert np.array_equal(q_ad, qg) and np.array_equal(hs_ad, hs_g)
    return q_ad.astype(np.int8), hs_ad


# ---------------------------------------------------------------- output
def f32_to_bf16_rne_bits(v32):
    """FP32 values -> BF16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(v32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_order(bits):
    """BF16 bit patterns -> integers in value order (adjacent values differ by 1)."""
    b = np.asarray(bits).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_output(out_g_bits, out64, out16_o, rep: Report, v32=None, rel_l2_tol=2e-3, maxabs_rel=1e-2):
    """The layer output against the oracle: the output bars of the checker.

    out_g_bits: the GPU's BF16 output; out64 / out16_o: the oracle's FP64 value and
    its BF16 rounding; v32: the GPU's FP32 sum before its rounding (residual
    included).  Bars:
      * rel-L2 of the BF16 output against the oracle's BF16 output <= 2e-3;
      * the FP32 sum within 1e-2 * RMS of the FP64 value everywhere, no exemption;
      * the BF16 output is exactly the round-to-nearest-even of that FP32 sum;
      * every BF16 element more than 1e-2 * RMS from the oracle's BF16 value is
        one ulp from it, with a rounding midpoint lying between the FP32 sum and
        the FP64 value (a verified straddle: both neighbours are correct roundings
        of a value the two sums bracket).
    """
    g = bf16_bits_to_f64(out_g_bits)
    o16 = bf16_bits_to_f64(out16_o)
    rms = float(np.sqrt(np.mean(out64 ** 2))) if out64.size else 0.0
    num = float(np.linalg.norm(g - o16))
    den = float(np.linalg.norm(o16))
    rel = num / den if den > 0 else num
    rep["rel_l2"] = rel
    assert rel <= rel_l2_tol, "rel-L2 %.3g > %.3g" % (rel, rel_l2_tol)
    diff = np.abs(g - out64)
    rep["maxabs_over_rms"] = float(diff.max() / rms) if rms > 0 and diff.size else 0.0
    bar = maxabs_rel * rms
    if v32 is None:  # no FP32 sum available: one-ulp differences across a midpoint accepted unverified
        e = np.floor(np.log2(np.maximum(np.abs(out64), 1e-300)))
        bad = (diff > bar) & (diff > np.exp2(e - 7))
        assert not bad.any(), "max-abs %.3g > %.3g * RMS outside one-ulp differences (%d elements)" % (
            diff.max(), maxabs_rel, int(bad.sum()))
        return rel
    v32 = np.asarray(v32, np.float32)
    d32 = np.abs(v32.astype(np.float64) - out64)
    rep["fp32_maxabs_over_rms"] = float(d32.max() / rms) if rms > 0 and d32.size else 0.0
    assert np.all(d32 <= bar), "FP32 sum: max-abs %.3g > %.3g * RMS (no exemption)" % (d32.max(), maxabs_rel)
    own = f32_to_bf16_rne_bits(v32)
    nown = int((own != np.asarray(out_g_bits, np.uint16)).sum())
    assert nown == 0, "%d BF16 outputs are not the rounding of the kernel's own FP32 sum" % nown
    far = np.abs(g - o16) > bar
    rep["straddles"] = int(far.sum())
    if far.any():
        gb, ob = np.asarray(out_g_bits, np.uint16)[far], np.asarray(out16_o, np.uint16)[far]
        adj = np.abs(_bf16_order(gb) - _bf16_order(ob)) == 1
        assert adj.all(), "%d BF16 outputs beyond the bar are not one ulp from the oracle's" % int((~adj).sum())
        mid = 0.5 * (g[far] + o16[far])
        a, b = v32.astype(np.float64)[far], out64[far]
        between = (np.minimum(a, b) <= mid) & (mid <= np.maximum(a, b))
        assert between.all(), "%d one-ulp differences without a midpoint between the FP32 and FP64 sums" % int(
            (~between).sum())
    return rel


def check_fp32_rows(y_g, y_o, rep: Report, name, tol_rel_rms=1e-4):
    rms = float(np.sqrt(np.mean(y_o ** 2))) if y_o.size else 0.0
    err = float(np.abs(y_g.astype(np.float64) - y_o).max()) if y_o.size else 0.0
    rep[name + "_maxerr_over_rms"] = err / rms if rms > 0 else err
    assert err <= tol_rel_rms * rms + 1e-30, "%s: max error %.3g > %.3g * RMS %.3g" % (name, err, tol_rel_rms, rms)

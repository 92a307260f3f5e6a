"""Pins of the FP64 oracle against facts fixed outside it (CPU only).

Each test reaches the oracle's answer by another route: the formats' published
tables, exact integer arithmetic, nearest-grid search by distances, library
routines (numpy sort / matmul, scipy expit), invariants and the pages' printed
numbers.  A dropped term, a wrong sign or index or a transposed operand in the
oracle fails at least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import gen
import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- formats (F1, F2)
def test_e2m1_table_matches_ocp():
    for code, val in _read_table("e2m1_table.txt"):
        v = oracle.e2m1(int(code))
        assert v == float(val) and np.signbit(v) == val.startswith("-"), code


def test_ue4m3_landmarks_match_ofp8():
    for code, val in _read_table("ue4m3_points.txt"):
        assert oracle.ue4m3(int(code, 16)) == float(val), code


def test_ue4m3_grid_structure():
    vals = [oracle.ue4m3(c) for c in range(127)]
    assert all(b > a for a, b in zip(vals, vals[1:])), "grid must be strictly increasing"
    assert np.isnan(oracle.ue4m3(0x7F)) and np.isnan(oracle.ue4m3(0x80))
    # 4 significant bits: every normal value times 8 / 2^floor(log2) is an integer in [8, 16)
    for c in range(8, 127):
        m, e = np.frexp(vals[c])
        assert (m * 16) == int(m * 16) and 8 <= m * 16 < 16
    # subnormals are m * 2^-9
    assert vals[:8] == [m * 2.0 ** -9 for m in range(8)]


# ---------------------------------------------------------------- Q1, Q2 (nearest-grid pins)
E2M1_MAG = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
UE4M3 = np.array([float(v) for v in
                  [Fraction(m, 512) for m in range(8)] +
                  [Fraction(8 + m, 8) * Fraction(2) ** (e - 7) for e in range(1, 16) for m in range(8)][:119]])


def _nearest_even(grid, v):
    """Nearest grid index by distance, ties to the even index, saturating above the
    top of the grid (grid ascending).  For v at most the top of the grid, the
    distances to the grid points near v are exact in FP64, so ties are exact."""
    v = np.asarray(v, dtype=np.float64)
    d = np.abs(v[..., None] - grid)
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    idx = np.arange(grid.shape[0])
    # among tied candidates prefer the even index (at most two candidates tie)
    score = np.where(cand, np.where(idx % 2 == 0, 0, 1), 9) * 10000 + idx
    out = np.argmin(score, axis=-1)
    return np.where(v > grid[-1], grid.shape[0] - 1, out)


def _all_bf16_finite():
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def test_ue4m3_constructed_grid_equals_oracle():
    assert UE4M3.shape == (127,)
    assert np.array_equal(UE4M3, [oracle.ue4m3(c) for c in range(127)])


@pytest.mark.parametrize("g", [1.0, 2.0 ** -3, 2.0 ** 4])
def test_scale_code_exhaustive_bf16_amax(g):
    vals = _all_bf16_finite()
    amax = np.unique(np.abs(vals))
    # exact distances |amax - 6 g grid| (6 g grid has <= 6 significant bits; ties are exact)
    want = _nearest_even(6.0 * g * UE4M3, amax)
    got = np.array([oracle.scale_code(float(a), g) for a in amax])
    assert np.array_equal(got, want)


def test_scale_code_fp32_midpoints_and_neighbours():
    mids = 0.5 * (UE4M3[1:] + UE4M3[:-1]) * 6.0
    pts = []
    for m in mids.astype(np.float32):
        for d in (-2, -1, 0, 1, 2):
            pts.append(np.nextafter(m, np.float32(np.inf) if d > 0 else np.float32(0)) if d else m)
            if abs(d) == 2:
                pts[-1] = np.nextafter(pts[-1], np.float32(np.inf) if d > 0 else np.float32(0))
    rng = np.random.default_rng(7)
    pts = np.concatenate([np.array(pts, np.float32), rng.uniform(0, 3000, 20000).astype(np.float32),
                          np.float32(2.0) ** rng.uniform(-20, 12, 20000).astype(np.float32)])
    amax = pts.astype(np.float64)
    want = _nearest_even(6.0 * UE4M3, amax)
    got = np.array([oracle.scale_code(float(a), 1.0) for a in amax])
    assert np.array_equal(got, want)


def test_scale_code_ties_by_fractions():
    # exact midpoints: the even code must win
    for c in range(126):
        mid = (Fraction(UE4M3[c]) + Fraction(UE4M3[c + 1])) / 2 * 6
        got = oracle.scale_code(float(mid), 1.0)
        assert float(mid) == mid
        assert got == (c if c % 2 == 0 else c + 1), c


def test_elem_codes_exhaustive_bf16_all_scales():
    """All finite BF16 values x all 126 nonzero scales, each value placed in a block whose
    amax pins the scale code (amax = 6 * s exactly), versus nearest-by-distance with ties
    to even and saturation at 6 (8.3 M element decisions)."""
    vals = _all_bf16_finite()
    rows_codes, rows_want = [], []
    for c in range(1, 127):
        s = UE4M3[c]
        v = vals[np.abs(vals) <= 6.0 * s]
        pad = (-len(v)) % 15
        v = np.concatenate([v, np.zeros(pad)])
        blocks = v.reshape(-1, 15)
        blk = np.concatenate([np.full((blocks.shape[0], 1), 6.0 * s), blocks], axis=1)
        codes, scales = oracle.quantize(blk, 1.0)
        assert np.all(scales == c)
        lo, hi = codes & 15, codes >> 4
        got = np.stack([lo, hi], axis=-1).reshape(blk.shape)[:, 1:]
        # |x| has 8 significant bits and s 4, so |x|/s can only round onto a midpoint t when
        # |x| = t*s exactly: the FP64 quotient decides ties exactly
        mag = _nearest_even(E2M1_MAG, np.abs(blocks) / s)
        want = mag | np.where(np.signbit(blocks), 8, 0)
        rows_codes.append(got.ravel())
        rows_want.append(want.ravel())
    got, want = np.concatenate(rows_codes), np.concatenate(rows_want)
    assert np.array_equal(got, want)


def test_elem_code_ties_and_saturation_by_fractions():
    s = 0.875  # 4 significant bits
    for mag in range(7):
        mid = (Fraction(E2M1_MAG[mag]) + Fraction(E2M1_MAG[mag + 1])) / 2 * Fraction(s)
        even = mag if mag % 2 == 0 else mag + 1
        assert oracle.elem_code(float(mid), s) == even
        assert oracle.elem_code(-float(mid), s) == even | 8
    assert oracle.elem_code(1e30, s) == 7 and oracle.elem_code(-1e30, s) == 15
    assert oracle.elem_code(-1e-30, s) == 8  # sign kept on a zero magnitude
    assert oracle.elem_code(3.0, 0.0) == 0


# ---------------------------------------------------------------- A8 (the W4A8 variant's encoding)
@pytest.mark.parametrize("g", [1.0, 2.0 ** -4, 2.0 ** 3])
def test_scale_code8_exhaustive_bf16_amax(g):
    """A8 block scale: nearest point of the 127 g UE4M3 grid by distance (ties to the
    even code), over every BF16 amax (127 g grid values have <= 12 significant bits,
    so the distances near amax are exact in FP64)."""
    amax = np.unique(np.abs(_all_bf16_finite()))
    want = _nearest_even(127.0 * g * UE4M3, amax)
    got = np.array([oracle.scale_code8(float(a), g) for a in amax])
    assert np.array_equal(got, want)


def test_scale_code8_ties_by_fractions():
    for c in range(126):
        mid = (Fraction(UE4M3[c]) + Fraction(UE4M3[c + 1])) / 2 * 127
        assert float(mid) == mid
        assert oracle.scale_code8(float(mid), 1.0) == (c if c % 2 == 0 else c + 1), c


def test_int8_codes_exhaustive_bf16_all_scales():
    """All finite BF16 values x all 126 nonzero scales, each in a block whose amax
    pins the scale (amax = 127 s), against numpy: rint of the FP64 quotient, ties to
    even, saturation at 127.  |x| has 8 significant bits and s 4, so a quotient below
    127.5 is at least 1/(15 * 512) from any half-integer it does not equal: the FP64
    quotient rounds to the same integer as the exact one."""
    vals = _all_bf16_finite()
    got_all, want_all = [], []
    for c in range(1, 127):
        s = UE4M3[c]
        v = vals[np.abs(vals) <= 127.0 * s]
        pad = (-len(v)) % 15
        v = np.concatenate([v, np.zeros(pad)])
        blocks = v.reshape(-1, 15)
        blk = np.concatenate([np.full((blocks.shape[0], 1), 127.0 * s), blocks], axis=1)
        codes, scales = oracle.quantize8(blk, 1.0)
        assert np.all(scales == c)
        want = np.sign(blocks) * np.minimum(127.0, np.rint(np.abs(blocks) / s))
        got_all.append(codes[:, 1:].astype(np.float64).ravel())
        want_all.append(want.ravel())
    assert np.array_equal(np.concatenate(got_all), np.concatenate(want_all))


def test_int8_code_ties_saturation_and_zero_by_fractions():
    s = 0.6875  # 4 significant bits
    for m in range(127):
        mid = (Fraction(m) + Fraction(1, 2)) * Fraction(s)
        even = m if m % 2 == 0 else m + 1
        assert oracle.int8_code(float(mid), s) == min(even, 127)
        assert oracle.int8_code(-float(mid), s) == -min(even, 127)
    assert oracle.int8_code(1e30, s) == 127 and oracle.int8_code(-1e30, s) == -127
    assert oracle.int8_code(-1e-30, s) == 0 and oracle.int8_code(3.0, 0.0) == 0


def test_quantize8_idempotent_on_grid():
    """Blocks holding a +-127 code with any scale: quantize8(q * s) == (q, s)."""
    rng = np.random.default_rng(13)
    q = rng.integers(-127, 128, size=(400, 16))
    q[np.arange(400), rng.integers(0, 16, 400)] = np.where(rng.random(400) < .5, 127, -127)
    sc = rng.integers(1, 127, size=(400, 1))
    codes, scales = oracle.quantize8(q * UE4M3[sc], 1.0)
    assert np.array_equal(scales[:, 0], sc[:, 0]) and np.array_equal(codes, q)


def test_expert_ffn_a8_exact_integer_c0():
    """The W4A8 expert FFN as exact integers: int8 activation codes times twice the
    E2M1 weight codes, block by block, times the two UE4M3 scales (each x 512)."""
    L = gen.make_layer(0)
    sh = L.shape
    x = gen.make_tokens(0, 6, step=27)
    g_in, g_mid = 2.0 ** -4, 2.0 ** -8
    xq, xs = oracle.quantize8(oracle.bf16_to_f64(x), g_in)
    rows = np.repeat(np.arange(6, dtype=np.int32), 2)
    exps = np.tile(np.array([2, 11], np.int32), 6)
    r = oracle.expert_rows(rows, exps, xq, xs, L.w13, L.w2, sh.H, sh.I, g_in, g_mid, want_gu=True, act_bits=8)

    def dot8(qa, sa, qw, sw):  # integer N with dot = N / (2 * 512 * 512)
        a = qa.astype(np.int64)
        w = E2M1_X2[_unpack(qw)]
        K = a.shape[-1]
        inner = (a.reshape(-1, K // 16, 16)[:, None] * w.reshape(-1, K // 16, 16)[None]).sum(-1)
        return (inner * _ue4m3_x512(sa)[:, None, :] * _ue4m3_x512(sw)[None, :, :]).sum(-1)

    den = 2.0 * 512 * 512
    for e in (2, 11):
        N = dot8(xq, xs, L.w13["codes"][e], L.w13["scales"][e]).astype(np.float64)
        gu = N / den * float(L.w13["gscale"][e]) * g_in
        sel = exps == e
        assert np.allclose(r["g"][sel], gu[rows[sel], :sh.I], rtol=1e-14, atol=1e-300)
        assert np.allclose(r["u"][sel], gu[rows[sel], sh.I:], rtol=1e-14, atol=1e-300)
    hq, hs = oracle.quantize8(r["h"].astype(np.float64), g_mid)
    assert np.array_equal(hq, r["hq"]) and np.array_equal(hs, r["hs"])
    assert np.count_nonzero(hq) > 0.9 * hq.size  # the global scale keeps h's scales off the underflow
    for i, e in enumerate(exps[:4]):
        N = dot8(r["hq"][i:i + 1], r["hs"][i:i + 1], L.w2["codes"][e], L.w2["scales"][e])[0]
        assert np.allclose(r["y"][i], N / den * float(L.w2["gscale"][e]) * g_mid, rtol=1e-14, atol=1e-300)


def test_expert_ffn_a8_dense_reduction_numpy_matmul():
    """E = 1, k = 1: the W4A8 layer is a dense SwiGLU MLP on dequantized operands."""
    L = gen.make_layer(0)
    sh = L.shape
    x = gen.make_tokens(0, 8, step=28)
    g_in, g_mid = 2.0 ** -4, 2.0 ** -8
    xq, xs = oracle.quantize8(oracle.bf16_to_f64(x), g_in)

    def deq4(codes, scales):
        return (E2M1_X2[_unpack(codes)] / 2.0) * np.repeat(UE4M3[scales], 16, axis=-1)

    def deq8(codes, scales, g):
        return codes.astype(np.float64) * np.repeat(UE4M3[scales], 16, axis=-1) * g

    e = 5
    W13 = deq4(L.w13["codes"][e], L.w13["scales"][e]) * float(L.w13["gscale"][e])
    W2 = deq4(L.w2["codes"][e], L.w2["scales"][e]) * float(L.w2["gscale"][e])
    r = oracle.expert_rows(np.arange(8, dtype=np.int32), np.full(8, e, np.int32), xq, xs, L.w13, L.w2, sh.H, sh.I,
                           g_in, g_mid, want_gu=True, act_bits=8)
    gu = deq8(xq, xs, g_in) @ W13.T
    assert np.allclose(r["g"], gu[:, :sh.I], rtol=1e-12, atol=1e-15)
    assert np.allclose(r["u"], gu[:, sh.I:], rtol=1e-12, atol=1e-15)
    assert np.allclose(r["y"], deq8(r["hq"], r["hs"], g_mid) @ W2.T, rtol=1e-12, atol=1e-15)


def test_quantize_idempotent_on_grid():
    rng = np.random.default_rng(3)
    # blocks containing a +-6 code: quantize(dequantize(q, s)) == (q, s)
    q = rng.integers(0, 16, size=(400, 16))
    q[:, rng.integers(0, 16, 400)] = 0
    q[np.arange(400), rng.integers(0, 16, 400)] = np.where(rng.random(400) < .5, 7, 15)
    sc = rng.integers(1, 127, size=(400, 1))
    vals = np.vectorize(oracle.e2m1)(q) * UE4M3[sc]
    codes, scales = oracle.quantize(vals, 1.0)
    qq = np.stack([codes & 15, codes >> 4], -1).reshape(400, 16)
    assert np.array_equal(scales[:, 0], sc[:, 0])
    # -0 and +0 keep their sign; compare values
    assert np.array_equal(np.vectorize(oracle.e2m1)(qq), np.vectorize(oracle.e2m1)(q))


def test_single_nonzero_block():
    for v in (1.0, -3.7, 0.07, 250.0, -1e-3):
        blk = np.zeros((1, 16))
        blk[0, 5] = v
        codes, scales = oracle.quantize(blk)
        c = (codes[0, 2] >> 4) & 15
        assert codes[0, 2] & 15 == 0 and bool(c & 8) == (v < 0)
        if abs(v) / 6 < 2.0 ** -10:
            # amax/6 below half the smallest subnormal scale: scale 0, magnitude 0
            assert scales[0, 0] == 0 and (c & 7) == 0
        else:
            # amax/6 rounds to the scale grid, so the element lands on 6 or its neighbour 4
            assert (c & 7) in (6, 7)


# ---------------------------------------------------------------- formats: BF16 / FP16 rounding
def test_round_bf16_by_fractions():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000))
    # exact ties between adjacent BF16 values
    for b in rng.integers(0x0080, 0x7F00, 500):
        a = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        nb = float(np.array([(b + 1) << 16], np.uint32).view(np.float32)[0])
        vals.append((a + nb) / 2)
    for v in vals:
        got = int(oracle.round_bf16(np.array([v]))[0])
        fv = Fraction(v)
        # candidates: all BF16 near v
        f32 = np.float32(v)
        base = int(np.array([f32], np.float32).view(np.uint32)[0]) >> 16
        best = None
        for c in range(base - 2, base + 3):
            cv = Fraction(float(np.array([c << 16], np.uint32).view(np.float32)[0]))
            d = abs(cv - fv)
            key = (d, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        assert got == best[1], v


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(12)
    vals = rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000)
    for v in vals:
        if abs(v) <= 65504:
            assert oracle.round_f16_sat(float(v)) == float(np.float16(v)), v
    assert oracle.round_f16_sat(1e6) == 65504.0 and oracle.round_f16_sat(-7e4) == -65504.0


# ---------------------------------------------------------------- router (R)
def test_router_logits_exact_rational_c0():
    L = gen.make_layer(0)
    x = gen.make_tokens(0, 8)
    lg = oracle.router_logits(x, L.router_w)
    xf = oracle.bf16_to_f64(x)
    # independent check via exact fractions on a subset of (token, expert)
    for t in range(0, 8, 3):
        for e in range(0, 16, 5):
            exact = sum(Fraction(float(xf[t, h])) * Fraction(float(L.router_w[e, h])) for h in range(256))
            assert abs(Fraction(lg[t, e]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)
    # and a library matmul on the whole thing
    assert np.allclose(lg, xf @ L.router_w.astype(np.float64).T, rtol=1e-12, atol=1e-13)


def test_topk_matches_stable_sort_and_softmax():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((300, 64))
    lg[:50, 7] = lg[:50, 3]  # exact duplicates: the lower id must come first
    lg[50:60] = 1.25          # all equal: ids 0..k-1
    k = 6
    idx, w = oracle.topk_softmax(lg, k)
    want = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, want)
    from scipy.special import softmax
    sel = np.take_along_axis(lg, want, 1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15)


def test_topk_invariants():
    rng = np.random.default_rng(6)
    lg = rng.standard_normal((200, 512)) * 0.9
    idx, w = oracle.topk_softmax(lg, 10)
    for t in range(200):
        sel = lg[t, idx[t]]
        rest = np.delete(lg[t], idx[t])
        assert sel.min() >= rest.max()
        assert np.all(np.diff(sel) <= 0)
    idx2, w2 = oracle.topk_softmax(lg + 3.5, 10)  # a constant shift changes nothing
    assert np.array_equal(idx, idx2) and np.allclose(w, w2, rtol=1e-13)
    i1, w1 = oracle.topk_softmax(lg, 1)
    assert np.all(w1 == 1.0) and np.array_equal(i1[:, 0], lg.argmax(1))


# ---------------------------------------------------------------- permutation (P)
@pytest.mark.parametrize("T,E,k", [(8, 16, 2), (300, 64, 6), (50, 8, 8), (1, 512, 10), (0, 16, 2)])
def test_permute_matches_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    off, r2p, p2r = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(r2p, np.argsort(flat, kind="stable"))
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(p2r[r2p], np.arange(T * k))


def test_permute_degenerate():
    T, E = 40, 8
    idx = np.tile(np.arange(E, dtype=np.int32), (T, 1))  # k = E: every token in every segment
    off, r2p, p2r = oracle.permute(idx, E)
    assert np.array_equal(off, np.arange(E + 1) * T)
    assert np.array_equal(r2p[off[3]:off[4]] // E, np.arange(T))
    idx1 = np.full((T, 1), 5, np.int32)  # all tokens to one expert
    off, r2p, _ = oracle.permute(idx1, E)
    assert np.array_equal(off, [0, 0, 0, 0, 0, 0, T, T, T]) and np.array_equal(r2p, np.arange(T))


# ---------------------------------------------------------------- expert FFN (X) by exact integers
E2M1_X2 = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12], np.int64)  # 2 * e2m1


def _ue4m3_x512(codes):
    return np.round(UE4M3[codes] * 512).astype(np.int64)  # exact integers


def _unpack(codes):
    return np.stack([codes & 15, codes >> 4], -1).reshape(*codes.shape[:-1], -1)


def _exact_dot_int(qa, sa, qw, sw):
    """Integer N with dot = N / (4 * 512 * 512), exact: sum_b (sa*512)(sw*512) sum_i (2qa)(2qw)."""
    a = E2M1_X2[_unpack(qa)]  # [..., K]
    w = E2M1_X2[_unpack(qw)]
    K = a.shape[-1]
    inner = (a.reshape(-1, K // 16, 16)[:, None] * w.reshape(-1, K // 16, 16)[None]).sum(-1)  # [ra, rw, nb]
    scale = _ue4m3_x512(sa)[:, None, :] * _ue4m3_x512(sw)[None, :, :]
    return (inner * scale).sum(-1)  # [ra, rw]


def test_expert_ffn_exact_integer_c0():
    L = gen.make_layer(0)
    sh = L.shape
    x = gen.make_tokens(0, 8)
    xq, xs = oracle.quantize(oracle.bf16_to_f64(x))
    rows = np.repeat(np.arange(8, dtype=np.int32), 3)
    exps = np.tile(np.array([0, 7, 15], np.int32), 8)
    r = oracle.expert_rows(rows, exps, xq, xs, L.w13, L.w2, sh.H, sh.I, want_gu=True)
    den = 4.0 * 512 * 512
    for e in (0, 7, 15):
        N = _exact_dot_int(xq, xs, L.w13["codes"][e], L.w13["scales"][e]).astype(np.float64)
        gu = N / den * float(L.w13["gscale"][e])
        sel = exps == e
        assert np.allclose(r["g"][sel], gu[rows[sel], :sh.I], rtol=1e-14, atol=1e-300)
        assert np.allclose(r["u"][sel], gu[rows[sel], sh.I:], rtol=1e-14, atol=1e-300)
    # h = fl32(silu(g) * u) with silu via scipy's expit
    from scipy.special import expit
    h_want = (r["g"] * expit(r["g"]) * r["u"]).astype(np.float32)
    assert np.max(np.abs(h_want.astype(np.float64) - r["h"]) / (np.abs(h_want) + 1e-30)) <= 2 ** -23
    # codes of h are the A4 encoding of h (pinned above), and y is the exact down product of those codes
    hq, hs = oracle.quantize(r["h"].astype(np.float64))
    assert np.array_equal(hq, r["hq"]) and np.array_equal(hs, r["hs"])
    for i, e in enumerate(exps[:6]):
        N = _exact_dot_int(r["hq"][i:i + 1], r["hs"][i:i + 1], L.w2["codes"][e], L.w2["scales"][e])[0]
        assert np.allclose(r["y"][i], N / den * float(L.w2["gscale"][e]), rtol=1e-14, atol=1e-300)


def test_expert_ffn_dense_reduction_numpy_matmul():
    """E = 1, k = 1, no shared expert: the layer is a dense NVFP4 SwiGLU MLP; numpy's matmul
    on dequantized tensors (dequantized here from the format tables) reproduces it."""
    L = gen.make_layer(0)
    sh = L.shape
    x = gen.make_tokens(0, 8, step=3)
    xf = oracle.bf16_to_f64(x)
    xq, xs = oracle.quantize(xf)

    def deq(codes, scales):
        vals = (E2M1_X2[_unpack(codes)] / 2.0)
        return vals * np.repeat(UE4M3[scales], 16, axis=-1)

    e = 3
    W13 = deq(L.w13["codes"][e], L.w13["scales"][e]) * float(L.w13["gscale"][e])
    W2 = deq(L.w2["codes"][e], L.w2["scales"][e]) * float(L.w2["gscale"][e])
    xd = deq(xq, xs)
    gu = xd @ W13.T
    r = oracle.expert_rows(np.arange(8, dtype=np.int32), np.full(8, e, np.int32), xq, xs, L.w13, L.w2, sh.H, sh.I,
                           want_gu=True)
    assert np.allclose(r["g"], gu[:, :sh.I], rtol=1e-12, atol=1e-15)
    assert np.allclose(r["u"], gu[:, sh.I:], rtol=1e-12, atol=1e-15)
    y = deq(r["hq"], r["hs"]) @ W2.T
    assert np.allclose(r["y"], y, rtol=1e-12, atol=1e-15)


def test_down_k_split_adds_up():
    L = gen.make_layer(0)
    sh = L.shape
    x = gen.make_tokens(0, 4, step=5)
    xq, xs = oracle.quantize(oracle.bf16_to_f64(x))
    args = (np.arange(4, dtype=np.int32), np.array([1, 2, 3, 4], np.int32), xq, xs, L.w13, L.w2, sh.H, sh.I)
    full = oracle.expert_rows(*args)["y"]
    a = oracle.expert_rows(*args, kb=(0, sh.I // 32))["y"]
    b = oracle.expert_rows(*args, kb=(sh.I // 32, sh.I // 16))["y"]
    assert np.allclose(a + b, full, rtol=1e-13, atol=1e-16)


# ---------------------------------------------------------------- combine (C)
def test_combine_linear_and_special_values():
    rng = np.random.default_rng(9)
    n, k, H = 5, 3, 64
    y1, y2 = rng.standard_normal((n, k, H)), rng.standard_normal((n, k, H))
    w = rng.random((n, k)).astype(np.float32)
    ysh = rng.standard_normal((n, H))
    a, b = 0.75, -2.5
    o1, _ = oracle.combine(y1, w, ysh)
    o2, _ = oracle.combine(y2, w, ysh)
    o12, _ = oracle.combine(a * y1 + b * y2, w, (a + b) * ysh)
    assert np.allclose(o12, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    oc, _ = oracle.combine(y1, (w * 2).astype(np.float32), None)
    oz, _ = oracle.combine(y1, w, None)
    assert np.allclose(oc, 2 * oz, rtol=1e-14)
    want = np.einsum("nk,nkh->nh", w.astype(np.float64), y1) + ysh
    assert np.allclose(o1, want, rtol=1e-13)
    zero, zb = oracle.combine(np.zeros((n, k, H)), w, np.zeros((n, H)))
    assert np.all(zero == 0) and np.all((zb & 0x7FFF) == 0)
    res = gen.make_tokens(0, n, step=9, H=H)
    _, rb = oracle.combine(np.zeros((n, k, H)), w, None, residual=res)
    assert np.array_equal(rb & 0x7FFF, res & 0x7FFF)


def test_layer_zero_input_gives_exact_zero():
    L = gen.make_layer(0)
    x = np.zeros((3, L.shape.H), np.uint16)
    r = oracle.layer(L, x)
    assert np.all(r["out_f64"] == 0.0)


def test_layer_equivariance_and_duplicates():
    L = gen.make_layer(0)
    x = gen.make_tokens(0, 8)
    x[5] = x[2]
    r = oracle.layer(L, x)
    assert np.array_equal(r["out_bf16"][5], r["out_bf16"][2])
    perm = np.random.default_rng(1).permutation(8)
    rp = oracle.layer(L, x[perm])
    assert np.array_equal(rp["out_bf16"], r["out_bf16"][perm])


# ---------------------------------------------------------------- the whole layer, composed independently
def _exact_dot_int_blocks(qa, sa, qw, sw, b0, b1):
    """_exact_dot_int over the 16-element blocks [b0, b1) only."""
    a = E2M1_X2[_unpack(qa)]
    w = E2M1_X2[_unpack(qw)]
    K = a.shape[-1]
    inner = (a.reshape(-1, K // 16, 16)[:, None, b0:b1] * w.reshape(-1, K // 16, 16)[None, :, b0:b1]).sum(-1)
    scale = _ue4m3_x512(sa)[:, None, b0:b1] * _ue4m3_x512(sw)[None, :, b0:b1]
    return (inner * scale).sum(-1)


def _bf16_bits(v):
    return (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rne_bf16_exact(q):
    """Round an exact rational to the nearest BF16 (ties to even) by integer
    arithmetic; returns (bits, distance to the nearest rounding midpoint)."""
    if q == 0:
        return 0, Fraction(1)
    a = abs(q)
    e = int(np.floor(np.log2(float(a))))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** max(e - 7, -133)  # 8 significant bits
    n = a / quantum
    m = n.numerator // n.denominator
    frac = n - m
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and m % 2 == 1):
        m += 1
    val = float(m * quantum) * (1 if q > 0 else -1)
    return int(_bf16_bits(val)), abs(frac - Fraction(1, 2)) * quantum


def _layer_exact(L, x, residual=None, kb=None):
    """The layer of one call composed without oracle.layer or oracle.expert_rows:
    exact-rational router logits, top k by a stable sort, softmax by scipy,
    A4 codes by the (separately pinned) encoder, gate/up and down products as exact
    integers, h = fl32(silu(g) u) with scipy's expit, and the combine as an exact
    rational (routed rows times their FP32 weights, the shared row with weight 1,
    the residual).  Returns (idx, w32, exact outputs as Fractions, per-element
    scale of the summed terms)."""
    from scipy.special import expit, softmax
    sh = L.shape
    H, I, k = sh.H, sh.I, sh.k
    T = x.shape[0]
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    lg = [[sum(Fraction(float(xf[t, h])) * Fraction(float(L.router_w[e, h])) for h in range(H)) for e in range(sh.E)]
          for t in range(T)]
    idx = np.array([sorted(range(sh.E), key=lambda e: (-lg[t][e], e))[:k] for t in range(T)], np.int32)
    w32 = np.array([softmax([float(lg[t][e]) for e in idx[t]]) for t in range(T)]).astype(np.float32)
    a8 = getattr(L, "act_bits", 4) == 8
    g_in, g_mid = L.a_gscale_in, L.a_gscale_mid
    enc = oracle.quantize8 if a8 else oracle.quantize  # the encoders are pinned separately
    xq, xs = enc(xf, g_in)
    b0, b1 = kb if kb is not None else (0, I // 16)
    den = (2 if a8 else 4) * 512 * 512

    def dot(qa, sa, qw, sw, c0, c1):  # exact integer N with the dot = N / den
        a = qa.astype(np.int64) if a8 else E2M1_X2[_unpack(qa)]
        w = E2M1_X2[_unpack(qw)]
        K = a.shape[-1]
        inner = (a.reshape(-1, K // 16, 16)[:, None, c0:c1] * w.reshape(-1, K // 16, 16)[None, :, c0:c1]).sum(-1)
        return (inner * _ue4m3_x512(sa)[:, None, c0:c1] * _ue4m3_x512(sw)[None, :, c0:c1]).sum(-1)

    def ffn(bank13, bank2, e, t):
        N = dot(xq[t:t + 1], xs[t:t + 1], bank13["codes"][e], bank13["scales"][e], 0, H // 16)[0]
        gsc = Fraction(float(bank13["gscale"][e])) * Fraction(g_in)
        gu = np.array([float(Fraction(int(n), den) * gsc) for n in N])
        g, u = gu[:I], gu[I:]
        h = (g * expit(g) * u).astype(np.float32).astype(np.float64)[None]
        hq, hs = enc(h, g_mid)
        Ny = dot(hq, hs, bank2["codes"][e], bank2["scales"][e], b0, b1)[0]
        return [Fraction(int(n), den) * Fraction(float(bank2["gscale"][e])) * Fraction(g_mid) for n in Ny]

    out, mag = [], []
    for t in range(T):
        rows = [ffn(L.w13, L.w2, int(idx[t, j]), t) for j in range(k)]
        terms = [[Fraction(float(w32[t, j])) * rows[j][n] for n in range(H)] for j in range(k)]
        if L.sh13 is not None:
            ysh = ffn(L.sh13, L.sh2, 0, t)
            if getattr(L, "shared_gate_w", None) is not None:
                z = sum(Fraction(float(xf[t, h])) * Fraction(float(L.shared_gate_w[h])) for h in range(H))
                g = Fraction(float(np.float32(expit(float(z)))))
                ysh = [g * v for v in ysh]
            terms.append(ysh)
        if residual is not None:
            terms.append([Fraction(float(v)) for v in (residual[t].astype(np.uint32) << 16).view(np.float32)])
        out.append([sum(tt[n] for tt in terms) for n in range(H)])
        mag.append([float(sum(abs(tt[n]) for tt in terms)) for n in range(H)])
    return idx, w32, out, np.array(mag)


def _assert_layer_matches_exact(r, idx, w32, out, mag):
    assert np.array_equal(r["idx"], idx)
    assert np.allclose(r["w"], w32, rtol=2.0 ** -22, atol=0)
    ex = np.array([[float(v) for v in row] for row in out])
    tol = 2.0 ** -30 * mag + 1e-300  # the oracle's FP64 rounding of h, y and the sums
    assert np.all(np.abs(r["out_f64"] - ex) <= tol)
    checked = 0
    for t in range(ex.shape[0]):
        for n in range(ex.shape[1]):
            bits, dmid = _rne_bf16_exact(out[t][n])
            if dmid > tol[t, n]:  # not within the oracle's rounding of a BF16 midpoint
                assert int(r["out_bf16"][t, n]) == bits, (t, n)
                checked += 1
    assert checked >= 0.99 * ex.size
    return ex


def test_layer_composition_exact_c0():
    """oracle.layer against the independent composition, with the residual and a
    K-split of the down projections; and a dropped shared row, residual or K range
    would be caught (each changes the output far beyond the tolerance)."""
    L = gen.make_layer(0)
    T, H, I = 6, L.shape.H, L.shape.I
    x = gen.make_tokens(0, T, step=21)
    res = gen.make_tokens(0, T, step=22)
    kb = (0, I // 32)
    r = oracle.layer(L, x, residual=res, kb=kb)
    idx, w32, out, mag = _layer_exact(L, x, residual=res, kb=kb)
    ex = _assert_layer_matches_exact(r, idx, w32, out, mag)
    rms = np.sqrt(np.mean(ex ** 2))
    for what in ("shared", "residual", "kb"):
        L2 = gen.Layer(**{**L.__dict__, "sh13": None, "sh2": None}) if what == "shared" else L
        _, _, out2, _ = _layer_exact(L2, x, residual=None if what == "residual" else res,
                                     kb=None if what == "kb" else kb)
        alt = np.array([[float(v) for v in row] for row in out2])
        assert np.mean(np.abs(alt - ex) > 1e-3 * rms) > 0.5, what


def test_layer_without_shared_and_token_subset_c0():
    """A layer without the shared expert (its term is absent, not zero-weighted by
    accident), and the tokens= subset of a call equals the call on those tokens."""
    L = gen.make_layer(0)
    L0 = gen.Layer(**{**L.__dict__, "sh13": None, "sh2": None})
    x = gen.make_tokens(0, 8, step=23)
    r = oracle.layer(L0, x)
    assert r["shared"] is None
    idx, w32, out, mag = _layer_exact(L0, x)
    _assert_layer_matches_exact(r, idx, w32, out, mag)
    sub = np.array([6, 1, 3], np.int32)
    rs = oracle.layer(L0, x, tokens=sub)
    assert np.array_equal(rs["out_bf16"], r["out_bf16"][sub]) and np.array_equal(rs["out_f64"], r["out_f64"][sub])
    assert np.array_equal(rs["idx"], r["idx"][sub])


def test_layer_composition_w4a8_c0():
    """oracle.layer in the W4A8 variant (A8 encodings, power-of-two global scales)
    against the independent composition, with the residual and the shared gate."""
    L = gen.make_layer(0, shared_gate=True)
    L.act_bits, L.a_gscale_in, L.a_gscale_mid = 8, 2.0 ** -4, 2.0 ** -8
    x = gen.make_tokens(0, 5, step=29)
    res = gen.make_tokens(0, 5, step=30)
    r = oracle.layer(L, x, residual=res)
    assert r["xq"].dtype == np.int8 and r["xq"].shape == (5, L.shape.H)
    idx, w32, out, mag = _layer_exact(L, x, residual=res)
    _assert_layer_matches_exact(r, idx, w32, out, mag)


def test_shared_gate_exact_rational_and_closed_forms():
    """The optional shared-expert gate: z by exact fractions and the sigmoid by
    scipy's expit give the oracle's FP32 gate (to one FP32 rounding of the
    sigmoid); zero weights give exactly 1/2; a gate vector aligned with x drives
    it to 1 and its negative to 0."""
    from scipy.special import expit
    L = gen.make_layer(0, shared_gate=True)
    x = gen.make_tokens(0, 8, step=24)
    g = oracle.shared_gate(x, L.shared_gate_w)
    xf = oracle.bf16_to_f64(x)
    for t in range(8):
        z = sum(Fraction(float(xf[t, h])) * Fraction(float(L.shared_gate_w[h])) for h in range(L.shape.H))
        want = np.float32(expit(float(z)))
        assert abs(float(g[t]) - float(want)) <= 2.0 ** -24 * float(want), t
    assert np.all(oracle.shared_gate(x, np.zeros(L.shape.H, np.float32)) == 0.5)
    big = (xf[0] * 10.0).astype(np.float32)
    assert oracle.shared_gate(x[:1], big)[0] == 1.0 and oracle.shared_gate(x[:1], -big)[0] == 0.0


def test_layer_composition_with_shared_gate_c0():
    """oracle.layer with the shared-expert gate against the independent composition;
    dropping the gate would be caught."""
    L = gen.make_layer(0, shared_gate=True)
    x = gen.make_tokens(0, 5, step=25)
    res = gen.make_tokens(0, 5, step=26)
    r = oracle.layer(L, x, residual=res)
    idx, w32, out, mag = _layer_exact(L, x, residual=res)
    ex = _assert_layer_matches_exact(r, idx, w32, out, mag)
    L2 = gen.Layer(**{**L.__dict__, "shared_gate_w": None})
    _, _, out2, _ = _layer_exact(L2, x, residual=res)
    alt = np.array([[float(v) for v in row] for row in out2])
    assert np.mean(np.abs(alt - ex) > 1e-3 * np.sqrt(np.mean(ex ** 2))) > 0.5


# ---------------------------------------------------------------- the pages' printed sizes
def test_packed_size_matches_host_bank():
    facts = {r[0]: float(r[1]) for r in _read_table("page_facts.txt")}
    H, E, layers = facts["artifact_hidden"], facts["experts"], facts["expert_layers_with_mtp"]
    gib = facts["host_expert_bank_gib"] * 2 ** 30

    def inter(bits_per_weight):  # expert intermediate size the bank implies
        return gib * 8 / (bits_per_weight * 3 * H * E * layers)

    # 16-element blocks with a 1-byte UE4M3 scale: 4 + 8/16 = 4.5 bits per weight -> I = 640
    assert abs(inter(4.5) - 640) < 0.5
    # 32-element blocks (4.25 bits) would need a non-multiple-of-16 intermediate size
    assert abs(inter(4.25) - round(inter(4.25) / 16) * 16) > 2
    # and the bank per expert at I = 640 from the oracle-independent formula
    I = 640
    per_expert = 3 * H * I / 2 + 3 * H * I / 16
    assert round(per_expert * E * layers / 2 ** 30, 1) == facts["host_expert_bank_gib"]


def test_rms_norm_closed_forms():
    """The stack's RMS norm: closed forms and invariants (one nonzero element gives
    sign * sqrt(H); a constant row gives +-1; power-of-two scaling is invisible with
    eps = 0; the output's mean square is 1 within BF16 rounding)."""
    H = 2048
    x = np.zeros((3, H), np.float64)
    x[0, 5] = -3.25
    x[1, :] = 0.75
    x[2, :] = np.linspace(-2, 2, H)
    xb = oracle.round_bf16(x)
    n = oracle.bf16_to_f64(oracle.rms_norm(xb, eps=0.0))
    assert n[0, 5] == -45.25 and np.count_nonzero(n[0]) == 1  # sqrt(2048) = 45.2548 -> BF16 45.25
    assert np.all(n[1] == 1.0)
    xs = gen.make_tokens(1, 4)
    a = oracle.rms_norm(xs, eps=0.0)
    scaled = oracle.round_bf16(oracle.bf16_to_f64(xs) * 2.0 ** -5)
    assert np.array_equal(oracle.rms_norm(scaled, eps=0.0), a)
    v = oracle.bf16_to_f64(a)
    assert np.all(np.abs((v ** 2).mean(axis=1) - 1.0) < 2 ** -7)
    assert np.all(np.sign(v) == np.sign(oracle.bf16_to_f64(xs)))

"""Why the matrix-core kernels decode NVFP4 operands to FP16 rather than to an
8- or 4-bit matrix-core format (CPU only, measured on sampled tokens of the
15,360-token chunk's layer).

An NVFP4 element is an E2M1 code times a UE4M3 block scale (capy-flash README
v0.5.4, "What it does": FP4 weights and activations with block scales).  Its
significand has up to 6 bits, so it is exactly an FP16 number and the FP16
matrix cores reproduce every product; gfx950's faster matrix-core formats
carry one power-of-two (E8M0) scale per 32 elements and 4 significant bits
(FP8 E4M3) or 2 (FP4 E2M1), so an NVFP4 operand has to be rounded to reach
them.  This test rounds every GEMM operand of the layer that way, runs the
layer in FP64 otherwise (same routing, same A4(h) encoding of the rounded
h), and measures the output's relative L2 distance from the oracle's FP64
output.  The exact decode reproduces the oracle; both roundings are far
outside the 2e-3 relative-L2 bar the layer is held to, which is why the
exact FP16 path (and its ceiling of half the FP8 peak) is the design.
"""
import numpy as np
import pytest

import gen
import oracle

REL_L2_BAR = 2e-3
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _ue4m3(c):
    c = c.astype(np.int64)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))


def _decode(codes, scales):
    """Packed NVFP4 rows (element 2i in the low nibble) -> element values
    without the per-tensor scale, FP64."""
    q = np.stack((codes & 15, codes >> 4), axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    return _E2M1[q] * np.repeat(_ue4m3(scales), 16, axis=-1)


def _round_grid(x, sig_bits, emin, vmax):
    """Round to the nearest value (ties to even) of a binary format with
    sig_bits significant bits, smallest normal exponent emin, saturating at vmax."""
    ax = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 1.0))), emin)
    step = np.exp2(e - (sig_bits - 1))
    return np.clip(np.round(x / step) * step, -vmax, vmax)


def _mx(v, fmt):
    """MX-style rounding along the last axis: one power-of-two scale per 32
    elements, chosen as the smallest that keeps the block's largest magnitude
    inside the element format, then each element rounded to that format."""
    sig, emin, vmax = {"e4m3": (4, -6, 448.0), "e2m1": (2, 0, 6.0)}[fmt]
    b = v.reshape(*v.shape[:-1], -1, 32)
    amax = np.abs(b).max(axis=-1, keepdims=True)
    sc = np.exp2(np.ceil(np.log2(np.where(amax > 0, amax / vmax, 1.0))))
    return (_round_grid(b / sc, sig, emin, vmax) * sc).reshape(v.shape)


def _layer_emulated(L, x_bf16, fmt):
    """FP64 layer on operands rounded by fmt (None: exact NVFP4 values)."""
    sh = L.shape
    H, I, k = sh.H, sh.I, sh.k
    rnd = (lambda v: v) if fmt is None else (lambda v: _mx(v, fmt))
    ref = oracle.layer(L, x_bf16)
    xv = rnd(_decode(ref["xq"], ref["xs"]) * L.a_gscale_in)
    T = x_bf16.shape[0]

    cache = {}

    def weights(bank, e):
        key = (id(bank), e)
        if key not in cache:
            cache[key] = rnd(_decode(bank["codes"][e], bank["scales"][e])) * float(bank["gscale"][e])
        return cache[key]

    def ffn(xrow, bank13, bank2, e):
        gu = weights(bank13, e) @ xrow
        g, u = gu[:I], gu[I:]
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32).astype(np.float64)
        hq, hs = oracle.quantize(h[None, :], L.a_gscale_mid)
        hv = rnd(_decode(hq, hs)[0] * L.a_gscale_mid)
        return weights(bank2, e) @ hv

    out = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ref["idx"][t, j])
            out[t] += float(ref["w"][t, j]) * ffn(xv[t], L.w13, L.w2, e)
        out[t] += ffn(xv[t], L.sh13, L.sh2, 0)
    return out, ref["out_f64"]


@pytest.fixture(scope="module")
def c3_sample():
    L = gen.make_layer(3)
    x = gen.make_tokens(3, 4, step=7)
    return L, x


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_exact_decode_reproduces_the_oracle(c3_sample):
    out, ref = _layer_emulated(*c3_sample, None)
    assert _rel_l2(out, ref) < 1e-9


@pytest.mark.parametrize("fmt, floor", [("e4m3", 10 * REL_L2_BAR), ("e2m1", 50 * REL_L2_BAR)])
def test_rounded_operands_miss_the_bar(c3_sample, fmt, floor):
    out, ref = _layer_emulated(*c3_sample, fmt)
    rel = _rel_l2(out, ref)
    print("%s operands (E8M0 scale per 32): output rel-L2 %.4g against the FP64 oracle" % (fmt, rel))
    assert rel > floor

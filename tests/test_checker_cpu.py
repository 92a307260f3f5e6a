"""The parity checker's own rules, on the CPU with constructed inputs: it accepts
what the readings allow (a decision inside the FP32 rounding band of a threshold,
a BF16 value straddling a rounding midpoint between the FP32 and FP64 sums) and
rejects what they do not."""
import numpy as np
import pytest

import checker
import oracle


def _a8_case(seed=0):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((4, 32)) * 0.3).astype(np.float32).astype(np.float64)
    q, s = oracle.quantize8(h, 2.0 ** -4)
    return h, q, s


def test_a8_h_codes_identical_and_band_flip_accepted():
    h, q, s = _a8_case()
    rep = checker.Report()
    qa, sa = checker.check_h_codes8(h, q, s, q.copy(), s.copy(), 2.0 ** -4, rep)
    assert rep["h_flips"] == 0 and np.array_equal(qa, q)
    # put one element just past a rounding threshold (inside the band): the GPU's
    # FP32 h may land on the other side, so the neighbouring code is accepted
    sc = oracle.ue4m3(int(s[1, 0])) * 2.0 ** -4
    m = abs(int(q[1, 5]))
    h2 = h.copy()
    h2[1, 5] = (m + 0.5) * sc * (1 + 2.0 ** -20)
    q2, s2 = oracle.quantize8(h2, 2.0 ** -4)
    assert np.array_equal(s2, s)
    g = q2.copy()
    g[1, 5] = q2[1, 5] - 1 if q2[1, 5] > 0 else q2[1, 5] + 1
    qa, _ = checker.check_h_codes8(h2, q2, s2, g, s2.copy(), 2.0 ** -4, rep)
    assert rep["h_flips"] == 1 and np.array_equal(qa, g)


def test_a8_h_code_flip_outside_band_rejected():
    h, q, s = _a8_case(1)
    g = q.copy()
    i = int(np.argmax(np.abs(q[2]) > 3))
    g[2, i] += 1 if g[2, i] < 127 else -1
    with pytest.raises(AssertionError):
        checker.check_h_codes8(h, q, s, g, s.copy(), 2.0 ** -4, checker.Report())


def test_output_straddle_verified_or_rejected():
    rng = np.random.default_rng(3)
    out64 = rng.standard_normal((2, 64)) * 10.0
    v32 = out64.astype(np.float32)
    o16 = oracle.round_bf16(out64)
    g = checker.f32_to_bf16_rne_bits(v32)
    rep = checker.Report()
    checker.check_output(g, out64, o16, rep, v32=v32)
    # a value just above a BF16 midpoint in FP64 and just below it in FP32: both
    # neighbours are correct roundings; the straddle is verified
    lo = np.float32(np.array([0x41200000], np.uint32).view(np.float32)[0])  # 10.0
    ulp = np.float64(2.0 ** -4)  # BF16 ulp at 10
    mid = float(lo) + ulp / 2
    out64[0, 0] = mid + 1e-9
    v32[0, 0] = np.float32(mid - 2.0 ** -20)
    o16 = oracle.round_bf16(out64)
    g = checker.f32_to_bf16_rne_bits(v32)
    assert g[0, 0] != o16[0, 0]
    checker.check_output(g, out64, o16, rep, v32=v32)
    assert rep["straddles"] >= 0
    # a BF16 output that is not the rounding of the kernel's own FP32 sum: rejected
    bad = g.copy()
    bad[1, 3] ^= 1
    with pytest.raises(AssertionError):
        checker.check_output(bad, out64, o16, checker.Report(), v32=v32)
    # an FP32 sum off by more than 1e-2 * RMS: rejected with no exemption
    v_bad = v32.copy()
    v_bad[1, 7] += np.float32(0.5)
    with pytest.raises(AssertionError):
        checker.check_output(checker.f32_to_bf16_rne_bits(v_bad), out64, o16, checker.Report(), v32=v_bad)

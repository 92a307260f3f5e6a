"""Split-K rounding check on one GPU: the down projection split into two halves of
I, as a two-way split of the experts would exchange partial sums (Richland article,
"Why it matters": partial sums exchanged in BF16 go wrong noticeably more often, FP16
with a power-of-two shift restores the unsplit behaviour).

Layer 0 of the 48-layer stack at 4,096 tokens (its RMS-normalised input).  The GPU
computes the two partial layer outputs out_A, out_B in FP32 (moe_expert_ffn_krange +
moe_combine_f32); they are checked against the oracle's partials.  Three ways to
finish the sum are then compared with the FP64 exact output on a token sample:
  unsplit     RNE_BF16(out_A + out_B), FP32 partials;
  split-BF16  RNE_BF16(bf16(out_A) + bf16(out_B));
  split-FP16  RNE_BF16(2^k f16(out_A 2^-k) + 2^k f16(out_B 2^-k)), k per tensor the
              smallest shift that keeps its largest magnitude within FP16's range.
A "large" error is above tau*|out| for tau in 2^-7, 2^-6, 2^-5, or above 2^-8 * RMS.
The pages fix only the direction (split-BF16 worse than unsplit, split-FP16 like it);
the size of the gap is parity unpinned.
"""
import numpy as np
import pytest
import torch

import gen
import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

T = 4096
N_SAMPLE = 128


def bf16_round_f32(v):
    """float32 array -> nearest-even BF16 values as float32 (finite inputs)."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def fp16_shifted(v, amax):
    k = max(0, int(np.ceil(np.log2(amax / 65504.0)))) if amax > 0 else 0
    s = np.float32(2.0 ** -k)
    h = np.clip(v * s, -65504, 65504).astype(np.float16).astype(np.float32)
    return h / s, k


def test_split_k_rounding():
    L = gen.make_layer(4, layer=0)
    DL = gh.device_layer(L)
    sh = L.shape
    x = oracle.rms_norm(gen.make_tokens(4, T, step=4096))
    xd = gh.to_dev(x.view(np.int16))
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_route(DL, xd, buf.topk_idx, buf.topk_w, buf.ws, T=T)
    moe.moe_permute(DL, buf.topk_idx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=T)
    half = sh.I // 32
    outs = {}
    for name, (kb0, kb1) in (("A", (0, half)), ("B", (half, 2 * half)), ("full", (0, 2 * half))):
        y = torch.empty_like(buf.y_rows)
        ys = torch.empty_like(buf.y_shared)
        moe.moe_expert_ffn_krange(DL, xd, buf.expert_off, buf.row2pair, kb0, kb1, y, ys, buf.ws, T=T)
        o = torch.empty((T, sh.H), dtype=torch.float32, device=gh.DEV)
        moe.moe_combine_f32(DL, y, ys, buf.pair2row, buf.topk_w, o, T=T)
        outs[name] = o
    torch.cuda.synchronize()
    A, B, F = (outs[n].cpu().numpy() for n in ("A", "B", "full"))
    assert np.isfinite(A).all() and np.isfinite(B).all()
    # the halves add up to the unsplit FP32 output (FP32 rounding apart)
    rms_f = float(np.sqrt((F.astype(np.float64) ** 2).mean()))
    assert float(np.abs(A.astype(np.float64) + B - F).max()) < 1e-5 * rms_f

    # oracle: exact partials and exact full output on a token sample, its own routing
    rng = np.random.default_rng(4096)
    tok = np.array(sorted(rng.choice(T, N_SAMPLE, replace=False)), np.int32)
    idx_g = buf.topk_idx.cpu().numpy()[tok]
    o_full = oracle.layer(L, x, tokens=tok)
    keep = np.all(o_full["idx"] == idx_g, axis=1)  # tokens whose routing agrees (near ties aside)
    assert keep.mean() > 0.95
    o_A = oracle.layer(L, x, tokens=tok, kb=(0, half))["out_f64"][keep]
    o_B = oracle.layer(L, x, tokens=tok, kb=(half, 2 * half))["out_f64"][keep]
    exact = o_full["out_f64"][keep]
    rows = tok[keep]
    for got, ref, name in ((A[rows], o_A, "A"), (B[rows], o_B, "B")):
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        gh.log("   partial %s: rel-L2 vs oracle %.2e" % (name, rel))
        assert rel < 2e-3

    a, b = A[rows], B[rows]
    a16, ka = fp16_shifted(a, float(np.abs(A).max()))
    b16, kb = fp16_shifted(b, float(np.abs(B).max()))
    variants = {
        "unsplit": bf16_round_f32(a + b),
        "split-BF16": bf16_round_f32(bf16_round_f32(a) + bf16_round_f32(b)),
        "split-FP16": bf16_round_f32(a16 + b16),
    }
    rms = float(np.sqrt((exact ** 2).mean()))
    rates = {}
    for name, v in variants.items():
        err = np.abs(v.astype(np.float64) - exact)
        r = {("tau=2^-%d" % e): float((err > 2.0 ** -e * np.abs(exact)).mean()) for e in (7, 6, 5)}
        r["2^-8*RMS"] = float((err > 2.0 ** -8 * rms).mean())
        rates[name] = r
        gh.log("   %-10s large-error rates %s" % (name, ", ".join("%s %.2e" % kv for kv in r.items())))
    gh.log("   FP16 shifts k_A=%d k_B=%d; tokens compared %d" % (ka, kb, len(rows)))
    u, s16, s8 = rates["unsplit"], rates["split-FP16"], rates["split-BF16"]
    assert s8["2^-8*RMS"] > u["2^-8*RMS"] and s8["tau=2^-7"] >= u["tau=2^-7"]
    assert s16["2^-8*RMS"] <= 1.5 * u["2^-8*RMS"] + 1e-3

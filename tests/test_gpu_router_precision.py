"""Reduced-precision prompt routers on the matrix cores, measured against exact
routing (capy-flash README v0.5.4, "Measured": moving the prompt router onto the
matrix units changes the order of its sums, so a near tie between two experts can
resolve the other way).

On the 15,360-token chunk (Zipf-skewed router), three routers pick the top 10 of
512 experts per token:
  exact   moe_route (FP64 sums of the exact products, refined near the k-th value);
  bf16    logits from BF16 x and BF16-rounded router rows, exact products
          summed in FP32 (torch matmul on the matrix cores);
  split3  the router rows split exactly into three BF16 pieces, three such
          products summed in FP32 (the arithmetic of the product's prompt router
          before its FP64 refinement).
A flip is a token whose selected set differs from the exact one.  The rates are
logged; the test asserts what the arithmetic fixes: split3 flips only on near
ties (FP64 margin below 1e-4 of the logit scale) and far less often than bf16.
The size of the bf16 rate is parity unpinned (the pages give none).
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

CFG = 3
T = 15360
N_EXACT_SAMPLE = 256


def split3(w):
    """FP32 -> three BF16 pieces (truncation) whose sum is exactly w."""
    u = w.view(torch.int32)
    w1 = (u & -65536).view(torch.float32)
    r1 = w - w1
    w2 = (r1.view(torch.int32) & -65536).view(torch.float32)
    w3 = r1 - w2
    return w1.bfloat16(), w2.bfloat16(), w3.bfloat16()


def test_router_flip_rates():
    L = gen.make_layer(CFG)
    DL = gh.device_layer(L, kmajor=False)
    x = gen.make_tokens(CFG, T)
    xd = gh.to_dev(x.view(np.int16))
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_route(DL, xd, buf.topk_idx, buf.topk_w, buf.ws, T=T)
    exact = torch.sort(buf.topk_idx.long(), dim=1).values
    # BF16-valued operands in FP32 matmuls: every product is exact and the sums
    # run in FP32 (a BF16 matmul would also round its output to BF16)
    torch.backends.cuda.matmul.allow_tf32 = False
    xf = xd.view(torch.bfloat16).float()
    W = DL.router_w
    k = DL.k
    logits = {"bf16": xf @ W.bfloat16().float().t().contiguous()}
    p1, p2, p3 = split3(W.contiguous())
    logits["split3"] = (xf @ p1.float().t().contiguous()) + (xf @ p2.float().t().contiguous()) + \
        (xf @ p3.float().t().contiguous())
    rates = {}
    for name, lg in logits.items():
        sel = torch.sort(torch.topk(lg, k, dim=1).indices, dim=1).values
        flips = torch.nonzero((sel != exact).any(dim=1)).flatten().cpu().numpy()
        rates[name] = (flips.size / T, flips)
        gh.log("   router %-6s: %d of %d tokens (%.2e) select another expert set" % (name, flips.size, T, flips.size / T))
    # split3 flips: near ties only, checked in FP64 by the oracle on those tokens
    f = rates["split3"][1]
    if f.size:
        l64 = oracle.router_logits(x[f], L.router_w)
        scale = np.abs(l64).max()
        for i, t in enumerate(f):
            srt = np.sort(l64[i])[::-1]
            assert srt[k - 1] - srt[k] < 1e-4 * scale, "token %d: split3 flip without a near tie" % t
    assert rates["split3"][0] <= rates["bf16"][0]
    assert rates["split3"][0] < 1e-2
    # the exact router agrees with the oracle on a sample (FP64 sums of exact products)
    s = np.random.default_rng(3).choice(T, N_EXACT_SAMPLE, replace=False)
    idx_o, _ = oracle.topk_softmax(oracle.router_logits(x[s], L.router_w), k)
    got = buf.topk_idx.cpu().numpy()[s]
    agree = np.mean([set(a) == set(b) for a, b in zip(got, idx_o)])
    gh.log("   exact router: %.4f of %d sampled tokens agree with the oracle" % (agree, N_EXACT_SAMPLE))
    assert agree > 0.99

"""GPU parity of the 48-layer stack: 48 decode-shaped layers with independent seeded
weights (43.8 GB resident at once), composed as
    n_l = RMSnorm(x_l),  x_{l+1} = RNE_BF16(x_l + MoE_l(n_l))
(the norm by moe_rms_norm, the residual added in the layer's combine).  Without the
norm the SwiGLU's quadratic growth makes the residual stream diverge within a few
layers.

The oracle runs its own chain from the generator's tokens (1 and 4 tokens, plus an
8-token sample for the 4,096-token chunk) and never sees a GPU result.  Teacher
forcing goes the other way: on layers 0, 1, 23 and 47 the GPU layer is run on the
oracle's input to that layer and checked with the full per-layer checker, so
near-tie flips and last-bit differences of earlier layers do not compound.  At
4,096 tokens the checked layer gets fresh generator tokens with the sampled rows
replaced by the oracle's chain state.  The GPU's own chains through all 48 layers
(1, 4 and 4,096 tokens) must stay finite and deterministic.  Free-running, the two
chains separate with depth (a near-tie expert choice or a last-bit difference in one
layer changes the next layer's input, and routing is discontinuous), so they are
compared only after the first layer (within the per-layer bar) and the divergence
at depth 48 is reported, with a loose bound that catches garbage.
"""
import time

import numpy as np
import pytest
import torch

import gen
import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

CFG = 4
N_LAYERS = 48
CHECK = (0, 1, 23, 47)
T_BIG = 4096
N_SAMPLE = 8


def gpu_chain(layers, x0, fused):
    """The stack on the GPU from x0; returns the final residual stream and the
    stream after the first layer."""
    T = x0.shape[0]
    buf = moe.Buffers(layers[0], T, gh.DEV)
    x = gh.to_dev(x0.view(np.int16))
    n = torch.empty_like(x)
    first = None
    for DL in layers:
        moe.moe_rms_norm(x, n)
        if fused:
            moe.moe_layer_forward(DL, n, buf, residual=x)
        else:
            moe.moe_forward(DL, n, buf, residual=x)
        x = buf.out.clone()
        if first is None:
            first = x
    torch.cuda.synchronize()
    return x, first


def oracle_step(Lh, x):
    n = oracle.rms_norm(x)
    return n, oracle.layer(Lh, n, residual=x)["out_bf16"]


def test_stack_teacher_forced():
    t0 = time.time()
    sample = np.array(sorted(np.random.default_rng(48).choice(T_BIG, N_SAMPLE, replace=False)), np.int32)
    x0 = {1: gen.make_tokens(CFG, 1, step=1), 4: gen.make_tokens(CFG, 4, step=4),
          T_BIG: gen.make_tokens(CFG, T_BIG, step=4096)}
    chain = {1: x0[1].copy(), 4: x0[4].copy(), "s": x0[T_BIG][sample].copy()}
    layers, kept, forced, after_first = [], {}, {}, {}
    for l in range(N_LAYERS):
        Lh = gen.make_layer(CFG, layer=l)
        layers.append(gh.device_layer(Lh))
        if l in CHECK:
            kept[l] = Lh
            forced[l] = {}
        for key in chain:
            n, nxt = oracle_step(Lh, chain[key])
            if l in CHECK:
                forced[l][key] = (n, chain[key])  # the layer's input and residual
            chain[key] = nxt
            if l == 0:
                after_first[key] = nxt
        del Lh
        if l % 8 == 7:
            gh.log("   stack: %d layers generated, uploaded and run by the oracle (%.0f s)" % (l + 1, time.time() - t0))

    # the GPU's own chains: finite, deterministic, close to the oracle's at 1 and 4 tokens
    for T in (1, 4, T_BIG):
        fused = T <= 4
        xa, fa = gpu_chain(layers, x0[T], fused)
        xb, _ = gpu_chain(layers, x0[T], fused)
        a = xa.cpu().numpy().view(np.uint16)
        assert np.array_equal(a, xb.cpu().numpy().view(np.uint16)), "stack run not deterministic at T=%d" % T
        af = oracle.bf16_to_f64(a)
        assert np.isfinite(af).all()
        if T <= 4:
            f1 = oracle.bf16_to_f64(fa.cpu().numpy().view(np.uint16))
            o1 = oracle.bf16_to_f64(after_first[T])
            rel1 = float(np.linalg.norm(f1 - o1) / np.linalg.norm(o1))
            o = oracle.bf16_to_f64(chain[T])
            rel = float(np.linalg.norm(af - o) / np.linalg.norm(o))
            gh.log("   stack T=%d: chains rel-L2 after layer 1 %.2e, after layer 48 %.2e (rms %.3f vs %.3f)" % (
                T, rel1, rel, np.sqrt((af ** 2).mean()), np.sqrt((o ** 2).mean())))
            assert rel1 < 2e-3, "first layer of the stack differs from the oracle's at T=%d" % T
            assert rel < 1.0 and 0.5 < np.sqrt((af ** 2).mean() / (o ** 2).mean()) < 2.0

    # teacher forcing: the checked layers on the oracle's inputs
    for l in CHECK:
        for T in (1, 4):
            n, x = forced[l][T]
            g = gh.run_layer(layers[l], n, residual=x, dump=("xq", "xs", "hq", "hs", "h"))
            rep = gh.check_layer(kept[l], n, g, residual=x)
            gh.log("   layer %d T=%d: %s" % (l, T, rep.line()))
        x = gen.make_tokens(CFG, T_BIG, step=5000 + l)
        x[sample] = forced[l]["s"][1]
        n = oracle.rms_norm(x)
        n[sample] = forced[l]["s"][0]
        g = gh.run_layer(layers[l], n, residual=x)
        rep = gh.check_layer(kept[l], n, g, tokens=sample, residual=x)
        gh.log("   layer %d T=%d (sampled rows at depth %d): %s" % (l, T_BIG, l, rep.line()))
    gh.log("   stack test %.0f s" % (time.time() - t0))

"""GPU parity of the layer's variants against the FP64 oracle:

  * the optional shared-expert gate (a reading: the pages print none; per token
    g = fl32(sigmoid(x . w_g)), the shared expert's rows times g) on the decode,
    weight-streaming, matrix-core and generic kernels, and through the fused
    decode call, which must equal the separate calls bit for bit;
  * the reduced-precision prompt routers (capy-flash README v0.5.4, "Measured":
    a router on the matrix units sums in another order and may resolve a near
    tie differently): MOE_ROUTER_SPLIT3_F32 and MOE_ROUTER_BF16, each against
    the oracle's top k on that router's own FP64 logits within the kernel's
    proven FP32 error radius, and their flip rates against the exact routing on
    the 15,360-token chunk (the rates are logged; their size is parity unpinned,
    the pages give none);
  * the router's BF16 pieces written once per layer (moe_pack_router): the exact
    router gives identical results with and without them.
"""
import numpy as np
import pytest
import torch

import checker
import gen
import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

ODD = gen.Shape(H=288, E=24, k=3, I=96)
_layers = {}


def gated_layer(name, cfg, shape=None):
    if name not in _layers:
        L = gen.make_layer(cfg, shape=shape, shared_gate=True)
        _layers[name] = (L, gh.device_layer(L))
    return _layers[name]


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), dtype=np.int32)


# decode kernels (T <= 4), weight streaming (20), matrix cores (300), generic (odd shape)
@pytest.mark.parametrize("name,cfg,T", [("c0", 0, 8), ("c1", 1, 1), ("c1", 1, 4), ("c1", 1, 20), ("c1", 1, 300),
                                        ("odd", 0, 20)])
def test_shared_gate_layer(name, cfg, T):
    gh.log("case: shared-expert gate %s T=%d" % (name, T))
    L, DL = gated_layer(name, cfg, ODD if name == "odd" else None)
    x = gen.make_tokens(cfg, T, step=61, H=L.shape.H)
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs"))
    gate = oracle.shared_gate(x, L.shared_gate_w)
    assert gate.min() < 0.45 and gate.max() > 0.55 or T < 4  # the gate really varies
    rep = gh.check_layer(L, x, g, tokens=None if T <= 64 else sample_tokens(T, 40, T))
    gh.log("  ", rep.line())


@pytest.mark.parametrize("T", [1, 3, 4])
def test_shared_gate_fused_matches_separate_calls(T):
    gh.log("case: shared-expert gate, fused decode call T=%d" % T)
    L, DL = gated_layer("c1", 1)
    x = gen.make_tokens(1, T, step=62)
    res = gen.make_tokens(1, T, step=63)
    ref = gh.run_layer(DL, x, residual=res, dump=())
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf, residual=gh.to_dev(res.view(np.int16)))
    torch.cuda.synchronize()
    assert np.array_equal(buf.y_shared.cpu().numpy(), ref["y_shared"])
    assert np.array_equal(buf.out.cpu().numpy().view(np.uint16), ref["out"])
    assert np.array_equal(buf.topk_idx.cpu().numpy(), ref["idx"])


def _mode_logits_and_radius(L, x, mode):
    """The oracle's FP64 logits of the router a mode computes, and the kernel's
    worst-case FP32 error radius gamma_d * sum_h |x_h w_eh| per logit."""
    W = L.router_w
    if mode == moe.MOE_ROUTER_BF16:
        W = (oracle.round_bf16(W.astype(np.float64)).astype(np.uint32) << 16).view(np.float32)
    lg = oracle.router_logits(x, W)
    xf = np.abs(oracle.bf16_to_f64(x))
    H = x.shape[1]
    pieces = 1 if mode == moe.MOE_ROUTER_BF16 else 3
    d = pieces * 2 * 16 + 8 + (H // 32 + 7) // 8  # additions on the longest path of the matrix-core sums
    u = 2.0 ** -23
    gamma = 1.01 * d * u / (1 - d * u) * (1 + 2.0 ** -6)
    rad = gamma * (xf @ np.abs(W.astype(np.float64)).T)
    return lg, rad


@pytest.mark.parametrize("mode", ["split3", "bf16"])
@pytest.mark.parametrize("T", [4, 300])
def test_reduced_router_parity(mode, T):
    m = {"split3": moe.MOE_ROUTER_SPLIT3_F32, "bf16": moe.MOE_ROUTER_BF16}[mode]
    gh.log("case: router mode %s T=%d" % (mode, T))
    L = gen.make_layer(1)
    DL = gh.device_layer(L).with_router_mode(m)
    x = gen.make_tokens(1, T, step=64)
    xd = gh.to_dev(x.view(np.int16))
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_route(DL, xd, buf.topk_idx, buf.topk_w, buf.ws, T=T)
    torch.cuda.synchronize()
    lg, rad = _mode_logits_and_radius(L, x, m)
    rep = checker.Report()
    checker.check_topk_radius(buf.topk_idx.cpu().numpy(), buf.topk_w.cpu().numpy(), lg, rad, L.shape.k, rep)
    gh.log("  ", rep.line())
    # the whole layer with this router: the rest of the layer checked on its selection
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs"))
    assert np.array_equal(g["idx"], buf.topk_idx.cpu().numpy())


def test_router_flip_rates_long_prefill():
    """Flip rates of the two reduced routers against the exact routing on the
    15,360-token Zipf chunk, through the library's own kernels."""
    T = 15360
    L = gen.make_layer(3)
    DL = gh.device_layer(L, kmajor=False)
    x = gen.make_tokens(3, T)
    xd = gh.to_dev(x.view(np.int16))
    sel = {}
    for name, m in (("exact", moe.MOE_ROUTER_EXACT), ("split3", moe.MOE_ROUTER_SPLIT3_F32),
                    ("bf16", moe.MOE_ROUTER_BF16)):
        gh.log("case: router flip rates, mode %s" % name)
        buf = moe.Buffers(DL, T, gh.DEV)
        moe.moe_route(DL.with_router_mode(m), xd, buf.topk_idx, buf.topk_w, buf.ws, T=T)
        torch.cuda.synchronize()
        sel[name] = (buf.topk_idx.cpu().numpy(), buf.topk_w.cpu().numpy())
        del buf
    exact_lg = oracle.router_logits(x, L.router_w)
    idx_o, _ = oracle.topk_softmax(exact_lg, L.shape.k)
    sets = lambda a: np.sort(a, axis=1)
    rates = {n: float((sets(v[0]) != sets(idx_o)).any(axis=1).mean()) for n, v in sel.items()}
    gh.log("   flip rates against the exact FP64 selection on %d tokens: %s" % (
        T, ", ".join("%s %.4f" % kv for kv in rates.items())))
    assert rates["exact"] == 0.0 and np.array_equal(sel["exact"][0], idx_o)
    rep = checker.Report()
    lg, rad = _mode_logits_and_radius(L, x, moe.MOE_ROUTER_SPLIT3_F32)
    checker.check_topk_radius(sel["split3"][0], sel["split3"][1], lg, rad, L.shape.k, rep)
    lg, rad = _mode_logits_and_radius(L, x, moe.MOE_ROUTER_BF16)
    checker.check_topk_radius(sel["bf16"][0], sel["bf16"][1], lg, rad, L.shape.k, rep)
    assert rates["split3"] < 1e-3 and rates["bf16"] > rates["split3"]


@pytest.mark.parametrize("cfg,T", [(1, 300), (3, 15360)])
def test_cached_router_pieces(cfg, T):
    gh.log("case: cached router pieces config %d T=%d" % (cfg, T))
    L = gen.make_layer(cfg)
    DL = gh.device_layer(L, kmajor=False)
    x = gh.to_dev(gen.make_tokens(cfg, T, step=65).view(np.int16))
    a = moe.Buffers(DL, T, gh.DEV)
    moe.moe_route(DL, x, a.topk_idx, a.topk_w, a.ws, T=T)
    DL.pack_router()
    b = moe.Buffers(DL, T, gh.DEV)
    moe.moe_route(DL, x, b.topk_idx, b.topk_w, b.ws, T=T)
    torch.cuda.synchronize()
    assert torch.equal(a.topk_idx, b.topk_idx) and torch.equal(a.topk_w, b.topk_w)
    # the pieces are the exact truncation split of every router weight
    p = DL.router_pieces.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    s = p.view(np.float32).astype(np.float64).sum(axis=0)
    assert np.array_equal(s, L.router_w.astype(np.float64))
    assert np.array_equal(p[0] >> 16, L.router_w.view(np.uint32) >> 16)

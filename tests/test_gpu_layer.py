"""GPU parity of the whole layer (route -> permute -> expert FFN -> combine) through
the C ABI, against the FP64 oracle on the same seeded inputs.

Sizes: the tiny layer in full; the decode layer at 1 and 4 tokens in full; a
ragged token count that spans several permutation chunks; the 4,096- and
15,360-token prefill chunks with Zipf-skewed routing on sampled tokens (every
token's routing, permutation and A4(x) are still checked in full); the
15,360-token tie-stress variant; degenerate inputs.
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

_layers = {}


def layer_for(cfg):
    if cfg not in _layers:
        L = gen.make_layer(cfg)
        _layers[cfg] = (L, gh.device_layer(L))
    return _layers[cfg]


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), dtype=np.int32)


# expert FFN paths: decode kernels (T <= 4), weight streaming (5..31 tokens),
# matrix cores (T >= 32; the tiny shape takes 4 and 2 K steps)
@pytest.mark.parametrize("cfg,T", [(0, 8), (1, 1), (1, 4), (1, 20), (1, 257), (0, 33), (0, 300)])
def test_layer_full(cfg, T):
    gh.log("case: config %d T=%d" % (cfg, T))
    L, DL = layer_for(cfg)
    x = gen.make_tokens(cfg, T, step=0 if T not in (257, 300) else 7)
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs", "h"))
    rep = gh.check_layer(L, x, g, tokens=None if T <= 64 else sample_tokens(T, 48, T))
    gh.log("  ", rep.line())


@pytest.mark.parametrize("cfg,T", [(2, 4096), (3, 15360)])
def test_layer_prefill_sampled(cfg, T):
    gh.log("case: config %d T=%d (Zipf routing)" % (cfg, T))
    L, DL = layer_for(cfg)
    x = gen.make_tokens(cfg, T)
    g = gh.run_layer(DL, x)
    counts = np.diff(g["off"])
    gh.log("   expert load: max %d min %d (head share %.3f)" % (counts.max(), counts.min(), counts.max() / T))
    rep = gh.check_layer(L, x, g, tokens=sample_tokens(T, 40, cfg))
    gh.log("  ", rep.line())


def tie_stress_inputs(L, x, n_pairs=32, frac=0.01, seed=99):
    """Twin router rows that agree except on the last 16 coordinates; chosen tokens get
    x = 0 there, so the twins' logits are exactly equal and sit at ranks k and k+1."""
    sh = L.shape
    H, E, k = sh.H, sh.E, sh.k
    rng = np.random.default_rng(seed)
    wr = L.router_w.copy()
    ids = rng.permutation(E)[:2 * n_pairs]
    pairs = [(int(ids[2 * i]), int(ids[2 * i + 1])) for i in range(n_pairs)]
    for a, b in pairs:
        wr[b, :H - 16] = wr[a, :H - 16]
    x0 = x.copy()
    x0[:, H - 16:] = 0
    lg = oracle.router_logits(x0, wr)
    cand = []
    for t in range(x.shape[0]):
        for a, b in pairs:
            v = lg[t, a]
            assert v == lg[t, b]
            if (lg[t] > v).sum() == k - 1:
                cand.append((t, a, b))
                break
    rng.shuffle(cand)
    chosen = cand[:int(round(frac * x.shape[0]))]
    xt = x.copy()
    for t, _, _ in chosen:
        xt[t, H - 16:] = 0
    return wr, xt, chosen


def test_layer_tie_stress_long_prefill():
    cfg, T = 3, 15360
    gh.log("case: config 3 tie-stress T=%d" % T)
    L, _ = layer_for(cfg)
    x = gen.make_tokens(cfg, T, step=1)
    wr, xt, chosen = tie_stress_inputs(L, x)
    assert len(chosen) == 154, len(chosen)
    DLt = gh.device_layer(L, router_w=wr)
    g = gh.run_layer(DLt, xt)
    for t, a, b in chosen:
        assert min(a, b) in g["idx"][t] and max(a, b) not in g["idx"][t], (t, a, b, g["idx"][t])
    import copy
    Lt = copy.copy(L)
    Lt.router_w = wr
    tok = np.array(sorted({t for t, _, _ in chosen[:24]} | set(sample_tokens(T, 16, 5).tolist())), np.int32)
    rep = gh.check_layer(Lt, xt, g, tokens=tok)
    gh.log("  ", rep.line(), "tied tokens:", len(chosen))


def test_route_injected_duplicate_logits():
    """logits_in with exact duplicates at every rank 1..11: lower id first, bit-exact."""
    L, DL = layer_for(1)
    E, k = L.shape.E, L.shape.k
    rng = np.random.default_rng(4)
    T = 300
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for t in range(T):
        order = np.argsort(-lg[t], kind="stable")
        r = t % 11
        lg[t, order[r + 1]] = lg[t, order[r]]  # duplicate at rank r / r+1
    lg[:20] = 0.5  # all equal
    lg[20:25, :] = -1.0
    lg[20:25, 100:110] = 2.0  # a block of equal winners
    idx = torch.empty((T, k), dtype=torch.int32, device=gh.DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=gh.DEV)
    moe.moe_route(DL, None, idx, w, None, logits_in=gh.to_dev(lg), T=T)
    torch.cuda.synchronize()
    idx_o, w_o = oracle.topk_softmax(lg.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), idx_o)
    assert np.allclose(w.cpu().numpy(), w_o, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("kind", ["one_expert", "k_equals_E", "ragged_many_chunks"])
def test_permute_adversarial(kind):
    E = 32 if kind == "k_equals_E" else 512
    k = E if kind == "k_equals_E" else (1 if kind == "one_expert" else 10)
    DL = moe.MoELayer(256, 128, E, k, torch.empty(1, device=gh.DEV), None, None)
    T = {"one_expert": 5000, "k_equals_E": 300, "ragged_many_chunks": 15361}[kind]
    rng = np.random.default_rng(T)
    if kind == "one_expert":
        idx = np.full((T, 1), 137, np.int32)
    elif kind == "k_equals_E":
        idx = np.array([rng.permutation(E) for _ in range(T)], np.int32)
    else:
        idx = np.array([rng.choice(E, size=k, replace=False) for _ in range(T)], np.int32)
    d_idx = gh.to_dev(idx)
    off = torch.empty(E + 1, dtype=torch.int32, device=gh.DEV)
    r2p = torch.empty(T * k, dtype=torch.int32, device=gh.DEV)
    p2r = torch.empty(T * k, dtype=torch.int32, device=gh.DEV)
    ws = DL.workspace(T, gh.DEV)
    moe.moe_permute(DL, d_idx, off, r2p, p2r, ws, T=T)
    torch.cuda.synchronize()
    checker.check_permutation(idx, E, off.cpu().numpy(), r2p.cpu().numpy(), p2r.cpu().numpy())


def test_zero_input_and_residual():
    L, DL = layer_for(1)
    T = 4
    x = np.zeros((T, L.shape.H), np.uint16)
    g = gh.run_layer(DL, x)
    assert np.all((g["out"] & 0x7FFF) == 0)
    res = gen.make_tokens(1, T, step=11)
    g2 = gh.run_layer(DL, x, residual=res)
    assert np.array_equal(g2["out"], res)


def test_residual_path_parity():
    L, DL = layer_for(0)
    x = gen.make_tokens(0, 8, step=2)
    res = gen.make_tokens(0, 8, step=3)
    g = gh.run_layer(DL, x, residual=res)
    rep = gh.check_layer(L, x, g, residual=res)
    gh.log("  ", rep.line())


def test_determinism_and_equivariance():
    L, DL = layer_for(1)
    T = 64
    x = gen.make_tokens(1, T, step=5)
    x[40] = x[3]  # a duplicated token
    a = gh.run_layer(DL, x)
    b = gh.run_layer(DL, x)
    for key in ("idx", "w", "off", "r2p", "p2r", "y_rows", "out", "hq", "hs"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["out"][40], a["out"][3])
    perm = np.random.default_rng(2).permutation(T)
    c = gh.run_layer(DL, x[perm])
    assert np.array_equal(c["out"], a["out"][perm])


def test_quantize_act_exhaustive_bf16():
    """Every finite BF16 value under every nonzero scale (blocks whose amax pins the
    scale), GPU moe_quantize_act vs the oracle, bit-exact."""
    b = np.arange(1 << 16, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    vals = f[np.isfinite(f)]
    blocks = []
    for c in range(1, 127):
        s = np.float32(oracle.ue4m3(c))
        v = vals[np.abs(vals) <= 6 * s]
        v = np.concatenate([v, np.zeros((-len(v)) % 15, np.float32)]).reshape(-1, 15)
        blocks.append(np.concatenate([np.full((v.shape[0], 1), 6 * s, np.float32), v], axis=1))
    blk = np.concatenate(blocks).astype(np.float32)
    bits = (blk.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), blk)
    rows = blk.shape[0]
    codes = torch.empty((rows, 8), dtype=torch.uint8, device=gh.DEV)
    scales = torch.empty((rows, 1), dtype=torch.uint8, device=gh.DEV)
    moe.moe_quantize_act(gh.to_dev(bits.view(np.int16)), codes, scales)
    torch.cuda.synchronize()
    qo, so = oracle.quantize(blk.astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), so)
    assert np.array_equal(codes.cpu().numpy(), qo)


@pytest.mark.parametrize("g", [1.0, 0.125, 16.0])
def test_quantize_act_fp32_thresholds(g):
    """FP32 inputs at and next to every scale and code threshold, plus random values."""
    rng = np.random.default_rng(int(g * 8))
    pts = []
    for c in range(126):
        m = np.float32(6 * g * 0.5 * (oracle.ue4m3(c) + oracle.ue4m3(c + 1)))
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(np.inf))]
    amax = np.array(pts, np.float32)
    n = amax.shape[0]
    blk = (rng.uniform(-1, 1, (n, 16)) * amax[:, None]).astype(np.float32)
    blk[:, 3] = amax * np.where(rng.random(n) < 0.5, 1, -1).astype(np.float32)
    s = np.array([oracle.ue4m3(oracle.scale_code(float(a), g)) * g for a in amax], np.float32)
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for j in range(7):  # element thresholds and neighbours in columns 4..15
        blk[:, 4 + j] = t[j] * s
        if j < 4:
            blk[:, 11 + j] = np.nextafter(t[j] * s, np.float32(np.inf))
    rnd = (rng.standard_normal((4000, 16)) * np.exp2(rng.uniform(-12, 8, (4000, 1)))).astype(np.float32)
    blk = np.concatenate([blk, rnd])
    rows = blk.shape[0]
    codes = torch.empty((rows, 8), dtype=torch.uint8, device=gh.DEV)
    scales = torch.empty((rows, 1), dtype=torch.uint8, device=gh.DEV)
    moe.moe_quantize_act(gh.to_dev(blk), codes, scales, gscale=g)
    torch.cuda.synchronize()
    qo, so = oracle.quantize(blk.astype(np.float64), g)
    assert np.array_equal(scales.cpu().numpy(), so)
    assert np.array_equal(codes.cpu().numpy(), qo)


@pytest.mark.parametrize("cfg,T", [(1, 1), (1, 2), (1, 4), (0, 4), (0, 8), (1, 7)])
def test_layer_forward_matches_separate_calls(cfg, T):
    """moe_layer_forward (fused decode kernels for T <= 4) writes exactly what the four
    separate calls write; the separate calls are checked against the oracle above."""
    gh.log("case: moe_layer_forward config %d T=%d" % (cfg, T))
    L, DL = layer_for(cfg)
    x = gen.make_tokens(cfg, T, step=13)
    res = gen.make_tokens(cfg, T, step=14)
    ref = gh.run_layer(DL, x, residual=res, dump=())
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf, residual=gh.to_dev(res.view(np.int16)))
    torch.cuda.synchronize()
    got = {"idx": buf.topk_idx, "w": buf.topk_w, "off": buf.expert_off, "r2p": buf.row2pair, "p2r": buf.pair2row,
           "y_rows": buf.y_rows, "y_shared": buf.y_shared, "out": buf.out}
    for key, t in got.items():
        a = t.cpu().numpy()
        b = ref[key]
        if key == "out":
            a = a.view(np.uint16)
        assert np.array_equal(a, b), key
    rep = gh.check_layer(L, x, dict(ref, **gh.run_layer(DL, x, residual=res)), residual=res)
    gh.log("  ", rep.line())


@pytest.mark.parametrize("T", [1, 4])
def test_fused_decode_exact_ties(T):
    """Router rows duplicated so that exactly equal FP64 logits sit inside every
    token's top k (the experts at ranks 0 and 3 get a twin) and at its boundary
    (the expert at rank k - 3 and its twin end up at ranks k - 1 and k).
    In the fused decode call every routed gate/up workgroup finds its (token,
    rank) pair's expert by itself; it must take the lower id first, exactly as
    the publishing workgroup and the separate calls do, and match the oracle."""
    import copy
    cfg = 1
    L, _ = layer_for(cfg)
    sh = L.shape
    x = gen.make_tokens(cfg, T, step=41)
    res = gen.make_tokens(cfg, T, step=42)
    gh.log("case: fused decode exact ties T=%d" % T)
    lg = oracle.router_logits(x, L.router_w)
    order = np.argsort(-lg, axis=1, kind="stable")
    busy = set(order[:, :sh.k + 6].reshape(-1).tolist())
    spare = [e for e in range(sh.E) if e not in busy]
    rng = np.random.default_rng(7)
    wr = L.router_w.copy()
    twins = []
    for t in range(T):
        for r in (0, 3, sh.k - 3):
            a = int(order[t, r])
            if any(a in tw for tw in twins):
                continue
            b = spare.pop(int(rng.integers(len(spare))))
            wr[b] = wr[a]
            twins.append((a, b))
    DLt = gh.device_layer(L, router_w=wr)
    ref = gh.run_layer(DLt, x, residual=res, dump=())
    buf = moe.Buffers(DLt, T, gh.DEV)
    moe.moe_layer_forward(DLt, gh.to_dev(x.view(np.int16)), buf, residual=gh.to_dev(res.view(np.int16)))
    torch.cuda.synchronize()
    got = {"idx": buf.topk_idx, "w": buf.topk_w, "off": buf.expert_off, "r2p": buf.row2pair, "p2r": buf.pair2row,
           "y_rows": buf.y_rows, "y_shared": buf.y_shared, "out": buf.out}
    for key, tns in got.items():
        a_ = tns.cpu().numpy()
        if key == "out":
            a_ = a_.view(np.uint16)
        assert np.array_equal(a_, ref[key]), key
    lg2 = oracle.router_logits(x, wr)
    n_inside = n_boundary = 0
    for t in range(T):
        sel = ref["idx"][t].tolist()
        for a, b in twins:
            assert lg2[t, a] == lg2[t, b]
            lo, hi = min(a, b), max(a, b)
            if hi in sel:
                assert lo in sel and sel.index(lo) == sel.index(hi) - 1, (t, a, b, sel)
                n_inside += 1
            elif lo in sel:
                n_boundary += sel.index(lo) == sh.k - 1
    assert n_inside >= 2 * T and n_boundary >= T, (n_inside, n_boundary)
    Lt = copy.copy(L)
    Lt.router_w = wr
    rep = gh.check_layer(Lt, x, dict(ref, **gh.run_layer(DLt, x, residual=res)), residual=res)
    gh.log("  ", rep.line(), "tied pairs inside the top k:", n_inside, "at the boundary:", n_boundary)


@pytest.mark.parametrize("cfg,T", [(1, 4), (0, 3)])
def test_fused_path_repeated_calls(cfg, T):
    """Several fused calls on one workspace and one set of outputs: every call
    routes its own batch and matches the four separate calls on that batch."""
    gh.log("case: fused workspace reuse config %d T=%d" % (cfg, T))
    L, DL = layer_for(cfg)
    buf = moe.Buffers(DL, T, gh.DEV)
    for step in (21, 22, 23):
        x = gen.make_tokens(cfg, T, step=step)
        ref = gh.run_layer(DL, x, dump=())
        moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf)
        torch.cuda.synchronize()
        assert np.array_equal(buf.topk_idx.cpu().numpy(), ref["idx"])
        assert np.array_equal(buf.out.cpu().numpy().view(np.uint16), ref["out"])


def test_rms_norm_matches_oracle():
    """The stack's RMS norm kernel: bit-exact against the FP64 oracle (both round an
    FP64 product once to BF16), on decode-sized and ragged batches."""
    for T, H, step in ((4, 2048, 31), (257, 2048, 32), (8, 256, 33)):
        x = gen.make_tokens(1, T, step=step)[:, :H].copy()
        x[0] = oracle.round_bf16(oracle.bf16_to_f64(x[0]) * 37.0)
        out = torch.empty((T, H), dtype=torch.int16, device=gh.DEV)
        moe.moe_rms_norm(gh.to_dev(x.view(np.int16)), out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle.rms_norm(x)), (T, H)


def test_pack_kmajor_layout():
    """moe_pack_kmajor is the byte permutation its header states (checked on the
    host copy of the tiny layer's banks)."""
    L, _ = layer_for(0)
    for bank in (L.w13, L.w2):
        codes, scales = bank["codes"], bank["scales"]
        n_exp, N, K = codes.shape[0], codes.shape[1], codes.shape[2] * 2
        c_out = torch.empty(codes.size, dtype=torch.uint8, device=gh.DEV)
        s_out = torch.empty(scales.size, dtype=torch.uint8, device=gh.DEV)
        moe.moe_pack_kmajor(gh.to_dev(codes), gh.to_dev(scales), n_exp, N, K, c_out, s_out)
        torch.cuda.synchronize()
        S = K // 64
        want_c = codes.reshape(n_exp, N, S, 32).transpose(0, 2, 1, 3).reshape(-1)
        want_s = scales.reshape(n_exp, N, S, 4).transpose(0, 2, 1, 3).reshape(-1)
        assert np.array_equal(c_out.cpu().numpy(), want_c)
        assert np.array_equal(s_out.cpu().numpy(), want_s)


@pytest.mark.parametrize("cfg,T", [(0, 300), (2, 4096)])
def test_kmajor_copies_give_identical_results(cfg, T):
    """The matrix-core kernels read the row-major banks or their K-step-major copies
    with the same arithmetic: every output is bit-identical (also with the routed
    banks in one layout and the shared banks in the other), and so is the split-K
    partial of the down projection."""
    gh.log("case: config %d T=%d, row-major vs K-step-major weights" % (cfg, T))
    L, DLk = layer_for(cfg)
    assert DLk.desc.w13k.codes is not None
    DLr = gh.device_layer(L, kmajor=False)
    # routed banks K-step-major, shared banks row-major (the matrix-core
    # kernels that take one layout for both are then not used)
    DLm = gh.device_layer(L)
    DLm.desc.sh13k = moe.Bank()
    DLm.desc.sh2k = moe.Bank()
    x = gen.make_tokens(cfg, T, step=11)
    a = gh.run_layer(DLr, x, dump=("hq", "hs"))
    b = gh.run_layer(DLk, x, dump=("hq", "hs"))
    m = gh.run_layer(DLm, x, dump=("hq", "hs"))
    for key in ("y_rows", "y_shared", "out", "hq", "hs"):
        assert np.array_equal(a[key], b[key]), key
        assert np.array_equal(m[key], b[key]), key
    half = L.shape.I // 32
    xd = gh.to_dev(x.view(np.int16))
    outs = []
    for DL in (DLr, DLk):
        buf = moe.Buffers(DL, T, gh.DEV)
        moe.moe_route(DL, xd, buf.topk_idx, buf.topk_w, buf.ws, T=T)
        moe.moe_permute(DL, buf.topk_idx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=T)
        moe.moe_expert_ffn_krange(DL, xd, buf.expert_off, buf.row2pair, half, 2 * half, buf.y_rows, buf.y_shared,
                                  buf.ws, T=T)
        torch.cuda.synchronize()
        outs.append((buf.y_rows.cpu().numpy(), buf.y_shared.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("first", [0, 502])
def test_layer_all_tokens_on_ten_experts(first):
    """Routing forced through logits_in: every token picks experts first..first+9
    (weights of logits 8, 7, ..., -1), so each of the ten segments holds all 4,096
    rows (32 row tiles of one expert) next to the shared expert's; first = 502
    puts the last expert id, 511, in play.  Sampled tokens against the oracle."""
    cfg, T = 2, 4096
    gh.log("case: config %d T=%d, all tokens on experts %d..%d" % (cfg, T, first, first + 9))
    L, DL = layer_for(cfg)
    E, k = L.shape.E, L.shape.k
    lg = np.full((T, E), -100.0, np.float32)
    lg[:, first:first + k] = np.arange(8, 8 - k, -1, dtype=np.float32)
    x = gen.make_tokens(cfg, T, step=88)
    g = gh.run_layer(DL, x, logits_in=lg)
    counts = np.diff(g["off"])
    assert np.all(counts[first:first + k] == T) and counts.sum() == T * k
    rep = gh.check_layer(L, x, g, tokens=sample_tokens(T, 32, first), logits64=lg.astype(np.float64))
    gh.log("  ", rep.line())


@pytest.mark.parametrize("T", [2, 4])
def test_decode_identical_tokens_share_every_expert(T):
    """T identical tokens at decode: every selected expert serves all T rows (the
    multi-row paths of the slot table and of the decode kernels).  The fused call
    equals the four separate calls bit for bit, every token's output is the same,
    and the separate calls are checked against the oracle."""
    gh.log("case: config 1, %d identical tokens" % T)
    L, DL = layer_for(1)
    x = np.repeat(gen.make_tokens(1, 1, step=91), T, axis=0)
    ref = gh.run_layer(DL, x)
    assert np.all(np.diff(ref["off"])[np.diff(ref["off"]) > 0] == T)
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf)
    torch.cuda.synchronize()
    out = buf.out.cpu().numpy().view(np.uint16)
    assert np.array_equal(out, ref["out"]) and np.array_equal(buf.topk_idx.cpu().numpy(), ref["idx"])
    assert all(np.array_equal(out[t], out[0]) for t in range(T))
    rep = gh.check_layer(L, x, ref)
    gh.log("  ", rep.line())


@pytest.mark.parametrize("T", [4, 20, 300])
def test_layer_activation_global_scales(T):
    """Power-of-two activation global scales (x encoded under 2^-2, h under 2^3)
    on the decode (fused call), weight-streaming and matrix-core paths, against
    the oracle under the same scales."""
    import dataclasses
    gh.log("case: config 1 T=%d, a_gscale_in 0.25, a_gscale_mid 8" % T)
    L = dataclasses.replace(gen.make_layer(1), a_gscale_in=0.25, a_gscale_mid=8.0)
    DL = gh.device_layer(L)
    x = gen.make_tokens(1, T, step=93)
    g = gh.run_layer(DL, x)
    rep = gh.check_layer(L, x, g, tokens=None if T <= 64 else sample_tokens(T, 32, T))
    gh.log("  ", rep.line())
    if T <= 4:
        buf = moe.Buffers(DL, T, gh.DEV)
        moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf)
        torch.cuda.synchronize()
        assert np.array_equal(buf.out.cpu().numpy().view(np.uint16), g["out"])


@pytest.mark.parametrize("T", [4, 20, 300])
def test_layer_without_shared_expert(T):
    """No shared expert (has_shared = 0, y_shared null): the decode (fused call and
    separate calls), weight-streaming and matrix-core paths against the oracle."""
    import dataclasses
    gh.log("case: config 1 T=%d without the shared expert" % T)
    L = dataclasses.replace(gen.make_layer(1), sh13=None, sh2=None)
    DL = gh.device_layer(L)
    assert DL.has_shared == 0
    x = gen.make_tokens(1, T, step=95)
    g = gh.run_layer(DL, x)
    rep = gh.check_layer(L, x, g, tokens=None if T <= 64 else sample_tokens(T, 32, T))
    gh.log("  ", rep.line())
    if T <= 4:
        buf = moe.Buffers(DL, T, gh.DEV)
        moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf)
        torch.cuda.synchronize()
        assert np.array_equal(buf.out.cpu().numpy().view(np.uint16), g["out"])


@pytest.mark.parametrize("variant", ["w4a4", "w4a8", "gate"])
@pytest.mark.parametrize("cfg,T", [(1, 1), (1, 2), (1, 4), (0, 3), (1, 7), (1, 300)])
def test_pre_norm_matches_norm_then_layer(cfg, T, variant):
    """pre_norm: moe_layer_forward on x with the norm inside (fused decode: in the router
    kernel; otherwise the norm kernel first) writes exactly what moe_rms_norm followed by
    moe_layer_forward writes, with the residual x added in both."""
    gh.log("case: pre_norm config %d T=%d %s" % (cfg, T, variant))
    L, DL = layer_for(cfg)
    if variant == "w4a8":
        DL = DL.with_act_bits(8)
    elif variant == "gate":
        wg = gen.normal_f32_rows(gen.stream_key(gen.BASE_SEED, cfg, 0, gen.TENSOR_SHGATE), np.array([0.02]), L.shape.H)[0]
        DL = DL.with_shared_gate(gh.to_dev(wg))
    x = gh.to_dev(gen.make_tokens(cfg, T, step=51).view(np.int16))
    eps = 1e-6
    ref = moe.Buffers(DL, T, gh.DEV)
    n = torch.empty_like(x)
    moe.moe_rms_norm(x, n, eps=eps)
    moe.moe_layer_forward(DL, n, ref, residual=x)
    DN = DL.with_pre_norm(eps)
    got = moe.Buffers(DN, T, gh.DEV)
    moe.moe_layer_forward(DN, x, got, residual=x)
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_w", "expert_off", "row2pair", "pair2row", "y_rows", "y_shared", "out"):
        a, b = getattr(got, key).cpu().numpy(), getattr(ref, key).cpu().numpy()
        assert np.array_equal(a, b), key

"""GPU parity, against the FP64 oracle, of the kernels that only unusual shapes
reach (every kernel the library can launch is compared with the oracle somewhere):

  * a hidden size that is not a multiple of 256 and an intermediate size whose
    32-column chunk count is not a power of two (H 288, I 96, E 24, k 3): the
    generic expert kernels (k_ffn_gateup, k_ffn_down) at 3, 20 and 300 tokens,
    the tiled FP32 router pass with the general selection kernel, and K-split
    partials of the down projection on the generic kernels;
  * K-split partials on the matrix-core path (H 2048, I 512, 40 tokens) over 3, 1
    and 5 K steps per tile: the chained down kernel at each of its three ring
    phase patterns (steps mod 3 = 0 and 2 here, 1 in the split-K rounding check)
    and the one-item kernel for a single step;
  * more than 512 experts: 1,024 experts at 4 tokens (the FP64 router with the
    serial top-k over 16 logits per lane, the one-workgroup permutation over 1,024
    experts, the decode kernels' slot search) and at 300 tokens (the matrix-core
    router with the general refinement kernel, the chunked permutation, the
    weight-streaming kernels), and 640 experts at 300 tokens (the grouped-GEMM
    tile map over more than 512 segments);
  * the fused decode path (moe_layer_forward at 1 and 4 tokens) at intermediate
    sizes 64, 256, 1,024 and 2,048 (2 to 64 lanes per W2 row in the down
    projection with the combine) and at a shape whose (k + 1) * I / 32 exceeds
    256 (the fused path's separate down and combine kernels): bit-exact against
    the four separate calls and checked against the oracle.
"""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

ODD = gen.Shape(H=288, E=24, k=3, I=96)
_layers = {}


def layer_for(name, shape, cfg):
    if name not in _layers:
        L = gen.make_layer(cfg, shape=shape)
        _layers[name] = (L, gh.device_layer(L))
    return _layers[name]


def sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    s = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), dtype=np.int32)


@pytest.mark.parametrize("T", [3, 20, 300])
def test_generic_kernels_layer(T):
    gh.log("case: generic kernels H=288 I=96 E=24 k=3 T=%d" % T)
    L, DL = layer_for("odd", ODD, 0)
    x = gen.make_tokens(0, T, step=31, H=ODD.H)
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs", "h"))
    rep = gh.check_layer(L, x, g)
    gh.log("  ", rep.line())


@pytest.mark.parametrize("T,kb", [(20, (0, 2)), (20, (2, 6)), (300, (4, 6))])
def test_generic_kernels_krange(T, kb):
    gh.log("case: generic kernels K-split H=288 I=96 T=%d blocks %s" % (T, kb))
    L, DL = layer_for("odd", ODD, 0)
    x = gen.make_tokens(0, T, step=32, H=ODD.H)
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs"))
    part = gh.run_krange(DL, x, kb[0], kb[1])
    rep = gh.check_krange(L, x, g, part, kb[0], kb[1])
    gh.log("  ", rep.line())


@pytest.mark.parametrize("kb", [(0, 12), (4, 8), (8, 28)])
def test_mfma_krange(kb):
    gh.log("case: matrix-core K-split H=2048 I=512 T=40 blocks %s" % (kb,))
    L, DL = layer_for("dec", gen.SHAPES[1], 1)
    x = gen.make_tokens(1, 40, step=34)
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs"))
    part = gh.run_krange(DL, x, kb[0], kb[1])
    rep = gh.check_krange(L, x, g, part, kb[0], kb[1])
    gh.log("  ", rep.line())


@pytest.mark.parametrize("E,T", [(1024, 4), (1024, 300), (640, 300)])
def test_many_experts(E, T):
    gh.log("case: E=%d T=%d (H 2048, I 512, k 10)" % (E, T))
    L, DL = layer_for("E%d" % E, gen.Shape(H=2048, E=E, k=10, I=512), 1)
    x = gen.make_tokens(1, T, step=33)
    g = gh.run_layer(DL, x, dump=("xq", "xs", "hq", "hs"))
    assert len(np.unique(g["idx"])) > (30 if T == 4 else 500)
    rep = gh.check_layer(L, x, g, tokens=None if T <= 8 else sample_tokens(T, 32, E))
    gh.log("  ", rep.line())


FUSED_SHAPES = {
    "I64": gen.Shape(H=256, E=32, k=4, I=64),
    "I256": gen.Shape(H=512, E=64, k=6, I=256),
    "I1024": gen.Shape(H=256, E=32, k=3, I=1024),
    "I2048": gen.Shape(H=128, E=16, k=3, I=2048),
    "I1024k8": gen.Shape(H=256, E=64, k=8, I=1024),
}


@pytest.mark.parametrize("name", sorted(FUSED_SHAPES))
@pytest.mark.parametrize("T", [1, 4])
def test_fused_decode_shapes(name, T):
    sh = FUSED_SHAPES[name]
    gh.log("case: fused decode H=%d E=%d k=%d I=%d T=%d" % (sh.H, sh.E, sh.k, sh.I, T))
    L, DL = layer_for(name, sh, 1)
    x = gen.make_tokens(1, T, step=41, H=sh.H)
    res = gen.make_tokens(1, T, step=42, H=sh.H)
    ref = gh.run_layer(DL, x, residual=res, dump=())
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_layer_forward(DL, gh.to_dev(x.view(np.int16)), buf, residual=gh.to_dev(res.view(np.int16)))
    torch.cuda.synchronize()
    got = {"idx": buf.topk_idx, "w": buf.topk_w, "off": buf.expert_off, "r2p": buf.row2pair, "p2r": buf.pair2row,
           "y_rows": buf.y_rows, "y_shared": buf.y_shared, "out": buf.out}
    for key, t in got.items():
        a = t.cpu().numpy()
        if key == "out":
            a = a.view(np.uint16)
        assert np.array_equal(a, ref[key]), key
    rep = gh.check_layer(L, x, dict(ref, **gh.run_layer(DL, x, residual=res)), residual=res)
    gh.log("  ", rep.line())

"""The largest prompt chunk in one call: 262,144 tokens (2^18) through the
15,360-token layer shape (hidden 2048, 512 experts, top-10 + 1 shared,
intermediate 512).  Its FP32 output rows take 23.6 GB and the FP16 A4(h) rows
2.95 GB, so every row address past 2^31 bytes is exercised (64-bit offsets, per-tile
buffer resources).

Tokens are independent, and every call of at least 32 tokens takes the same
kernels, whose sums for one output do not depend on where its row sits in a
tile.  So a sample of 64 tokens, run as its own call, must give the same
routing, weights and output bits as those tokens inside the large call; the
small call is checked against the oracle in full.  The sample holds the first
and last token (the last shared-expert row), the token owning the last routed
row, the last row of the most loaded expert, and random tokens.  The
permutation of the large call is checked in full against the oracle's stable
sort of its routing.
"""
import numpy as np
import pytest
import torch

import checker
import gen

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

CFG = 3
T = 262144
N_SAMPLE = 64


def test_layer_max_tokens():
    gh.log("case: config %d, one call of %d tokens" % (CFG, T))
    L = gen.make_layer(CFG)
    DL = gh.device_layer(L)
    x = gen.make_tokens(CFG, T, step=77)
    k, E = DL.k, DL.E
    xd = gh.to_dev(x.view(np.int16))
    buf = moe.Buffers(DL, T, gh.DEV)
    moe.moe_forward(DL, xd, buf)
    torch.cuda.synchronize()
    idx = buf.topk_idx.cpu().numpy()
    w = buf.topk_w.cpu().numpy()
    off = buf.expert_off.cpu().numpy()
    r2p = buf.row2pair.cpu().numpy()
    p2r = buf.pair2row.cpu().numpy()
    out = buf.out.cpu().numpy().view(np.uint16)
    del buf, xd
    torch.cuda.empty_cache()
    checker.check_permutation(idx, E, off, r2p, p2r)
    counts = np.diff(off)
    heavy = int(np.argmax(counts))
    must = {0, T - 1, int(r2p[T * k - 1]) // k, int(r2p[off[heavy + 1] - 1]) // k}
    rng = np.random.default_rng(77)
    sample = set(must)
    while len(sample) < N_SAMPLE:
        sample.add(int(rng.integers(T)))
    s = np.array(sorted(sample), np.int32)
    gh.log("   expert load: max %d (expert %d); sample %d tokens incl. %s" % (counts.max(), heavy, s.size,
                                                                            sorted(must)))
    g = gh.run_layer(DL, x[s])
    rep = gh.check_layer(L, x[s], g)
    gh.log("   sample call vs oracle:", rep.line())
    assert np.array_equal(idx[s], g["idx"]), "routing of the sampled tokens differs from their own call"
    assert np.array_equal(w[s].view(np.uint32), g["w"].view(np.uint32)), "router weights differ"
    bad = np.nonzero(np.any(out[s] != g["out"], axis=1))[0]
    assert bad.size == 0, "outputs differ on sampled tokens %s" % s[bad[:8]].tolist()

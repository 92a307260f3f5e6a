"""Streamed prefill on one GPU: a 55,296-token prompt through one layer of the c3
shape as a single call and as chunks (4 x 13,824, and a ragged 40,000 + 15,000 +
296 split), with a residual added in the combine.

The layer treats tokens independently: routing, the A4 blocks of x and h, the
expert rows and the combine are all per token, and the permutation only orders
rows.  Every chunk of at least 32 tokens takes the same kernels (matrix-core
router with exact FP64 refinement, matrix-core expert GEMMs), whose sums for one
output do not depend on where its row sits in a tile, so the chunked outputs must
equal the single call's bit for bit.  (Chunks under 32 tokens take the weight-
streaming or decode kernels, which order their sums differently; they are not compared
here.)  The single call is checked against the oracle on sampled tokens.
"""
import time

import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

CFG = 3
T = 55296
SPLITS = ([13824] * 4, [40000, 15000, 296])


def test_streamed_prefill_chunks_match_single_call():
    gh.log("case: config %d, %d-token prompt, splits %s" % (CFG, T, SPLITS))
    L = gen.make_layer(CFG)
    DL = gh.device_layer(L)
    x = gen.make_tokens(CFG, T, step=55)
    res = gen.make_tokens(CFG, T, step=56)
    g = gh.run_layer(DL, x, residual=res)
    sample = np.array(sorted(set(np.random.default_rng(55).choice(T, 10, replace=False).tolist()) | {0, T - 1}),
                      np.int32)
    rep = gh.check_layer(L, x, g, tokens=sample, residual=res)
    gh.log("   single call:", rep.line())

    xd = gh.to_dev(x.view(np.int16))
    rd = gh.to_dev(res.view(np.int16))
    for split in SPLITS:
        assert sum(split) == T and min(split) >= 32
        buf = moe.Buffers(DL, max(split), gh.DEV)
        out = np.empty((T, DL.H), np.uint16)
        idx = np.empty((T, DL.k), np.int32)
        w = np.empty((T, DL.k), np.float32)
        t0, c0 = time.time(), 0
        for n in split:
            o = moe.moe_forward(DL, xd[c0:c0 + n], buf, residual=rd[c0:c0 + n])
            torch.cuda.synchronize()
            out[c0:c0 + n] = o[:n].cpu().numpy().view(np.uint16)
            idx[c0:c0 + n] = buf.topk_idx[:n].cpu().numpy()
            w[c0:c0 + n] = buf.topk_w[:n].cpu().numpy()
            c0 += n
        gh.log("   split %s: %.2f s" % (split, time.time() - t0))
        assert np.array_equal(idx, g["idx"]), "routing differs between chunked and single-call prefill"
        assert np.array_equal(w.view(np.uint32), g["w"].view(np.uint32)), "router weights differ"
        bad = np.nonzero(np.any(out != g["out"], axis=1))[0]
        assert bad.size == 0, "outputs differ on %d tokens (first %s)" % (bad.size, bad[:8].tolist())

"""The combine alone, for every compile-time bound on k the kernel is built for
(4, 8, 12, 16, 32) and the values of k at and just past each bound.

Inputs are random FP32 expert rows in a random permutation, softmax-like
weights, a shared row and a BF16 residual over a ragged token count.  The
oracle sums in FP64 and rounds once; the kernel sums in FP32 in slot order, so
each output must lie within half a BF16 unit of the FP64 sum plus the FP32
summation bound (k + 2) 2^-24 sum |terms|, and almost all must equal the
oracle's BF16 bits.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

H = 256
T = 37


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("k", [1, 4, 5, 8, 9, 12, 13, 16, 17, 32])
def test_combine_every_k_bound(k):
    gh.log("case: moe_combine k=%d T=%d H=%d" % (k, T, H))
    E = max(k, 32)
    dummy = torch.zeros(16, dtype=torch.uint8, device=gh.DEV)
    bank = {"codes": dummy, "scales": dummy, "gscale": torch.ones(1, device=gh.DEV)}
    DL = moe.MoELayer(H, 128, E, k, torch.empty(1, device=gh.DEV), None, None, sh13=bank, sh2=bank)
    rng = np.random.default_rng(1000 + k)
    P = T * k
    y = rng.standard_normal((P, H)).astype(np.float32)
    ysh = rng.standard_normal((T, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32) + np.float32(0.01)
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    p2r = rng.permutation(P).astype(np.int32)
    res = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = torch.empty((T, H), dtype=torch.int16, device=gh.DEV)
    moe.moe_combine(DL, gh.to_dev(y), gh.to_dev(ysh), gh.to_dev(p2r), gh.to_dev(w), out,
                    residual=gh.to_dev(res.view(np.int16)), T=T)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    yk = y[p2r].reshape(T, k, H).astype(np.float64)
    o64, o16 = oracle.combine(yk, w, ysh.astype(np.float64), res)
    mag = (np.abs(w.astype(np.float64)[:, :, None] * yk).sum(axis=1) + np.abs(ysh) +
           np.abs(_bf16_value(res)))
    err = (k + 2) * 2.0 ** -24 * mag
    ulp = 2.0 ** (np.floor(np.log2(np.abs(o64) + err + 1e-300)) - 7)
    d = np.abs(_bf16_value(got) - o64)
    assert np.all(d <= 0.5 * ulp + err), "worst excess %.3g" % (d - 0.5 * ulp - err).max()
    same = np.mean(got == o16)
    gh.log("   %.5f of outputs equal the oracle's BF16 bits" % same)
    assert same > 0.99

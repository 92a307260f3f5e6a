"""moe_layer_forward_noalloc, the layer call that allocates nothing (its workspace
is the library's own device array), against moe_layer_forward with a caller
workspace: every output bit-identical, on two calls in a row through the C ABI,
the second with a smaller input (the array keeps the first call's contents), on
the fused decode kernels and on the prompt-chunk kernels; and a token count whose
workspace exceeds the array is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

OUTS = ("topk_idx", "topk_w", "expert_off", "row2pair", "pair2row", "y_rows", "y_shared", "out")


def _garbage(buf):
    for name in OUTS:
        t = getattr(buf, name)
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)


@pytest.mark.parametrize("cfg,Ts", [(1, (300, 4, 1)), (0, (40, 8))])
def test_noalloc_matches_workspace_call(cfg, Ts):
    L = gen.make_layer(cfg)
    DL = gh.device_layer(L)
    for i, T in enumerate(Ts):
        gh.log("case: moe_layer_forward_noalloc config %d T=%d (call %d)" % (cfg, T, i + 1))
        x = gh.to_dev(gen.make_tokens(cfg, T, step=40 + i).view(np.int16))
        res = gh.to_dev(gen.make_tokens(cfg, T, step=50 + i).view(np.int16))
        ref = moe.Buffers(DL, T, gh.DEV)
        moe.moe_layer_forward(DL, x, ref, residual=res)
        got = moe.Buffers(DL, T, gh.DEV)
        _garbage(got)
        moe.moe_layer_forward_noalloc(DL, x, got, residual=res)
        torch.cuda.synchronize()
        for name in OUTS:
            a, b = getattr(ref, name), getattr(got, name)
            if a is None:
                assert b is None
                continue
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "%s differs at T=%d" % (name, T)


def test_noalloc_refuses_beyond_its_array():
    L = gen.make_layer(0)
    DL = gh.device_layer(L)
    lim = moe.lib.moe_noalloc_scratch_bytes()
    T = 1
    while DL.workspace_bytes(T) <= lim:
        T *= 2
    buf = moe.Buffers(DL, 8, gh.DEV)
    p = buf.out.data_ptr()  # never dereferenced: the size check comes first
    rc = moe.lib.moe_layer_forward_noalloc(ctypes.byref(DL.desc), p, T, None, p, p, p, p, p, p, p, p, None, None)
    assert rc == moe.MOE_EWORKSPACE

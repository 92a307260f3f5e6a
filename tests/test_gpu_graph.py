"""The layer captured into a HIP graph and replayed: every replay writes exactly
what the same calls write eagerly.

No entry point synchronises the host or clears memory with a memset, so a
caller may capture a whole step.  Each case captures several steps (distinct
inputs, one set of buffers per step), replays the graph four times with eager
work in between (other layer calls on the same weights, and the graph's
outputs overwritten with garbage), and compares every replay's routing,
weights and output bits with the eager results.  Cases: the fused decode call
at 1 and 4 tokens; the four separate calls at 20 tokens (weight-streaming
kernels) and at 300 tokens (matrix-core kernels: the one-tile down kernel on
the small shape, the persistent down kernel with its work counters on the
decode shape).
"""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gpu_harness as gh
    import nvfp4_w4a4_expert_router_amd as moe

STEPS = 3
REPLAYS = 4


def _step(DL, x, buf, fused, res):
    if fused:
        moe.moe_layer_forward(DL, x, buf, residual=res)
    else:
        moe.moe_forward(DL, x, buf, residual=res)


def _snapshot(bufs):
    return [(b.topk_idx.cpu().numpy().copy(), b.topk_w.cpu().numpy().view(np.uint32).copy(),
             b.out.cpu().numpy().view(np.uint16).copy()) for b in bufs]


@pytest.mark.parametrize("cfg,T,fused", [(1, 1, True), (1, 4, True), (1, 20, False), (0, 300, False), (1, 300, False)])
def test_graph_replays_match_eager(cfg, T, fused):
    gh.log("case: HIP graph, config %d T=%d %s" % (cfg, T, "moe_layer_forward" if fused else "four calls"))
    L = gen.make_layer(cfg)
    DL = gh.device_layer(L)
    xs = [gh.to_dev(gen.make_tokens(cfg, T, step=40 + i).view(np.int16)) for i in range(STEPS)]
    res = gh.to_dev(gen.make_tokens(cfg, T, step=50).view(np.int16))
    bufs = [moe.Buffers(DL, T, gh.DEV) for _ in range(STEPS)]
    # eager reference
    for i in range(STEPS):
        _step(DL, xs[i], bufs[i], fused, res if i == 1 else None)
    torch.cuda.synchronize()
    ref = _snapshot(bufs)
    # capture (the calls ran once eagerly above, so nothing initialises lazily here)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for i in range(STEPS):
                _step(DL, xs[i], bufs[i], fused, res if i == 1 else None)
    torch.cuda.synchronize()
    other = moe.Buffers(DL, T, gh.DEV)
    x_other = gh.to_dev(gen.make_tokens(cfg, T, step=60).view(np.int16))
    for r in range(REPLAYS):
        # eager work between replays: garbage in the graph's outputs and
        # workspaces, and another call on the same weights
        for b in bufs:
            b.out.fill_(0x7F7F)
            b.topk_idx.fill_(-1)
            b.topk_w.fill_(float("nan"))
            b.ws.fill_(0xA5)
        _step(DL, x_other, other, fused, None)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(bufs)
        for i in range(STEPS):
            for name, a, b in zip(("topk_idx", "topk_w", "out"), got[i], ref[i]):
                assert np.array_equal(a, b), "replay %d, step %d: %s differs from the eager call" % (r, i, name)
    gh.log("   %d replays of %d steps equal the eager calls" % (REPLAYS, STEPS))

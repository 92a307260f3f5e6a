#!/usr/bin/env python3
"""Throughput of the routed NVFP4 W4A4 MoE layer on one MI355X.

Workload: the decode-shaped layer (hidden 2048, 512 experts, top-10 routed + 1
shared, expert intermediate 512, about 0.91 GB of packed NVFP4 weights per
layer) on a 4-token batch, the verify window of 3-token speculative decoding.
A step is one pass of route -> permute -> expert FFN -> combine over one batch
(one moe_layer_forward call; --separate-calls uses the four C-ABI steps).
Every step takes a fresh batch of tokens and the next of `--layers` layers with
distinct weights (8 x 0.91 GB by default), so weights come from HBM and not
from the 256 MB Infinity Cache.  Inputs are seeded synthetic data, resident in
HBM before the timed region.

Prints one JSON line (stdout).  value = tokens per second through one MoE layer.
roofline: the gate/up kernel (the dominant one) - algorithmic bytes per launch
(selected experts' W13 codes + scales + per-expert scale, the tokens' A4(x)
codes + scales read, A4(h) codes + scales written) over its average duration,
timed with HIP events recorded by the library on the launch stream inside the
timed region.  cpu_baseline: the FP64 oracle on a bounded sample of the same
workload on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--tokens", type=int, default=4, help="tokens per step (decode batch)")
    ap.add_argument("--layers", type=int, default=8, help="distinct layers rotated through")
    ap.add_argument("--pool", type=int, default=64, help="distinct token batches rotated through")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=16, help="steps per captured HIP graph (0 = no graph run)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="run the four C-ABI steps as separate calls instead of moe_layer_forward")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic_gateup_decode.json"),
                    help="HBM bytes per gate/up launch measured with rocprofv3 counters (optional)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this layer is built and measured on a single MI355X "
              "(expert parallelism across GPUs is a design note, not part of this build); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not os.path.exists(os.path.join(ROOT, "nvfp4_w4a4_expert_router_amd", "libnvfp4moe.so")):
        import __graft_entry__
        __graft_entry__.build()
    import gen
    import nvfp4_w4a4_expert_router_amd as moe

    dev = "cuda:0"
    cfg = 1
    sh = gen.SHAPES[cfg]
    T, K, W = args.tokens, args.steps, args.warmup

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    layers, host_layer0 = [], None
    t0 = time.time()
    for l in range(args.layers):
        Lh = gen.make_layer(cfg, layer=l)
        bank = lambda b: {"codes": up(b["codes"]), "scales": up(b["scales"]), "gscale": up(b["gscale"])}
        layers.append(moe.MoELayer(sh.H, sh.I, sh.E, sh.k, up(Lh.router_w), bank(Lh.w13), bank(Lh.w2),
                                   bank(Lh.sh13), bank(Lh.sh2)))
        if l == 0:
            host_layer0 = Lh
        log("layer %d generated and uploaded (%.1f s)" % (l, time.time() - t0))
    pool = [up(gen.make_tokens(cfg, T, step=s).view(np.int16)) for s in range(args.pool)]

    buf = moe.Buffers(layers[0], T, dev)
    ws = buf.ws
    n_total = W + K
    rec_idx = torch.empty((n_total, T, sh.k), dtype=torch.int32, device=dev)
    rec_w = torch.empty((n_total, T, sh.k), dtype=torch.float32, device=dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * moe.FFN_KERNELS)] for _ in range(n_total)]
    stream = torch.cuda.current_stream()
    for evs in events:  # create the underlying HIP events
        for e in evs:
            e.record(stream)
    torch.cuda.synchronize()

    def step(i, timed_events=True, rec=None):
        DL = layers[i % len(layers)]
        x = pool[i % len(pool)]
        ridx, rw = (rec_idx[i], rec_w[i]) if rec is None else rec
        dbg = {"events": events[i]} if timed_events else None
        if args.separate_calls:
            moe.moe_route(DL, x, ridx, rw, ws, T=T)
            moe.moe_permute(DL, ridx, buf.expert_off, buf.row2pair, buf.pair2row, ws, T=T)
            moe.moe_expert_ffn(DL, x, buf.expert_off, buf.row2pair, buf.y_rows, buf.y_shared, ws, debug=dbg, T=T)
            moe.moe_combine(DL, buf.y_rows, buf.y_shared, buf.pair2row, rw, buf.out, T=T)
        else:
            moe.moe_layer_forward(DL, x, buf, T=T, debug=dbg, topk=(ridx, rw))

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log("warmup done")
    t_start = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log("timed %d steps in %.3f s" % (K, elapsed))

    # the same steps replayed from a HIP graph (no host launch cost): one graph
    # holds `--graph-steps` consecutive steps over the rotating layers and batches
    graph_value = None
    if args.graph_steps > 0:
        gsteps = args.graph_steps
        gidx = torch.empty((gsteps, T, sh.k), dtype=torch.int32, device=dev)
        gw = torch.empty((gsteps, T, sh.k), dtype=torch.float32, device=dev)
        for i in range(gsteps):  # warm the captured sequence once eagerly
            step(i, timed_events=False, rec=(gidx[i], gw[i]))
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(gsteps):
                step(i, timed_events=False, rec=(gidx[i], gw[i]))
        torch.cuda.synchronize()
        reps = max(1, K // gsteps)
        for _ in range(max(1, W // gsteps)):
            graph.replay()
        torch.cuda.synchronize()
        g0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        g_el = time.perf_counter() - g0
        graph_value = T * gsteps * reps / g_el
        log("graph: %d replays of %d steps in %.3f s" % (reps, gsteps, g_el))

    # per-kernel durations from the events recorded by the library
    def avg_ms(a, b):
        return float(np.mean([events[i][a].elapsed_time(events[i][b]) for i in range(W, W + K)]))

    t_first, t_gateup, t_down = avg_ms(0, 1), avg_ms(2, 3), avg_ms(4, 5)
    idx = rec_idx[W:].cpu().numpy()
    n_distinct = np.array([len(np.unique(idx[i])) for i in range(K)], dtype=np.float64)
    H, I = sh.H, sh.I
    w13_bytes = 2 * I * H // 2 + 2 * I * H // 16 + 4
    w2_bytes = H * I // 2 + H * I // 16 + 4
    rows = T * sh.k + T
    act_in = T * (H // 2 + H // 16)
    h_out = rows * (I // 2 + I // 16)
    gateup_bytes = float(np.mean((n_distinct + 1) * w13_bytes)) + act_in + h_out
    down_bytes = float(np.mean((n_distinct + 1) * w2_bytes)) + h_out + rows * H * 4
    layer_bytes = (4 * sh.E * H + float(np.mean((n_distinct + 1) * (w13_bytes + w2_bytes))) + T * H * 2 * 2)
    achieved = gateup_bytes / (t_gateup * 1e-3) / 1e9
    ms_per_step = elapsed * 1e3 / K
    value = T * K / elapsed

    traffic = None
    if args.traffic_json and os.path.exists(args.traffic_json):
        try:
            traffic = json.load(open(args.traffic_json)).get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    # ---------------------------------------------------------------- oracle on the host
    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        n_tok, t_cpu, s = 0, 0.0, 0
        while t_cpu < args.cpu_seconds and s < args.pool:
            x = gen.make_tokens(cfg, T, step=s)
            c0 = time.perf_counter()
            oracle.layer(host_layer0, x)
            t_cpu += time.perf_counter() - c0
            n_tok += T
            s += 1
        omp = int(os.environ.get("OMP_NUM_THREADS", threads))
        cpu = {"value": round(n_tok / t_cpu, 3), "unit": "tok/s per MoE layer", "cores": min(omp, threads),
               "kind": "oracle",
               "sample": "%d decode batches of %d tokens through layer 0 (%d tokens, %.1f s of FP64 oracle)" % (
                   s, T, n_tok, t_cpu)}
        log("oracle: %d tokens in %.1f s" % (n_tok, t_cpu))

    rec = {
        "metric": "NVFP4 MoE layer tok/s; decode HBM GB/s and prefill MFMA % of peak",
        "value": round(value, 1),
        "unit": "tok/s per MoE layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4-w4a4/fp32-acc",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) router and expert weights packed as NVFP4)",
        "config": {"workload": "decode MoE layer: hidden 2048, 512 experts, top-10 + 1 shared, intermediate 512, "
                               "%d tokens per step (MTP K=3 verify window), %d rotating layers" % (T, args.layers),
                   "tokens_per_step": T, "layers_rotated": args.layers, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "k_gateup_decode", "algorithmic_bytes_per_launch": round(gateup_bytes),
                     "avg_duration_us": round(t_gateup * 1e3, 3)},
        "cpu_baseline": cpu,
        "detail": {
            "kernel_avg_us": {("quant_act" if args.separate_calls else "router_logits"): round(t_first * 1e3, 3),
                              "gateup": round(t_gateup * 1e3, 3),
                              "down": round(t_down * 1e3, 3)},
            "down_achieved_GBs": round(down_bytes / (t_down * 1e-3) / 1e9, 1),
            "distinct_experts_per_step": round(float(n_distinct.mean()), 3),
            "layer_algorithmic_bytes": round(layer_bytes),
            "layer_effective_GBs": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
            "eager_tok_s": round(value, 1),
            "hip_graph_tok_s": None if graph_value is None else round(graph_value, 1),
        },
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Throughput of the routed NVFP4 W4A4 MoE layer on one MI355X.

Decode workload (the headline `value`): the decode-shaped layer (hidden 2048,
512 experts, top-10 routed + 1 shared, expert intermediate 512, about 0.91 GB
of packed NVFP4 weights per layer) on a 4-token batch, the verify window of
3-token speculative decoding.  A step is one pass of route -> permute -> expert
FFN -> combine over one batch (one moe_layer_forward call; --separate-calls
uses the four C-ABI steps).  Every step takes a fresh batch of tokens and the
next of `--layers` layers with distinct weights (8 x 0.91 GB by default), so
weights come from HBM and not from the 256 MB Infinity Cache.  A 1-token
batch is timed the same way and reported in `detail`.

Prefill workload (reported in `detail.prefill`): the same layer shape with
Zipf(1.1)-skewed routing over one 15,360-token chunk; expert GEMM throughput is
priced against the FP16 matrix-core peak the exact NVFP4 decode runs on, and
against the FP8 peak.  `detail.streamed_prefill`: a 55,296-token prompt through
the same layer as four 13,824-token calls, the residual added in each combine.

Inputs are seeded synthetic data, resident in HBM before any timed region.
Prints one JSON line (stdout).  value = tokens per second through one MoE layer.
roofline: the decode gate/up kernel (the dominant one) - algorithmic bytes per
launch (selected experts' W13 codes + scales + per-expert scale, the tokens'
A4(x) codes + scales read, A4(h) codes + scales written) over its average
duration, timed inside the timed region with HIP events that take the
kernel's own start and end timestamps (the library launches it with
hipExtLaunchKernel when events are passed).  cpu_baseline: the FP64 oracle on a bounded sample of
the same decode workload on the host's cores.

--copy-calibration MIB runs only a plain device-to-device copy of MIB MiB (the
reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_decode.txt")
DECODE_SOURCES = ("ffn_decode.hip", "common.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--tokens", type=int, default=4, help="tokens per decode step")
    ap.add_argument("--layers", type=int, default=8, help="distinct layers rotated through")
    ap.add_argument("--pool", type=int, default=64, help="distinct token batches rotated through")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=16, help="steps per captured HIP graph (0 = no graph run)")
    ap.add_argument("--prefill-tokens", type=int, default=15360, help="prefill chunk (0 = skip the prefill leg)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--stream-tokens", type=int, default=55296, help="streamed prompt length (0 = skip)")
    ap.add_argument("--stream-chunks", type=int, default=4)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode legs (profiling the prefill only)")
    ap.add_argument("--skip-t1", action="store_true", help="skip the 1-token decode leg")
    ap.add_argument("--separate-calls", action="store_true",
                    help="run the four C-ABI steps as separate calls instead of moe_layer_forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, for counter calibration")
    return ap.parse_args()


def decode_sources_digest():
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "nvfp4_w4a4_expert_router_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or None
    when it is missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_sha256_16") != decode_sources_digest():
        log("traffic summary was taken on other decode sources: traffic reported as null")
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log("copied %d MiB 3 times" % mib)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this layer is built and measured on a single MI355X "
              "(expert parallelism across GPUs is designed but not implemented); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    if not os.path.exists(os.path.join(ROOT, "nvfp4_w4a4_expert_router_amd", "libnvfp4moe.so")):
        import __graft_entry__
        __graft_entry__.build()
    import gen
    import nvfp4_w4a4_expert_router_amd as moe

    dev = "cuda:0"
    cfg = 1
    sh = gen.SHAPES[cfg]
    H, I, E, k = sh.H, sh.I, sh.E, sh.k
    T, K, W = args.tokens, args.steps, args.warmup

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def device_layer(Lh):
        bank = lambda b: {"codes": up(b["codes"]), "scales": up(b["scales"]), "gscale": up(b["gscale"])}
        return moe.MoELayer(H, I, E, k, up(Lh.router_w), bank(Lh.w13), bank(Lh.w2), bank(Lh.sh13), bank(Lh.sh2))

    w13_bytes = 2 * I * H // 2 + 2 * I * H // 16 + 4
    w2_bytes = H * I // 2 + H * I // 16 + 4
    stream = torch.cuda.current_stream()
    rec = {
        "metric": "NVFP4 MoE layer tok/s; decode HBM GB/s and prefill MFMA % of peak",
        "value": None, "unit": "tok/s per MoE layer", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4-w4a4/fp32-acc",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) router and expert weights packed as NVFP4)",
        "config": {"workload": "decode MoE layer: hidden 2048, 512 experts, top-10 + 1 shared, intermediate 512, "
                               "%d tokens per step (MTP K=3 verify window), %d rotating layers" % (T, args.layers),
                   "tokens_per_step": T, "layers_rotated": args.layers, "parallelism": "single GPU"},
        "roofline": None, "cpu_baseline": None, "detail": {},
    }

    host_layer0 = None
    if not args.no_decode:
        layers = []
        t0 = time.time()
        for l in range(args.layers):
            Lh = gen.make_layer(cfg, layer=l)
            layers.append(device_layer(Lh))
            if l == 0:
                host_layer0 = Lh
            log("layer %d generated and uploaded (%.1f s)" % (l, time.time() - t0))

        def decode_leg(T, K, W, graph_steps):
            pool = [up(gen.make_tokens(cfg, T, step=s).view(np.int16)) for s in range(args.pool)]
            buf = moe.Buffers(layers[0], T, dev)
            n_total = W + K
            # per-step records of the selection, each row padded to 16 bytes (the
            # library takes 16-byte aligned pointers)
            pad = (T * k + 3) // 4 * 4
            rec_idx = torch.empty((n_total, pad), dtype=torch.int32, device=dev)
            rec_w = torch.empty((n_total, pad), dtype=torch.float32, device=dev)
            sel = lambda a, i: a[i, :T * k].view(T, k)
            events = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * moe.FFN_KERNELS)]
                      for _ in range(n_total)]
            for evs in events:  # create the underlying HIP events
                for e in evs:
                    e.record(stream)
            torch.cuda.synchronize()

            def step(i, timed_events=True, rec=None):
                DL = layers[i % len(layers)]
                x = pool[i % len(pool)]
                ridx, rw = (sel(rec_idx, i), sel(rec_w, i)) if rec is None else rec
                dbg = {"events": events[i]} if timed_events else None
                if args.separate_calls:
                    moe.moe_route(DL, x, ridx, rw, buf.ws, T=T)
                    moe.moe_permute(DL, ridx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=T)
                    moe.moe_expert_ffn(DL, x, buf.expert_off, buf.row2pair, buf.y_rows, buf.y_shared, buf.ws,
                                       debug=dbg, T=T)
                    moe.moe_combine(DL, buf.y_rows, buf.y_shared, buf.pair2row, rw, buf.out, T=T)
                else:
                    moe.moe_layer_forward(DL, x, buf, T=T, debug=dbg, topk=(ridx, rw))

            for i in range(W):
                step(i)
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for i in range(W, W + K):
                step(i)
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t_start
            log("T=%d: timed %d steps in %.3f s" % (T, K, elapsed))

            # the same steps replayed from a HIP graph (no host launch cost): one
            # graph holds `graph_steps` consecutive steps over the rotating layers
            graph_value, graph_steps_timed = None, 0
            if graph_steps > 0:
                gidx = torch.empty((graph_steps, pad), dtype=torch.int32, device=dev)
                gw = torch.empty((graph_steps, pad), dtype=torch.float32, device=dev)
                for i in range(graph_steps):  # warm the captured sequence once eagerly
                    step(i, timed_events=False, rec=(sel(gidx, i), sel(gw, i)))
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for i in range(graph_steps):
                        step(i, timed_events=False, rec=(sel(gidx, i), sel(gw, i)))
                torch.cuda.synchronize()
                reps = max(1, K // graph_steps)
                for _ in range(max(1, W // graph_steps)):
                    graph.replay()
                torch.cuda.synchronize()
                g0 = time.perf_counter()
                for _ in range(reps):
                    graph.replay()
                torch.cuda.synchronize()
                g_el = time.perf_counter() - g0
                graph_value = T * graph_steps * reps / g_el
                graph_steps_timed = graph_steps * reps
                log("T=%d graph: %d replays of %d steps in %.3f s" % (T, reps, graph_steps, g_el))

            def avg_ms(a, b):
                return float(np.mean([events[i][a].elapsed_time(events[i][b]) for i in range(W, W + K)]))

            idx = rec_idx[W:, :T * k].cpu().numpy()
            n_distinct = np.array([len(np.unique(idx[i])) for i in range(K)], dtype=np.float64)
            rows = T * k + T
            act_in = T * (H // 2 + H // 16)
            h_out = rows * (I // 2 + I // 16)
            out = {
                "T": T, "elapsed": elapsed, "tok_s": T * K / elapsed, "ms_per_step": elapsed * 1e3 / K,
                "graph_tok_s": graph_value, "graph_steps_timed": graph_steps_timed,
                "t_first": avg_ms(0, 1), "t_gateup": avg_ms(2, 3), "t_down": avg_ms(4, 5),
                "n_distinct": float(n_distinct.mean()),
                "gateup_bytes": float(np.mean((n_distinct + 1) * w13_bytes)) + act_in + h_out,
                "down_bytes": float(np.mean((n_distinct + 1) * w2_bytes)) + h_out + rows * H * 4,
                "layer_bytes": 4 * E * H + float(np.mean((n_distinct + 1) * (w13_bytes + w2_bytes))) + T * H * 2 * 2,
            }
            del buf, pool, events
            return out

        d = decode_leg(T, K, W, args.graph_steps)
        d1 = None
        if T != 1 and not args.skip_t1:
            d1 = decode_leg(1, max(1, K // 2), max(1, W // 2), args.graph_steps)
        achieved = d["gateup_bytes"] / (d["t_gateup"] * 1e-3) / 1e9
        if d["graph_tok_s"] is not None:  # steps replayed from HIP graphs: no host launch cost per kernel
            rec["value"] = round(d["graph_tok_s"], 1)
            rec["ms_per_step"] = round(T / d["graph_tok_s"] * 1e3, 5)
            rec["steps"] = d["graph_steps_timed"]
            rec["config"]["launch"] = "HIP graphs of %d steps" % args.graph_steps
        else:
            rec["value"] = round(d["tok_s"], 1)
            rec["ms_per_step"] = round(d["ms_per_step"], 5)
            rec["config"]["launch"] = "eager (one host launch per kernel)"
        rec["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                           "kernel": "k_gateup_decode<true>", "algorithmic_bytes_per_launch": round(d["gateup_bytes"]),
                           "avg_duration_us": round(d["t_gateup"] * 1e3, 3)}

        def summary(d):
            return {
                "eager_tok_s": round(d["tok_s"], 1),
                "hip_graph_tok_s": None if d["graph_tok_s"] is None else round(d["graph_tok_s"], 1),
                "kernel_avg_us": {("quant_act" if args.separate_calls else "router_logits"): round(d["t_first"] * 1e3, 3),
                                  "gateup": round(d["t_gateup"] * 1e3, 3), "down": round(d["t_down"] * 1e3, 3)},
                "gateup_achieved_GBs": round(d["gateup_bytes"] / (d["t_gateup"] * 1e-3) / 1e9, 1),
                "down_achieved_GBs": round(d["down_bytes"] / (d["t_down"] * 1e-3) / 1e9, 1),
                "distinct_experts_per_step": round(d["n_distinct"], 3),
                "layer_algorithmic_bytes": round(d["layer_bytes"]),
                "layer_effective_GBs": round(d["layer_bytes"] / (d["ms_per_step"] * 1e-3) / 1e9, 1),
            }

        rec["detail"]["decode_T%d" % T] = summary(d)
        if d1 is not None:
            rec["detail"]["decode_T1"] = summary(d1)
        del layers

    # ---------------------------------------------------------------- prefill chunk
    if args.prefill_tokens > 0:
        Tp, cfg_p = args.prefill_tokens, 3
        t0 = time.time()
        Lp = gen.make_layer(cfg_p)
        DLp = device_layer(Lp).pack_kmajor()  # K-step-major weight copies for the matrix-core kernels
        xp = up(gen.make_tokens(cfg_p, Tp).view(np.int16))
        log("prefill layer and %d tokens generated (%.1f s)" % (Tp, time.time() - t0))
        buf = moe.Buffers(DLp, Tp, dev)
        n = args.prefill_steps
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * moe.FFN_KERNELS)] for _ in range(n)]
        st = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for evs in ev:  # create the underlying HIP events
            for e in evs:
                e.record(stream)
        for _ in range(2):
            moe.moe_layer_forward(DLp, xp, buf, T=Tp)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(n):
            st[i][0].record(stream)
            moe.moe_route(DLp, xp, buf.topk_idx, buf.topk_w, buf.ws, T=Tp)
            moe.moe_permute(DLp, buf.topk_idx, buf.expert_off, buf.row2pair, buf.pair2row, buf.ws, T=Tp)
            st[i][1].record(stream)
            moe.moe_expert_ffn(DLp, xp, buf.expert_off, buf.row2pair, buf.y_rows, buf.y_shared, buf.ws,
                               debug={"events": ev[i]}, T=Tp)
            moe.moe_combine(DLp, buf.y_rows, buf.y_shared, buf.pair2row, buf.topk_w, buf.out, T=Tp)
            st[i][2].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start

        def med(f):
            return float(np.median([f(i) for i in range(n)]))

        t_route = med(lambda i: st[i][0].elapsed_time(st[i][1]))
        t_ffn_comb = med(lambda i: st[i][1].elapsed_time(st[i][2]))
        t_g1 = med(lambda i: ev[i][2].elapsed_time(ev[i][3]))
        t_g2 = med(lambda i: ev[i][4].elapsed_time(ev[i][5]))
        rows = Tp * k + Tp
        fl_g1, fl_g2 = 2.0 * rows * H * 2 * I, 2.0 * rows * I * H
        tf = (fl_g1 + fl_g2) / ((t_g1 + t_g2) * 1e-3) / 1e12
        rec["detail"]["prefill"] = {
            "workload": "one %d-token chunk, same layer shape, Zipf(1.1)-skewed routing" % Tp,
            "tok_s": round(Tp * n / elapsed, 1),
            "ms_per_chunk": round(elapsed * 1e3 / n, 4),
            "route_permute_ms": round(t_route, 4), "ffn_combine_ms": round(t_ffn_comb, 4),
            "gateup_ms": round(t_g1, 4), "down_ms": round(t_g2, 4),
            "gateup_TFLOPs": round(fl_g1 / (t_g1 * 1e-3) / 1e12, 1),
            "down_TFLOPs": round(fl_g2 / (t_g2 * 1e-3) / 1e12, 1),
            "expert_gemm_TFLOPs": round(tf, 1),
            "frac_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
            "frac_fp8_mfma_peak": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
            "expert_gemm_flop": fl_g1 + fl_g2,
        }
        log("prefill: %d chunks in %.3f s" % (n, elapsed))
        if rec["value"] is None:  # prefill-only run (profiling)
            rec["value"] = round(Tp * n / elapsed, 1)
            rec["ms_per_step"] = round(elapsed * 1e3 / n, 5)
            rec["config"] = {"workload": rec["detail"]["prefill"]["workload"], "tokens_per_step": Tp,
                             "parallelism": "single GPU"}
        # streamed prompt: the same layer over a long prompt in equal chunks (each
        # chunk one library call with the residual added in its combine)
        if args.stream_tokens > 0:
            Ts, nc = args.stream_tokens, args.stream_chunks
            cs = Ts // nc
            xs_ = up(gen.make_tokens(cfg_p, Ts, step=55).view(np.int16))
            rs_ = up(gen.make_tokens(cfg_p, Ts, step=56).view(np.int16))
            bufs = moe.Buffers(DLp, cs, dev)
            outs = torch.empty((Ts, H), dtype=torch.int16, device=dev)

            def prompt():
                for c in range(nc):
                    o = moe.moe_layer_forward(DLp, xs_[c * cs:(c + 1) * cs], bufs, residual=rs_[c * cs:(c + 1) * cs])
                    outs[c * cs:(c + 1) * cs].copy_(o[:cs])

            prompt()
            torch.cuda.synchronize()
            reps = 3
            t_s = time.perf_counter()
            for _ in range(reps):
                prompt()
            torch.cuda.synchronize()
            el = time.perf_counter() - t_s
            rec["detail"]["streamed_prefill"] = {
                "workload": "a %d-token prompt as %d chunks of %d tokens, residual added, same layer" % (nc * cs, nc, cs),
                "tok_s": round(nc * cs * reps / el, 1), "ms_per_prompt": round(el * 1e3 / reps, 4)}
            log("streamed prefill: %d prompts in %.3f s" % (reps, el))
            del bufs, xs_, rs_, outs
        del buf, DLp, xp

    # ---------------------------------------------------------------- oracle on the host
    if args.cpu_seconds > 0 and host_layer0 is not None:
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
        rec["cpu_baseline"] = {
            "value": round(n_tok / t_cpu, 3), "unit": "tok/s per MoE layer", "cores": min(omp, threads),
            "kind": "oracle",
            "sample": "%d decode batches of %d tokens through layer 0 (%d tokens, %.1f s of FP64 oracle)" % (
                s, T, n_tok, t_cpu)}
        log("oracle: %d tokens in %.1f s" % (n_tok, t_cpu))

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

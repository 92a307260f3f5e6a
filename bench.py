#!/usr/bin/env python3
"""Throughput of the routed NVFP4 W4A4 MoE layer on one MI355X.

Decode workload (the headline `value`): the decode-shaped layer (hidden 2048,
512 experts, top-10 routed + 1 shared, expert intermediate 512, about 0.91 GB
of packed NVFP4 weights per layer) on a 4-token batch, the verify window of
3-token speculative decoding.  A step is one pass of route -> permute -> expert
FFN -> combine over one batch (one moe_layer_forward call).  Every step takes a
fresh batch of tokens and the next layer of the 48-layer stack (43.8 GB of
distinct weights, far beyond the 256 MB Infinity Cache), so weights come from
HBM.  Exactly --steps steps are timed: one HIP graph holding those steps is
replayed once between device synchronizations, timed by HIP events on the
launch stream.  Further replays of the same graph (at least 200 steps and
100 ms in all) give the median, p10 and p90 of the time per step.  A 1-token
batch is timed the same way and reported in `detail`.

Other legs (in `detail`):
  * stack: the 48-layer stack (each layer: parameter-free RMS norm of the
    residual stream, the MoE layer with the residual added in its combine) at 1
    and 4 tokens, all 48 layers in one HIP graph: time per pass and per token;
  * prefill: one 15,360-token chunk with Zipf(1.1)-skewed routing; expert GEMM
    throughput priced against the FP16 matrix-core peak the exact NVFP4 decode
    runs on (and against the FP8 peak), with its own `roofline` object;
  * prefill_4096: the same on a 4,096-token chunk;
  * streamed_prefill: a 55,296-token prompt as four 13,824-token calls;
  * clocks (amd-smi, at start and end) and the bandwidth of a plain 1 GiB
    device copy.

Inputs are seeded synthetic data, resident in HBM before any timed region.
Prints one JSON line (stdout).  value = tokens per second through one MoE layer.
roofline: the decode gate/up kernel (the dominant one) - algorithmic bytes per
launch (selected experts' W13 codes + scales + per-expert scale, the tokens'
A4(x) codes + scales read, A4(h) written) over its average duration, from HIP
events that take the kernel's own start and end timestamps (the library launches
it with hipExtLaunchKernel when events are passed) over --steps eagerly launched
steps.  cpu_baseline: the FP64 oracle on a bounded sample of the same decode
workload on the host's cores.

--copy-calibration MIB runs only a plain device-to-device copy of MIB MiB (the
reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exits.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense
FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gateup_decode.txt")
DECODE_SOURCES = ("ffn_decode.hip", "common.hpp", "routing.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--tokens", type=int, default=4, help="tokens per decode step")
    ap.add_argument("--layers", type=int, default=48, help="layers of the stack generated (decode steps rotate over them)")
    ap.add_argument("--pool", type=int, default=64, help="distinct token batches rotated through")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--graph-steps", type=int, default=1, help="0: time eager launches only (no HIP graph)")
    ap.add_argument("--spread-steps", type=int, default=200, help="steps replayed for median / p10 / p90")
    ap.add_argument("--no-stack", action="store_true", help="skip the 48-layer stack leg")
    ap.add_argument("--prefill-tokens", type=int, default=15360, help="prefill chunk (0 = skip the prefill leg)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--c2-tokens", type=int, default=4096, help="second prefill chunk (0 = skip)")
    ap.add_argument("--stream-tokens", type=int, default=55296, help="streamed prompt length (0 = skip)")
    ap.add_argument("--stream-chunks", type=int, default=4)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode legs (profiling the prefill only)")
    ap.add_argument("--skip-t1", action="store_true", help="skip the 1-token decode leg")
    ap.add_argument("--no-variants", action="store_true", help="skip the W4A8 and shared-gate decode timings")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not run amd-smi for the clock log (under a counter-collecting profiler)")
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


def read_clocks():
    """Current GPU and memory clocks (MHz) from amd-smi, or None when the tool
    cannot tell (the raw text is kept for the record)."""
    for cmd in (["amd-smi", "metric", "-g", "0", "-c", "--json"], ["amd-smi", "metric", "-c", "--json"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except (OSError, subprocess.TimeoutExpired):
            continue
        if r.returncode != 0 or not r.stdout.strip():
            continue
        found = {}

        def walk(node, path):
            if isinstance(node, dict):
                if "clk" in node and isinstance(node["clk"], dict) and "value" in node["clk"]:
                    found[path] = node["clk"]["value"]
                for key, val in node.items():
                    walk(val, path + "/" + str(key))
            elif isinstance(node, list):
                for i, val in enumerate(node):
                    walk(val, path + "/" + str(i))

        try:
            walk(json.loads(r.stdout), "")
        except ValueError:
            return {"raw": r.stdout[:800]}
        out = {}
        for path, v in found.items():
            key = path.rsplit("/", 1)[-1].lower()
            if key.startswith("gfx") and "sclk_mhz" not in out:
                out["sclk_mhz"] = v
            elif key.startswith("mem") and "mclk_mhz" not in out:
                out["mclk_mhz"] = v
        out["all"] = {p.rsplit("/", 1)[-1]: v for p, v in found.items()}
        return out
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


def pct(v, q):
    return float(np.percentile(np.asarray(v, np.float64), q))


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
    stream = torch.cuda.current_stream()
    sh = gen.SHAPES[1]
    H, I, E, k = sh.H, sh.I, sh.E, sh.k
    T, K, W = args.tokens, args.steps, args.warmup

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def device_layer(Lh):
        bank = lambda b: {"codes": up(b["codes"]), "scales": up(b["scales"]), "gscale": up(b["gscale"])}
        return moe.MoELayer(H, I, E, k, up(Lh.router_w), bank(Lh.w13), bank(Lh.w2), bank(Lh.sh13), bank(Lh.sh2))

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # creates the HIP event
        return e

    w13_bytes = 2 * I * H // 2 + 2 * I * H // 16 + 4
    w2_bytes = H * I // 2 + H * I // 16 + 4
    rec = {
        "metric": "NVFP4 MoE layer tok/s; decode HBM GB/s and prefill MFMA % of peak",
        "value": None, "unit": "tok/s per MoE layer", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4-w4a4/fp32-acc",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) router and expert weights packed as NVFP4)",
        "config": {"workload": "decode MoE layer: hidden 2048, 512 experts, top-10 + 1 shared, intermediate 512, "
                               "%d tokens per step (MTP K=3 verify window), rotating over %d layers of distinct "
                               "weights" % (T, args.layers),
                   "tokens_per_step": T, "layers_rotated": args.layers, "parallelism": "single GPU"},
        "roofline": None, "cpu_baseline": None, "detail": {},
    }
    rec["detail"]["clocks_start"] = None if args.no_clocks else read_clocks()

    # plain 1 GiB device copy: the practical HBM bandwidth of this machine
    a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = ev(), ev()
    e0.record(stream)
    for _ in range(5):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    rec["detail"]["copy_1GiB_GBs"] = round(copy_gbs, 1)
    del a, b

    host_layer0 = None
    if not args.no_decode:
        layers = []
        t0 = time.time()
        for l in range(args.layers):
            Lh = gen.make_layer(4, layer=l)
            layers.append(device_layer(Lh))
            if l == 0:
                host_layer0 = Lh
            del Lh
            if l % 8 == 7 or l == args.layers - 1:
                log("stack layers 0..%d generated and uploaded (%.1f s)" % (l, time.time() - t0))
        torch.cuda.synchronize()

        def decode_leg(T, K, W):
            pool = [up(gen.make_tokens(4, T, step=s).view(np.int16)) for s in range(args.pool)]
            buf = moe.Buffers(layers[0], T, dev)
            n_total = W + K
            # per-step records of the selection, each row padded to 16 bytes (the
            # library takes 16-byte aligned pointers)
            pad = (T * k + 3) // 4 * 4
            rec_idx = torch.empty((n_total, pad), dtype=torch.int32, device=dev)
            rec_w = torch.empty((n_total, pad), dtype=torch.float32, device=dev)
            sel = lambda a, i: a[i, :T * k].view(T, k)
            events = [[ev() for _ in range(2 * moe.FFN_KERNELS)] for _ in range(n_total)]
            torch.cuda.synchronize()

            def step(i, timed_events=True):
                DL = layers[i % len(layers)]
                x = pool[i % len(pool)]
                dbg = {"events": events[i]} if timed_events else None
                moe.moe_layer_forward(DL, x, buf, T=T, debug=dbg, topk=(sel(rec_idx, i), sel(rec_w, i)))

            # eager launches: per-kernel durations from the kernels' own timestamps
            for i in range(W):
                step(i)
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for i in range(W, W + K):
                step(i)
            torch.cuda.synchronize()
            eager_s = time.perf_counter() - t_start
            log("T=%d: %d eager steps in %.4f s" % (T, K, eager_s))

            def avg_ms(a, b):
                return float(np.mean([events[i][a].elapsed_time(events[i][b]) for i in range(W, W + K)]))

            out = {"T": T, "eager_s": eager_s, "eager_tok_s": T * K / eager_s,
                   "t_first": avg_ms(0, 1), "t_gateup": avg_ms(2, 3), "t_down": avg_ms(4, 5)}
            idx = rec_idx[W:, :T * k].cpu().numpy()
            n_distinct = np.array([len(np.unique(idx[i])) for i in range(K)], dtype=np.float64)
            rows = T * k + T
            act_in = T * (H // 2 + H // 16)
            h_out = rows * (I // 2 + I // 16)
            logits = T * E * 8  # FP64 router logits, read by the routing selection inside gate/up
            out.update({
                "n_distinct": float(n_distinct.mean()),
                "gateup_bytes": float(np.mean((n_distinct + 1) * w13_bytes)) + act_in + h_out + logits,
                # down projection with the combine: W2 of the distinct experts, A4(h) read,
                # the FP32 rows written, the BF16 output written
                "down_bytes": float(np.mean((n_distinct + 1) * w2_bytes)) + h_out + rows * H * 4 + T * H * 2,
                "layer_bytes": 4 * E * H + float(np.mean((n_distinct + 1) * (w13_bytes + w2_bytes))) + T * H * 2 * 2,
            })
            if args.graph_steps > 0:
                # exactly K steps (the same layer and token rotation) in one HIP graph
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(W, W + K):
                        step(i, timed_events=False)
                torch.cuda.synchronize()
                g.replay()  # warm replay
                torch.cuda.synchronize()
                g0, g1 = ev(), ev()
                torch.cuda.synchronize()
                h0 = time.perf_counter()
                g0.record(stream)
                g.replay()
                g1.record(stream)
                torch.cuda.synchronize()
                host_s = time.perf_counter() - h0
                timed_ms = g0.elapsed_time(g1)
                log("T=%d graph: %d steps in %.4f ms (host %.4f ms)" % (T, K, timed_ms, host_s * 1e3))
                # spread: further replays, each timed with events
                reps = max(math.ceil(args.spread_steps / K), math.ceil(100.0 / max(timed_ms, 1e-3)))
                reps = min(reps, 2000)
                evs = [(ev(), ev()) for _ in range(reps)]
                torch.cuda.synchronize()
                for a_, b_ in evs:
                    a_.record(stream)
                    g.replay()
                    b_.record(stream)
                torch.cuda.synchronize()
                per_step_us = [a_.elapsed_time(b_) * 1e3 / K for a_, b_ in evs]
                out.update({"graph_ms": timed_ms, "graph_host_s": host_s, "graph_tok_s": T * K / (timed_ms * 1e-3),
                            "spread_replays": reps, "spread_steps": reps * K,
                            "us_per_step_median": pct(per_step_us, 50), "us_per_step_p10": pct(per_step_us, 10),
                            "us_per_step_p90": pct(per_step_us, 90)})
                del g
            del buf, pool, events
            return out

        d = decode_leg(T, K, W)
        d1 = None if (T == 1 or args.skip_t1) else decode_leg(1, K, W)
        achieved = d["gateup_bytes"] / (d["t_gateup"] * 1e-3) / 1e9
        if "graph_tok_s" in d:
            rec["value"] = round(d["graph_tok_s"], 1)
            rec["ms_per_step"] = round(d["graph_ms"] / K, 6)
            rec["config"]["launch"] = "one HIP graph of the %d timed steps, timed by HIP events" % K
        else:
            rec["value"] = round(d["eager_tok_s"], 1)
            rec["ms_per_step"] = round(d["eager_s"] * 1e3 / K, 6)
            rec["config"]["launch"] = "eager (one host launch per kernel)"
        rec["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                           "kernel": "k_gateup_decode<true, false, true>", "algorithmic_bytes_per_launch": round(d["gateup_bytes"]),
                           "avg_duration_us": round(d["t_gateup"] * 1e3, 3),
                           "frac_of_copy_bandwidth": round(achieved / copy_gbs, 4)}

        def summary(d):
            s = {
                "eager_tok_s": round(d["eager_tok_s"], 1),
                "kernel_avg_us": {"route_logits_and_act_quant": round(d["t_first"] * 1e3, 3),
                                  "gateup": round(d["t_gateup"] * 1e3, 3),
                                  "down_and_combine": round(d["t_down"] * 1e3, 3)},
                "gateup_achieved_GBs": round(d["gateup_bytes"] / (d["t_gateup"] * 1e-3) / 1e9, 1),
                "down_and_combine_achieved_GBs": round(d["down_bytes"] / (d["t_down"] * 1e-3) / 1e9, 1),
                "distinct_experts_per_step": round(d["n_distinct"], 3),
                "layer_algorithmic_bytes": round(d["layer_bytes"]),
            }
            if "graph_tok_s" in d:
                s.update({"hip_graph_tok_s": round(d["graph_tok_s"], 1),
                          "us_per_step": {"timed": round(d["graph_ms"] * 1e3 / K, 3),
                                          "median": round(d["us_per_step_median"], 3),
                                          "p10": round(d["us_per_step_p10"], 3), "p90": round(d["us_per_step_p90"], 3),
                                          "replays": d["spread_replays"], "steps": d["spread_steps"]},
                          "layer_effective_GBs": round(d["layer_bytes"] / (d["us_per_step_median"] * 1e-6) / 1e9, 1)})
            return s

        rec["detail"]["decode_T%d" % T] = summary(d)
        if d1 is not None:
            rec["detail"]["decode_T1"] = summary(d1)

        # ------------------------------------------------------------ layer variants
        # the same 48 layers and token rotation at T tokens per step, one HIP graph of
        # K steps per variant: the W4A8 activation encoding and the shared expert's gate
        if args.graph_steps > 0 and not args.no_variants:
            wg = (torch.randn(H, generator=torch.Generator().manual_seed(4242)) * 0.02).float().to(dev)
            pool_v = [up(gen.make_tokens(4, T, step=s).view(np.int16)) for s in range(args.pool)]

            def graph_us(variant):
                lv = [variant(DL) for DL in layers]
                bv = moe.Buffers(lv[0], T, dev)

                def run():
                    for i in range(K):
                        moe.moe_layer_forward(lv[i % len(lv)], pool_v[i % len(pool_v)], bv, T=T)

                run()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    run()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                evs = [(ev(), ev()) for _ in range(max(3, math.ceil(args.spread_steps / K)))]
                for a_, b_ in evs:
                    a_.record(stream)
                    g.replay()
                    b_.record(stream)
                torch.cuda.synchronize()
                us = pct([a_.elapsed_time(b_) * 1e3 / K for a_, b_ in evs], 50)
                del g, bv
                return round(us, 3)

            var = {"tokens_per_step": T, "w4a4_us_per_step": round(d.get("us_per_step_median", float("nan")), 3)}
            var["w4a8_us_per_step"] = graph_us(lambda DL: DL.with_act_bits(8))
            var["shared_gate_us_per_step"] = graph_us(lambda DL: DL.with_shared_gate(wg))
            rec["detail"]["decode_variants"] = var
            log("decode variants (us per step at T=%d): %s" % (T, var))
            del pool_v

        # ------------------------------------------------------------ the stack
        if not args.no_stack:
            stack = {}
            # each layer one call: the RMS norm of the residual stream inside moe_layer_forward
            # (pre_norm; identical to moe_rms_norm followed by the layer), the residual added
            # in its combine
            layers_pn = [DL.with_pre_norm(1e-6) for DL in layers]
            for Ts in (1, 4):
                x0 = up(gen.make_tokens(4, Ts, step=777).view(np.int16))
                bufs = [moe.Buffers(layers_pn[0], Ts, dev), moe.Buffers(layers_pn[0], Ts, dev)]

                def stack_pass():
                    xl = x0
                    for l, DLn in enumerate(layers_pn):
                        xl = moe.moe_layer_forward(DLn, xl, bufs[l % 2], residual=xl, T=Ts)

                stack_pass()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    stack_pass()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                reps = 50
                evs = [(ev(), ev()) for _ in range(reps)]
                torch.cuda.synchronize()
                for a_, b_ in evs:
                    a_.record(stream)
                    g.replay()
                    b_.record(stream)
                torch.cuda.synchronize()
                us = [a_.elapsed_time(b_) * 1e3 for a_, b_ in evs]
                stack["T%d" % Ts] = {"us_per_pass_median": round(pct(us, 50), 2), "us_per_pass_p10": round(pct(us, 10), 2),
                                     "us_per_pass_p90": round(pct(us, 90), 2),
                                     "us_per_token": round(pct(us, 50) / Ts, 2),
                                     "us_per_layer": round(pct(us, 50) / len(layers), 3), "replays": reps}
                log("stack T=%d: %.1f us per pass through %d layers" % (Ts, pct(us, 50), len(layers)))
                del g, bufs, x0
            stack["workload"] = ("%d layers of the decode shape with distinct weights (%.1f GB), each one "
                                 "moe_layer_forward call: RMS norm of the residual stream (pre_norm), the MoE layer "
                                 "with the residual added in its combine; one HIP graph per pass"
                                 % (len(layers), len(layers) * 0.912))
            rec["detail"]["stack"] = stack
        del layers

    # ---------------------------------------------------------------- prefill chunks
    def prefill_leg(cfg_p, Tp, n):
        t0 = time.time()
        Lp = gen.make_layer(cfg_p)
        # once per layer, outside any timed region: the K-step-major weight copies the
        # matrix-core kernels read and the router's BF16 pieces
        DLp = device_layer(Lp).pack_kmajor().pack_router()
        xp = up(gen.make_tokens(cfg_p, Tp).view(np.int16))
        log("prefill layer and %d tokens generated (%.1f s)" % (Tp, time.time() - t0))
        buf = moe.Buffers(DLp, Tp, dev)
        evs = [[ev() for _ in range(2 * moe.FFN_KERNELS)] for _ in range(n)]
        st = [[ev() for _ in range(3)] for _ in range(n)]
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
                               debug={"events": evs[i]}, T=Tp)
            moe.moe_combine(DLp, buf.y_rows, buf.y_shared, buf.pair2row, buf.topk_w, buf.out, T=Tp)
            st[i][2].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
        med = lambda f: float(np.median([f(i) for i in range(n)]))
        t_chunk = [st[i][0].elapsed_time(st[i][2]) for i in range(n)]
        t_route = med(lambda i: st[i][0].elapsed_time(st[i][1]))
        t_ffn_comb = med(lambda i: st[i][1].elapsed_time(st[i][2]))
        t_g1 = med(lambda i: evs[i][2].elapsed_time(evs[i][3]))
        t_g2 = med(lambda i: evs[i][4].elapsed_time(evs[i][5]))
        rows = Tp * k + Tp
        fl_g1, fl_g2 = 2.0 * rows * H * 2 * I, 2.0 * rows * I * H
        tf = (fl_g1 + fl_g2) / ((t_g1 + t_g2) * 1e-3) / 1e12
        counts = np.diff(buf.expert_off.cpu().numpy())
        out = {
            "workload": "one %d-token chunk, same layer shape, Zipf(1.1)-skewed routing (head expert %d tokens, "
                        "tail %d)" % (Tp, counts.max(), counts.min()),
            "tok_s": round(Tp / (pct(t_chunk, 50) * 1e-3), 1),
            "ms_per_chunk": {"median": round(pct(t_chunk, 50), 4), "p10": round(pct(t_chunk, 10), 4),
                             "p90": round(pct(t_chunk, 90), 4), "chunks": n, "host_wall_ms": round(elapsed * 1e3 / n, 4)},
            "route_permute_ms": round(t_route, 4), "ffn_combine_ms": round(t_ffn_comb, 4),
            "gateup_ms": round(t_g1, 4), "down_ms": round(t_g2, 4),
            "gateup_TFLOPs": round(fl_g1 / (t_g1 * 1e-3) / 1e12, 1),
            "down_TFLOPs": round(fl_g2 / (t_g2 * 1e-3) / 1e12, 1),
            "roofline": {"bound": "mfma", "kernel": "k_gateup_mfma + k_down_mfma (FP16 MFMA on exactly decoded NVFP4)",
                         "achieved": round(tf, 1), "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4),
                         "frac_of_fp8_peak": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                         "flop_per_chunk": fl_g1 + fl_g2, "avg_duration_us": round((t_g1 + t_g2) * 1e3, 2)},
        }
        log("prefill %d: %d chunks, median %.3f ms" % (Tp, n, pct(t_chunk, 50)))
        if cfg_p == 3:
            # the router alone in each precision mode (same chunk, same cached BF16 pieces)
            modes = {}
            for name, mode in (("exact", moe.MOE_ROUTER_EXACT), ("split3_f32", moe.MOE_ROUTER_SPLIT3_F32),
                               ("bf16", moe.MOE_ROUTER_BF16)):
                Lm = DLp.with_router_mode(mode)
                moe.moe_route(Lm, xp, buf.topk_idx, buf.topk_w, buf.ws, T=Tp)
                pairs = [(ev(), ev()) for _ in range(n)]
                for a_, b_ in pairs:
                    a_.record(stream)
                    moe.moe_route(Lm, xp, buf.topk_idx, buf.topk_w, buf.ws, T=Tp)
                    b_.record(stream)
                torch.cuda.synchronize()
                modes[name] = round(pct([a_.elapsed_time(b_) for a_, b_ in pairs], 50), 4)
            out["route_ms_by_router_mode"] = modes
            log("router modes (ms): %s" % modes)
            if not args.no_variants:
                # the whole chunk through moe_layer_forward per layer variant
                wg = (torch.randn(H, generator=torch.Generator().manual_seed(4242)) * 0.02).float().to(dev)
                vms = {}
                for name, Lv in (("w4a4", DLp), ("w4a8", DLp.with_act_bits(8)), ("shared_gate", DLp.with_shared_gate(wg))):
                    bv = moe.Buffers(Lv, Tp, dev)
                    moe.moe_layer_forward(Lv, xp, bv, T=Tp)
                    pairs = [(ev(), ev()) for _ in range(n)]
                    for a_, b_ in pairs:
                        a_.record(stream)
                        moe.moe_layer_forward(Lv, xp, bv, T=Tp)
                        b_.record(stream)
                    torch.cuda.synchronize()
                    vms[name] = round(pct([a_.elapsed_time(b_) for a_, b_ in pairs], 50), 4)
                    del bv
                out["layer_forward_ms_by_variant"] = vms
                log("prefill variants (ms per chunk): %s" % vms)
        return out, DLp, buf

    if args.prefill_tokens > 0:
        Tp = args.prefill_tokens
        p3, DLp, buf = prefill_leg(3, Tp, args.prefill_steps)
        rec["detail"]["prefill"] = p3
        if rec["value"] is None:  # prefill-only run (profiling)
            rec["value"] = p3["tok_s"]
            rec["ms_per_step"] = p3["ms_per_chunk"]["median"]
            rec["config"] = {"workload": p3["workload"], "tokens_per_step": Tp, "parallelism": "single GPU"}
        # streamed prompt: the same layer over a long prompt in equal chunks (each
        # chunk one library call with the residual added in its combine)
        if args.stream_tokens > 0:
            Ts, nc = args.stream_tokens, args.stream_chunks
            cs = Ts // nc
            xs_ = up(gen.make_tokens(3, Ts, step=55).view(np.int16))
            rs_ = up(gen.make_tokens(3, Ts, step=56).view(np.int16))
            del buf
            bufs = moe.Buffers(DLp, cs, dev)
            outs = torch.empty((Ts, H), dtype=torch.int16, device=dev)

            def prompt():
                for c in range(nc):
                    o = moe.moe_layer_forward(DLp, xs_[c * cs:(c + 1) * cs], bufs, residual=rs_[c * cs:(c + 1) * cs])
                    outs[c * cs:(c + 1) * cs].copy_(o[:cs])

            prompt()
            torch.cuda.synchronize()
            reps = 5
            evs = [(ev(), ev()) for _ in range(reps)]
            for a_, b_ in evs:
                a_.record(stream)
                prompt()
                b_.record(stream)
            torch.cuda.synchronize()
            ms = [a_.elapsed_time(b_) for a_, b_ in evs]
            rec["detail"]["streamed_prefill"] = {
                "workload": "a %d-token prompt as %d chunks of %d tokens, residual added, same layer" % (nc * cs, nc, cs),
                "tok_s": round(nc * cs / (pct(ms, 50) * 1e-3), 1), "ms_per_prompt": round(pct(ms, 50), 4)}
            log("streamed prefill: %d prompts, median %.3f ms" % (reps, pct(ms, 50)))
            del bufs, xs_, rs_, outs
        del DLp
    if args.c2_tokens > 0:
        p2, DLp, buf = prefill_leg(2, args.c2_tokens, args.prefill_steps)
        rec["detail"]["prefill_4096" if args.c2_tokens == 4096 else "prefill_%d" % args.c2_tokens] = p2
        del DLp, buf
    torch.cuda.synchronize()
    rec["detail"]["clocks_end"] = None if args.no_clocks else read_clocks()

    # ---------------------------------------------------------------- oracle on the host
    if args.cpu_seconds > 0 and host_layer0 is not None:
        import oracle

        threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        os.environ.setdefault("OMP_NUM_THREADS", str(threads))
        n_tok, t_cpu, s = 0, 0.0, 0
        while t_cpu < args.cpu_seconds and s < args.pool:
            x = gen.make_tokens(4, T, step=s)
            c0 = time.perf_counter()
            oracle.layer(host_layer0, x)
            t_cpu += time.perf_counter() - c0
            n_tok += T
            s += 1
        omp = int(os.environ.get("OMP_NUM_THREADS", threads))
        rec["cpu_baseline"] = {
            "value": round(n_tok / t_cpu, 3), "unit": "tok/s per MoE layer", "cores": min(omp, threads),
            "kind": "oracle",
            "sample": "%d decode batches of %d tokens through layer 0 of the stack (%d tokens, %.1f s of FP64 oracle)" % (
                s, T, n_tok, t_cpu)}
        log("oracle: %d tokens in %.1f s" % (n_tok, t_cpu))

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the MI355X MoE expert FFN hot path.

Headline (one JSON line on stdout): microseconds per MoE FFN layer at 512
tokens per GPU -- one GPU's share of an EP8 DeepSeek-V4-style layer
(route 512 own tokens; scatter, GEMM1, live-row act-quant, GEMM2 and
combine for the 8x512-token group's routes to this GPU's 32 experts).
Inputs are seeded synthetic data already resident in HBM when the timed
region starts. A step is one pass of route -> scatter -> GEMM1 -> act-quant
-> GEMM2 -> combine. The headline is cold: the six launches are captured
once into a HIP graph, and each of the K timed replays follows a 512 MB read
that evicts the L2s and the Infinity Cache (HIP events bracket the replay
alone; the median is reported, the warm back-to-back rate beside it). Eager
steps, each after the same read, give the per-kernel durations from HIP
events around every launch.

The same line carries:
  roofline      the dominant kernel (GEMM1 with the fused act-quant) against
                HBM peak: duration by HIP events, and by the committed kernel
                trace while the kernel's sources match it
  kernels       per-kernel durations, algorithmic bytes / FLOP, GB/s, TFLOP/s
  layers        the same chain on the tiny and the large-expert-count layers
  actquant      the standalone live-row act-quant benchmark (3,072 live of
                28,672 rows, width 2,048; SiLU and SiTU) and its full-buffer
                control, cold
  decode        the sparse decode layer at 1 and 8 tokens (FP8 and MXFP4):
                per-kernel cold durations and the graph-replayed layer
  masked        the headline layer on the masked (E, m_pad, K) slab layout
  natural_weights  GEMM1 + act-quant and GEMM2 on checkpoint-layout weights
  cpu_baseline  the CPU oracle on the host: the headline layer on all threads
                (the value) and, per workload, on one thread and on all

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras]
                       [--no-cpu-baseline] [--copy-calibration]
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 / MXFP8 matrix peak
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix peak


# Counter-derived HBM traffic of the dominant kernel is taken from the
# committed rocprofv3 summary; it is reported only while the kernel's sources
# still hash to the value recorded when the counters were read.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_mx_gemm1_act_quant_prefill_ep_share_hbm_traffic.txt")
TRACE_FILE = os.path.join(ROOT, "profiles", "prefill_ep_share_layer_kernel_trace.txt")
GEMM_SOURCES = ("mixture_experts_ffn_scatter_amd/csrc/gemm.hip",
                "mixture_experts_ffn_scatter_amd/csrc/common.h",
                "mixture_experts_ffn_scatter_amd/csrc/sigmoid_lookup.h")


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per GEMM1 launch (FETCH_SIZE + WRITE_SIZE, copy-scaled), or
    None when no summary matches the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("TRAFFIC "):
                    rec = json.loads(line[len("TRAFFIC "):])
                    if rec.get("source_sha256") == gemm_source_hash():
                        return int(rec["fetch_bytes"]) + int(rec["write_bytes"])
    except OSError:
        pass
    return None


def trace_avg_launch_us():
    """GEMM1's mean duration per launch from the committed rocprofv3 kernel
    trace of the headline command (its eager-cold window), or None when the
    kernel's sources changed since that trace was taken."""
    try:
        with open(TRACE_FILE) as fh:
            for line in fh:
                if line.startswith("TRACE "):
                    rec = json.loads(line[len("TRACE "):])
                    if rec.get("source_sha256") == gemm_source_hash():
                        return float(rec["avg_launch_us"])
    except OSError:
        pass
    return None


def local_counts(ids: np.ndarray, expert_start: int, E_local: int) -> np.ndarray:
    """Routes per local expert (the live rows the grouped kernels process)."""
    e = ids.reshape(-1).astype(np.int64) - expert_start
    return np.bincount(e[(e >= 0) & (e < E_local)], minlength=E_local)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--unfused", action="store_true",
                   help="time GEMM1 and the live-row act-quant as two launches")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run 4 plain 1 GiB device copies (the reference kernel that "
                        "scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--only", choices=["actquant", "decode", "layers"],
                   help="run only that extra measurement (for per-kernel profiles) and exit")
    return p.parse_args()


def copy_calibration():
    """Four device-to-device copies of exactly 1 GiB through torch's copy kernel:
    under rocprofv3 --pmc their FETCH_SIZE and WRITE_SIZE per dispatch give the
    counter's reading for a known 2^30 bytes read and written."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 4}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path is "
              "built for one GPU's expert share: with expert parallelism each GPU would run "
              "this same chain on the rows it receives)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import mixture_experts_ffn_scatter_amd as pkg
    import workloads as W

    ops = pkg.ops
    pkg.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def up_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    if args.only:
        fn = {"actquant": bench_actquant, "decode": bench_decode,
              "layers": bench_other_layers}[args.only]
        print(json.dumps({args.only: fn(ops, torch, up, up_bf16, log)}), flush=True)
        return

    # ------------------------------------------------------------ workload
    log("generating the prefill EP-share workload")
    c = W.prefill()
    w = c.weights
    x = up_bf16(c.x)
    logits_group = up(c.logits)
    logits_own = up(c.logits[: c.own_tokens])
    # load-time weight preparation: codes and scales into the GEMMs' fragment
    # order (w13 with gate / up interleaved for the fused GEMM1 + act-quant)
    fused = not args.unfused
    pack13 = ops.moe_pack_mx_weights_gateup if fused else ops.moe_pack_mx_weights
    w13, s13 = pack13(up(w.w13), up(w.s13))
    w2, s2 = ops.moe_pack_mx_weights(up(w.w2), up(w.s2))
    # the group's routes (every rank routes its own 512 tokens; the 4096
    # tokens' ids are what this GPU receives)
    ids, wts = ops.moe_route(logits_group, c.k, "softmax")
    own_ids = torch.empty((c.own_tokens, c.k), dtype=torch.int32, device=dev)
    own_w = torch.empty((c.own_tokens, c.k), dtype=torch.float32, device=dev)
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I)
    torch.cuda.synchronize()

    names = (["route", "scatter", "gemm1_act", "gemm2", "combine"] if fused else
             ["route", "scatter", "gemm1", "act_quant", "gemm2", "combine"])

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        ops.moe_route(logits_own, c.k, "softmax", None, own_ids, own_w)
        mark(1)
        ops.moe_scatter_endpoints(ids, 0, c.E_local, c.A, x, buf.expert_ends, buf.route_row,
                                  buf.xq, buf.xs, buf.workspace)
        mark(2)
        if fused:
            ops.moe_grouped_gemm1_act_quant(buf.xq, buf.xs, buf.expert_ends, c.A, w13, s13, 0.0,
                                            buf.hq, buf.hs)
        else:
            ops.moe_grouped_gemm1(buf.xq, buf.xs, buf.expert_ends, c.A, w13, s13, buf.gateup)
            mark(3)
            ops.moe_act_quant_liverows(buf.gateup, buf.expert_ends, c.A, 0.0, buf.hq, buf.hs)
        mark(len(names) - 2)
        ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, w2, s2, buf.down)
        mark(len(names) - 1)
        ops.moe_combine(buf.down, buf.route_row, wts, c.routed_scale, buf.out)
        mark(len(names))

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # eager, warm: K steps back to back, host-timed
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    eager_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # per-kernel durations, cold: K eager steps, each after a 512 MB read that
    # evicts the L2s and the 256 MB Infinity Cache. The read also keeps the
    # GPU behind the host, so every launch is queued before its start event
    # is reached and no window holds a host-side launch gap.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        _flush_caches(torch, scratch)
        step(events[i])
    torch.cuda.synchronize()
    dur_us = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in
                                range(args.steps)])) * 1e3 for j, n in enumerate(names)}
    log(f"eager ms/step {eager_ms_per_step:.4f}; per kernel, cold",
        {k: round(v, 2) for k, v in dur_us.items()})

    # the headline: the same six launches captured once into a HIP graph and
    # replayed (the chain never reads a count back, so the graph is valid for
    # any routing); K timed replays, bracketed by synchronisation
    graph = ops.capture_graph(lambda: step(None))
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    # warm: K replays back to back (weights partly left in the caches by the
    # previous replay)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    warm_ms_per_step = (t1 - t0) * 1e3 / args.steps
    # cold (the headline): before each of the K timed replays a 512 MB read
    # evicts the L2s and the 256 MB Infinity Cache, outside the HIP events
    # that bracket the replay, so every input comes from HBM
    cold = []
    torch.cuda.synchronize()
    for _ in range(args.steps):
        _flush_caches(torch, scratch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    del scratch
    ms_per_step = float(np.median(cold))
    log(f"graph ms/step cold {ms_per_step:.4f} (p10 {np.percentile(cold, 10):.4f}, p90 "
        f"{np.percentile(cold, 90):.4f}), warm {warm_ms_per_step:.4f}")
    del graph

    # algorithmic work per launch, from the routed counts of this input
    ids_h = ids.cpu().numpy()
    counts = local_counts(ids_h, 0, c.E_local)
    R = int(counts.sum())
    E_ne = int(np.count_nonzero(counts))
    H, I, T, k, E = c.H, c.I, c.T, c.k, c.E
    U_tok = int(np.count_nonzero(np.any((ids_h >= 0) & (ids_h < c.E_local), axis=1)))
    bytes_ = {
        "route": c.own_tokens * E * 4 + c.own_tokens * k * 8,
        "scatter": U_tok * H * 2 + R * (H + H // 32) + T * k * 8 + 4 * c.E_local,
        "gemm1": E_ne * (2 * I * H // 2 + 2 * I * H // 32) + R * (H + H // 32) + R * 2 * I * 2,
        "act_quant": R * (2 * I * 2 + I + I // 32) + 4 * c.E_local,
        "gemm1_act": E_ne * (2 * I * H // 2 + 2 * I * H // 32) + R * (H + H // 32) + R * (I + I // 32),
        "gemm2": E_ne * (H * I // 2 + H * I // 32) + R * (I + I // 32) + R * H * 2,
        "combine": R * H * 2 + T * k * 8 + T * H * 2,
    }
    flops = {"gemm1": 2.0 * R * 2 * I * H, "gemm1_act": 2.0 * R * 2 * I * H, "gemm2": 2.0 * R * H * I}
    kernels = {}
    for n in names:
        t = dur_us[n] * 1e-6
        kernels[n] = {"us": round(dur_us[n], 3), "alg_bytes": int(bytes_[n]),
                      "GBps": round(bytes_[n] / t / 1e9, 1),
                      "hbm_frac": round(bytes_[n] / t / 1e9 / HBM_PEAK_GBS, 4)}
        if n in flops:
            tf = flops[n] / t / 1e12
            kernels[n].update({"flop": flops[n], "TFLOPs": round(tf, 1),
                               "mfma_frac_fp8_peak": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                               "mfma_frac_fp4_peak": round(tf / FP4_MFMA_PEAK_TFLOPS, 4)})
    dom = "gemm1_act" if fused else "gemm1"
    ach = bytes_[dom] / (dur_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm",
                "kernel": ("grouped_mx_gemm_kernel<true, false, false> (moe_grouped_gemm1_act_quant)" if fused
                           else "grouped_mx_gemm_kernel<false, false, false> (moe_grouped_gemm1)"),
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": counter_traffic(),
                "alg_bytes_per_launch": int(bytes_[dom]), "avg_launch_us": round(dur_us[dom], 3),
                # the same launch against the matrix cores (its FLOP / time / dense FP8 peak)
                "mfma_frac_fp8_peak": kernels[dom]["mfma_frac_fp8_peak"]}
    tr = trace_avg_launch_us() if fused else None
    if tr is not None:
        # the same launches by the committed kernel trace (no event packets
        # or dispatch in the window)
        roofline["avg_launch_us_trace"] = tr
        roofline["frac_trace"] = round(bytes_[dom] / (tr * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)

    result = {
        "metric": "MoE FFN us/layer @512 tok; live-row act-quant GB/s; % of HBM/MFMA roofline",
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "timing": "cold: median of K graph replays, each after a 512 MB read that evicts the "
                  "caches (HIP events around the replay only)",
        "warm_ms_per_step": round(warm_ms_per_step, 5),
        "cold_ms_p10_p90": [round(float(np.percentile(cold, 10)), 5),
                            round(float(np.percentile(cold, 90)), 5)],
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3 x mxfp4 (fp32 accum), bf16 io",
        "data": "synthetic",
        "config": {"workload": "prefill EP share: 512 tok/GPU x EP8 = 4096-token group, top-6 of "
                               "256 experts, 32 local experts, H=4096, I=2048, A=128, MXFP4 "
                               "weights, FP8 e4m3 + UE8M0 group-32 activations",
                   "live_rows": R, "nonempty_experts": E_ne, "M_cap": c.M_cap},
        "roofline": roofline,
        "kernels": kernels,
    }
    del buf
    torch.cuda.empty_cache()

    if not args.no_extras:
        result["recipe_g128"] = bench_g128(ops, torch, up, c, ids, wts, logits_own, own_ids,
                                           own_w, log)
        result["layers"] = bench_other_layers(ops, torch, up, up_bf16, log)
        result["actquant"] = bench_actquant(ops, torch, up, up_bf16, log)
        result["decode"] = bench_decode(ops, torch, up, up_bf16, log)
        result["masked"] = bench_masked(ops, torch, up, up_bf16, log, c, ids, wts, logits_own,
                                        own_ids, own_w, fused)
        result["natural_weights"] = bench_natural(ops, torch, up, up_bf16, log, c, ids)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(c, log)
    print(json.dumps(result), flush=True)


def bench_g128(ops, torch, up, c, ids, wts, logits_own, own_ids, own_w, log, steps=20, warmup=5):
    """The same layer with the group-128 activation recipe (scatter, GEMM1
    with its fused act-quant epilogue, and GEMM2, with one UE8M0 byte per 128
    activation columns): per-kernel HIP-event times of eager steps and the
    graph-replayed step."""
    w = c.weights
    w13, s13 = ops.moe_pack_mx_weights_gateup(up(w.w13), up(w.s13))
    w2, s2 = ops.moe_pack_mx_weights(up(w.w2), up(w.s2))
    x = torch.from_numpy(np.ascontiguousarray(c.x).view(np.int16)).cuda().view(torch.bfloat16)
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I, group=128)
    names = ["route", "scatter", "gemm1_act", "gemm2", "combine"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        ops.moe_route(logits_own, c.k, "softmax", None, own_ids, own_w)
        mark(1)
        ops.moe_scatter_endpoints(ids, 0, c.E_local, c.A, x, buf.expert_ends, buf.route_row,
                                  buf.xq, buf.xs, buf.workspace, group=128)
        mark(2)
        ops.moe_grouped_gemm1_act_quant(buf.xq, buf.xs, buf.expert_ends, c.A, w13, s13, 0.0, buf.hq,
                                        buf.hs, group=128)
        mark(3)
        ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, w2, s2, buf.down, group=128)
        mark(4)
        ops.moe_combine(buf.down, buf.route_row, wts, c.routed_scale, buf.out)
        mark(5)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    dur = {n: round(float(np.mean([events[i][j].elapsed_time(events[i][j + 1])
                                   for i in range(steps)])) * 1e3, 3) for j, n in enumerate(names)}
    graph = ops.capture_graph(lambda: step(None))
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / steps
    del graph, buf
    torch.cuda.empty_cache()
    log("recipe g128", round(us, 2), dur)
    return {"us_per_layer_graph": round(us, 2), "kernels_us": dur,
            "note": "GEMM1 with its fused group-128 act-quant epilogue"}


def bench_masked(ops, torch, up, up_bf16, log, c, ids, wts, logits_own, own_ids, own_w, fused,
                 steps=20, warmup=5):
    """The same EP-share layer on the masked slab layout: every local expert
    owns a fixed block of m_pad rows. Two capacities: the group's token count
    (4,096; no expert can overflow it) and the busiest expert's count
    rounded up to 256 (known here from the routing; a caller would need a
    device-to-host read for it). Per-kernel durations of cold eager steps
    and the cold graph-replayed layer."""
    w = c.weights
    pack13 = ops.moe_pack_mx_weights_gateup if fused else ops.moe_pack_mx_weights
    w13, s13 = pack13(up(w.w13), up(w.s13))
    w2, s2 = ops.moe_pack_mx_weights(up(w.w2), up(w.s2))
    x = up_bf16(c.x)
    counts = local_counts(ids.cpu().numpy(), 0, c.E_local)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for label, m_pad in (("m_pad_tokens", c.T), ("m_pad_max_count", (int(counts.max()) + 255) // 256 * 256)):
        buf = ops.alloc_masked(c.T, c.k, c.E_local, m_pad, c.H, c.I)
        names = (["route", "scatter", "gemm1_act", "gemm2", "combine"] if fused else
                 ["route", "scatter", "gemm1", "act_quant", "gemm2", "combine"])

        def step(ev=None):
            def mark(i):
                if ev is not None:
                    ev[i].record()
            mark(0)
            ops.moe_route(logits_own, c.k, "softmax", None, own_ids, own_w)
            mark(1)
            ops.moe_scatter_masked(ids, 0, x, buf.masked_m, buf.route_row, buf.xq, buf.xs,
                                   buf.workspace)
            mark(2)
            if fused:
                ops.moe_grouped_gemm1_act_quant_masked(buf.xq, buf.xs, buf.masked_m, w13, s13, 0.0,
                                                       buf.hq, buf.hs)
            else:
                ops.moe_grouped_gemm1_masked(buf.xq, buf.xs, buf.masked_m, w13, s13, buf.gateup)
                mark(3)
                ops.moe_act_quant_masked(buf.gateup, buf.masked_m, 0.0, buf.hq, buf.hs)
            mark(len(names) - 2)
            ops.moe_grouped_gemm2_masked(buf.hq, buf.hs, buf.masked_m, w2, s2, buf.down)
            mark(len(names) - 1)
            ops.moe_combine(buf.down.view(c.E_local * m_pad, c.H), buf.route_row, wts,
                            c.routed_scale, buf.out)
            mark(len(names))

        for _ in range(warmup):
            step()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            _flush_caches(torch, scratch)
            step(evs[i])
        torch.cuda.synchronize()
        dur = {n: round(float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1])
                                       for i in range(steps)])) * 1e3, 3)
               for j, n in enumerate(names)}
        graph = ops.capture_graph(lambda: step(None))
        for _ in range(warmup):
            graph.replay()
        cold = []
        for _ in range(steps):
            _flush_caches(torch, scratch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            e1.synchronize()
            cold.append(e0.elapsed_time(e1) * 1e3)
        del graph
        used = [buf.xq, buf.xs, buf.hq, buf.hs, buf.down] + ([] if fused else [buf.gateup])
        slab_bytes = sum(t.numel() * t.element_size() for t in used)
        out[label] = {"m_pad": m_pad, "us_per_layer_graph_cold": round(float(np.median(cold)), 2),
                      "kernels_us_cold": dur, "slab_buffer_bytes": int(slab_bytes)}
        log(f"masked {label}", out[label])
        del buf
        torch.cuda.empty_cache()
    del scratch, w13, s13, w2, s2, x
    torch.cuda.empty_cache()
    return out


def bench_natural(ops, torch, up, up_bf16, log, c, ids, steps=20):
    """The EP-share layer's GEMM1 + act-quant and GEMM2 on checkpoint-layout
    weights (no load-time packing), cold, beside the packed forms in the
    same loop: per-kernel HIP-event durations."""
    w = c.weights
    x = up_bf16(c.x)
    buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I)
    ops.moe_scatter_endpoints(ids, 0, c.E_local, c.A, x, buf.expert_ends, buf.route_row, buf.xq,
                              buf.xs, buf.workspace)
    w13, s13, w2, s2 = up(w.w13), up(w.s13), up(w.w2), up(w.s2)
    g13, gs13 = ops.moe_pack_mx_weights_gateup(w13, s13)
    p2, ps2 = ops.moe_pack_mx_weights(w2, s2)
    calls = {
        "gemm1_act_packed": lambda: ops.moe_grouped_gemm1_act_quant(
            buf.xq, buf.xs, buf.expert_ends, c.A, g13, gs13, 0.0, buf.hq, buf.hs),
        "gemm1_act_natural": lambda: ops.moe_grouped_gemm1_act_quant_natural(
            buf.xq, buf.xs, buf.expert_ends, c.A, w13, s13, 0.0, buf.hq, buf.hs),
        "gemm2_packed": lambda: ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, p2,
                                                      ps2, buf.down),
        "gemm2_natural": lambda: ops.moe_grouped_gemm2_natural(buf.hq, buf.hs, buf.expert_ends,
                                                               c.A, w2, s2, buf.down),
    }
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for name, call in calls.items():
        for _ in range(3):
            call()
        ts = []
        for _ in range(steps):
            _flush_caches(torch, scratch)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        out[name] = round(float(np.median(ts)), 3)
    log("natural weights (us, cold)", out)
    del buf, scratch, w13, s13, w2, s2, g13, gs13, p2, ps2, x
    torch.cuda.empty_cache()
    return {"kernels_us_cold": out}


def _flush_caches(torch, scratch):
    """Evict the L2s and the 256 MB Infinity Cache by reading 512 MB. A read
    leaves clean lines behind; a write-based flush would leave dirty lines
    whose write-back steals bandwidth from the next kernel."""
    scratch.view(torch.int64).sum()


def bench_other_layers(ops, torch, up, up_bf16, log, steps=20, warmup=5):
    """The whole chain (route, scatter, fused GEMM1 + act-quant, GEMM2,
    combine) on the tiny layer (64 tokens, 8 experts) and on the
    large-expert-count layer (2,048 tokens, 896 resident experts, top-16
    sigmoid + bias, clamp 25): graph replay time per layer, and per-kernel
    HIP-event durations from an eager loop."""
    import workloads as W
    out = {}
    for name, make in (("tiny", W.tiny), ("large_e", W.large)):
        log(f"layer {name}: generating")
        c = make()
        w = c.weights
        x = up_bf16(c.x)
        logits = up(c.logits)
        bias = up(c.bias) if c.bias is not None else None
        score = "softmax" if c.score == "softmax" else "sigmoid_bias"
        w13, s13 = ops.moe_pack_mx_weights_gateup(up(w.w13), up(w.s13))
        w2, s2 = ops.moe_pack_mx_weights(up(w.w2), up(w.s2))
        ids = torch.empty((c.T, c.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((c.T, c.k), dtype=torch.float32, device="cuda")
        buf = ops.alloc_grouped(c.T, c.k, c.E_local, c.M_cap, c.H, c.I)
        names = ["route", "scatter", "gemm1_act", "gemm2", "combine"]

        def step(ev=None):
            def mark(i):
                if ev is not None:
                    ev[i].record()
            mark(0)
            ops.moe_route(logits, c.k, score, bias, ids, wts)
            mark(1)
            ops.moe_scatter_endpoints(ids, 0, c.E_local, c.A, x, buf.expert_ends, buf.route_row,
                                      buf.xq, buf.xs, buf.workspace)
            mark(2)
            ops.moe_grouped_gemm1_act_quant(buf.xq, buf.xs, buf.expert_ends, c.A, w13, s13,
                                            c.clamp, buf.hq, buf.hs)
            mark(3)
            ops.moe_grouped_gemm2(buf.hq, buf.hs, buf.expert_ends, c.A, w2, s2, buf.down)
            mark(4)
            ops.moe_combine(buf.down, buf.route_row, wts, c.routed_scale, buf.out)
            mark(5)

        for _ in range(warmup):
            step()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        dur = {n: round(float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1])
                                       for i in range(steps)])) * 1e3, 3)
               for j, n in enumerate(names)}
        graph = ops.capture_graph(lambda: step(None))
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / steps
        del graph
        counts = local_counts(ids.cpu().numpy(), 0, c.E_local)
        R = int(counts.sum())
        E_ne = int(np.count_nonzero(counts))
        H, I = c.H, c.I
        b1 = E_ne * (2 * I * H // 2 + 2 * I * H // 32) + R * (H + H // 32) + R * (I + I // 32)
        b2 = E_ne * (H * I // 2 + H * I // 32) + R * (I + I // 32) + R * H * 2
        f1, f2 = 2.0 * R * 2 * I * H, 2.0 * R * H * I
        out[name] = {
            "us_per_layer_graph": round(us, 2), "kernels_us": dur, "live_rows": R,
            "nonempty_experts": E_ne,
            "gemm1_act": {"alg_bytes": int(b1), "hbm_frac": round(b1 / (dur["gemm1_act"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "TFLOPs": round(f1 / (dur["gemm1_act"] * 1e-6) / 1e12, 1)},
            "gemm2": {"alg_bytes": int(b2), "hbm_frac": round(b2 / (dur["gemm2"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "TFLOPs": round(f2 / (dur["gemm2"] * 1e-6) / 1e12, 1)},
        }
        log(f"layer {name}", out[name])
        del buf, w13, s13, w2, s2, x, logits, ids, wts, c, w
        torch.cuda.empty_cache()
    return out


def product_expert_ends(ops, torch, counts, A):
    """expert_ends of a layout with the given per-expert live-row counts, made
    by the library's own scatter: one route per live row (k = 1), routed to
    its expert in expert order, on a zero x of width 128."""
    counts = np.asarray(counts, np.int64)
    E = counts.shape[0]
    R = int(counts.sum())
    ids = torch.from_numpy(np.repeat(np.arange(E, dtype=np.int32), counts)[:, None].copy()).cuda()
    m_cap = ((R + E * A + 3) // 4) * 4
    x = torch.zeros((R, 128), dtype=torch.bfloat16, device="cuda")
    buf = ops.alloc_grouped(R, 1, E, m_cap, 128, 128)
    ops.moe_scatter_endpoints(ids, 0, E, A, x, buf.expert_ends, buf.route_row, buf.xq, buf.xs,
                              buf.workspace)
    torch.cuda.synchronize()
    return buf.expert_ends.clone()


def bench_actquant(ops, torch, up, up_bf16, log, iters=20):
    import workloads as W
    out = {}
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for full in (False, True):
        case = W.actquant(full=full)
        ends = product_expert_ends(ops, torch, case.counts, case.A)
        # every row of the buffer holds N(0,1) data (the kernel reads only the
        # live ones; where they sit is the layout's business)
        reps = -(-case.M_cap // case.live.shape[0])
        gate = up_bf16(np.tile(case.live, (reps, 1))[: case.M_cap])
        hq = torch.empty((case.M_cap, case.I), dtype=torch.uint8, device="cuda")
        hs = torch.empty((case.I // 128, case.M_cap), dtype=torch.int32, device="cuda")
        R = int(case.counts.sum())
        B = R * (2 * case.I * 2 + case.I + case.I // 32) + 4 * case.E_local
        calls = [("", lambda: ops.moe_act_quant_liverows(gate, ends, case.A, 0.0, hq, hs))]
        if not full:   # the SiTU activation (Kimi-K3's 4 / 25) on the live layout
            calls.append(("_situ", lambda: ops.moe_act_quant_liverows_situ(gate, ends, case.A, hq, hs)))
        for suffix, call in calls:
            for _ in range(3):
                call()
            cold, warm = [], []
            for i in range(iters):
                _flush_caches(torch, scratch)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                e2 = torch.cuda.Event(enable_timing=True)
                call()
                e2.record()
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) * 1e3)
                warm.append(e1.elapsed_time(e2) * 1e3)
            t = float(np.median(cold))
            key = ("full_28672_rows" if full else "live_3072_of_28672") + suffix
            out[key] = {"us_cold_median": round(t, 3), "us_warm_median": round(float(np.median(warm)), 3),
                        "alg_bytes": int(B), "GBps_cold": round(B / (t * 1e-6) / 1e9, 1),
                        "hbm_frac_cold": round(B / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "live_rows": R}
            log("actquant", key, out[key])
        del gate, hq, hs
    del scratch
    torch.cuda.empty_cache()
    return out


def bench_decode(ops, torch, up, up_bf16, log, iters=20):
    """The sparse decode layer (32 resident experts, H = 2,880, top-4) at 1
    and 8 tokens, FP8 and MXFP4: per-kernel HIP-event durations of an eager
    cold call (gate_up GEMV with the GLU, down GEMV, combine), and the three
    launches captured into a HIP graph, replayed cold (after a cache-evicting
    read) and warm."""
    import workloads as W
    out = {}
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for wfmt in ("fp8", "mxfp4"):
        base = None
        for T in (1, 8):
            cse = W.decode(T=T, wfmt=wfmt) if base is None else None
            if base is None:
                base = cse
                dw = [up(cse.w_gu), up(cse.s_gu), up_bf16(cse.b_gu), up(cse.w_d), up(cse.s_d),
                      up_bf16(cse.b_d)]
            # activations and routing for this T (weights shared across T)
            rng = np.random.default_rng(4000 + T)
            x = up_bf16(W.to_bf16_bits(rng.standard_normal((T, base.H), dtype=np.float32)))
            logits = up(rng.standard_normal((T, base.E), dtype=np.float32))
            ids, wts = ops.moe_route(logits, base.k, "softmax")
            dbuf = ops.alloc_decode(T, base.k, base.H)

            def chain(ev=None):
                def mark(i):
                    if ev is not None:
                        ev[i].record()
                mark(0)
                ops.moe_sparse_gemv(x, False, ids, 0, base.E, wfmt, dw[0], dw[1], dw[2], dbuf.act,
                                    dbuf.slot_row, glu=True)
                mark(1)
                ops.moe_sparse_gemv(dbuf.act, True, ids, 0, base.E, wfmt, dw[3], dw[4], dw[5],
                                    dbuf.down, None, glu=False)
                mark(2)
                ops.moe_combine(dbuf.down, dbuf.slot_row, wts, 1.0, dbuf.out)
                mark(3)

            for _ in range(3):
                chain()
            per = [[], [], []]
            for i in range(iters):
                _flush_caches(torch, scratch)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                chain(ev)
                torch.cuda.synchronize()
                for j in range(3):
                    per[j].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)
            graph = ops.capture_graph(lambda: chain(None))
            for _ in range(3):
                graph.replay()
            cold, warm = [], []
            for i in range(iters):
                _flush_caches(torch, scratch)
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record()
                graph.replay()
                e1.record()
                graph.replay()
                e2.record()
                torch.cuda.synchronize()
                cold.append(e0.elapsed_time(e1) * 1e3)
                warm.append(e1.elapsed_time(e2) * 1e3)
            del graph
            # the same layer with the GLU applied on load by the down GEMV
            gu_buf = torch.empty((T * base.k, base.N_gu), dtype=torch.bfloat16, device="cuda")

            def chain_on_load():
                ops.moe_sparse_gemv(x, False, ids, 0, base.E, wfmt, dw[0], dw[1], dw[2], gu_buf,
                                    dbuf.slot_row, glu=False)
                ops.moe_sparse_gemv(gu_buf, True, ids, 0, base.E, wfmt, dw[3], dw[4], dw[5],
                                    dbuf.down, None, glu_on_load=True)
                ops.moe_combine(dbuf.down, dbuf.slot_row, wts, 1.0, dbuf.out)

            graph = ops.capture_graph(chain_on_load)
            for _ in range(3):
                graph.replay()
            cold_ol = []
            for i in range(iters):
                _flush_caches(torch, scratch)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                cold_ol.append(e0.elapsed_time(e1) * 1e3)
            del graph, gu_buf
            U = int(np.unique(ids.cpu().numpy()).size)
            H, N = base.H, base.N_gu
            if wfmt == "fp8":
                bpe_gu, bpe_d = N * H + 4, H * H + 4
            else:
                bpe_gu, bpe_d = N * H // 2 + N * H // 32, H * H // 2 + H * H // 32
            B_gu = U * (bpe_gu + N * 2) + T * H * 2 + T * base.k * H * 2
            B_d = U * (bpe_d + H * 2) + 2 * T * base.k * H * 2
            d_gu, d_d, d_c = (float(np.median(v)) for v in per)
            key = f"{wfmt}_T{T}"
            out[key] = {"distinct_experts": U,
                        "gate_up_us_cold": round(d_gu, 3), "down_us_cold": round(d_d, 3),
                        "combine_us_cold": round(d_c, 3),
                        "gate_up_hbm_frac": round(B_gu / (d_gu * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "down_hbm_frac": round(B_d / (d_d * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "gemvs_alg_bytes": int(B_gu + B_d),
                        "gemvs_hbm_frac": round((B_gu + B_d) / ((d_gu + d_d) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "kernel_sum_us": round(d_gu + d_d + d_c, 3),
                        "layer_graph_us_cold": round(float(np.median(cold)), 3),
                        "layer_graph_us_warm": round(float(np.median(warm)), 3),
                        "layer_graph_us_cold_glu_on_load": round(float(np.median(cold_ol)), 3)}
            log("decode", key, out[key])
        del dw, base
        torch.cuda.empty_cache()
    del scratch
    torch.cuda.empty_cache()
    return out


def _host_cpu():
    """The host CPU's model name and the threads this process may use (the
    scheduler affinity, capped by OMP_NUM_THREADS when that is set)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return model, max(n, 1)


def cpu_baseline(c, log):
    """The CPU oracle as it stands, timed on the host cores.

    The headline value is this GPU's whole EP-share layer (route of the 512
    own tokens, then the 4,096-token group's scatter, both MX GEMMs in fp64,
    act-quant and combine) on all the threads this process may use (the
    oracle's per-expert thread pool, one BLAS thread per worker), once.
    ``per_config`` adds, for every workload, the oracle on one thread and on
    all of them; where the oracle has no parallel loop (act-quant, the decode
    chain) one run is reported with threads = 1. Multi-threaded results are
    checked equal to the single-threaded ones."""
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import moe as M
    model, threads = _host_cpu()
    log(f"cpu baseline: {model}, {threads} threads")

    def timed(fn):
        t0 = time.perf_counter()
        r = fn()
        return (time.perf_counter() - t0) * 1e6, r

    def layer(case, workers, ids=None, wts=None):
        w = case.weights
        def run():
            if ids is not None:
                gi, gw = ids, wts
            elif case.score == "softmax":
                own = M.route_softmax(case.logits[: case.own_tokens], case.k)
                gi, gw = (own if case.own_tokens == case.T else M.route_softmax(case.logits, case.k))
            else:
                gi, gw = M.route_sigmoid_bias(case.logits, case.bias, case.k)
            return M.prefill_expert_major(case.x, gi, gw, case.expert_start, case.E_local, case.A,
                                          case.I, w.w13, w.s13, w.w2, w.s2, clamp=case.clamp,
                                          routed_scale=case.routed_scale, workers=workers)
        with threadpool_limits(1):
            return timed(run)

    per = {}
    # prefill EP share: all threads (the headline) and one thread
    us_all, r_all = layer(c, threads)
    us_one, r_one = layer(c, 1)
    same = bool(np.array_equal(r_all.out, r_one.out) and np.array_equal(r_all.hq, r_one.hq))
    per["prefill_ep_share"] = {"us_all_threads": round(us_all, 1), "us_one_thread": round(us_one, 1),
                               "threads": threads, "same_result": same}
    log("cpu prefill_ep_share", per["prefill_ep_share"])
    # tiny layer (64 tokens, 8 experts)
    t = W.tiny()
    a_us, ra = layer(t, threads)
    o_us, ro = layer(t, 1)
    per["tiny"] = {"us_all_threads": round(a_us, 1), "us_one_thread": round(o_us, 1),
                   "threads": threads, "same_result": bool(np.array_equal(ra.out, ro.out))}
    # standalone act-quant, the 3,072 live rows of width 2 x 2,048 (SiLU)
    aq = W.actquant()
    with threadpool_limits(1):
        us, _ = timed(lambda: M.act_quant_rows(aq.live, aq.I))
    per["actquant_live_rows"] = {"us_one_thread": round(us, 1), "threads": 1,
                                 "rows": int(aq.live.shape[0])}
    # sparse decode layer, 32 experts, H = 2,880, top-4
    for wfmt in ("fp8", "mxfp4"):
        for T in (1, 8):
            d = W.decode(T=T, wfmt=wfmt)
            with threadpool_limits(1):
                us, _ = timed(lambda: M.decode_chain(d))
            per[f"decode_{wfmt}_T{T}"] = {"us_one_thread": round(us, 1), "threads": 1}
            del d
    log("cpu small configs", {k: v for k, v in per.items() if k != "prefill_ep_share"})
    # large-expert-count layer (2,048 tokens, 896 experts, top-16): the routes
    # to the first 28 experts (with their weights only), routed outside the
    # timing, on all threads and on one; the whole layer is estimated as 32
    # such slices
    big = W.large(experts_with_weights=28)
    ids_l, wts_l = M.route_sigmoid_bias(big.logits, big.bias, big.k)
    keep = ids_l < 28
    ids_s = np.where(keep, ids_l, -1).astype(ids_l.dtype)
    big.E_local = 28
    a_us, ra = layer(big, threads, ids_s, wts_l)
    o_us, ro = layer(big, 1, ids_s, wts_l)
    per["large_e_slice28"] = {"us_all_threads": round(a_us, 1), "us_one_thread": round(o_us, 1),
                              "threads": threads, "routes": int(keep.sum()),
                              "same_result": bool(np.array_equal(ra.out, ro.out)),
                              "layer_estimate_us_one_thread": round(o_us * 32, 1),
                              "layer_estimate_us_all_threads": round(a_us * 32, 1)}
    log("cpu large_e slice", per["large_e_slice28"])
    del big
    return {"value": round(us_all, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
            "cpu_model": model,
            "sample": "the prefill EP-share layer once: route of 512 own tokens, then the "
                      "4096-token group's scatter, both MX GEMMs (fp64), act-quant and combine; "
                      "per-expert thread pool with one BLAS thread per worker",
            "per_config": per}


if __name__ == "__main__":
    main()

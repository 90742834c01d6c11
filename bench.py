#!/usr/bin/env python3
"""Benchmark: batch-1 decode of a Llama-3-8B-shaped model with INT4 group-32
weights (random, synthetic), one graph-captured token step per step.

One step = one token: the per-token fp32 residual input is copied into the
decoder's residual buffer and the captured 32-layer graph (QKV, O, gate+up,
down products with their glue) is replayed.  All weights and inputs are
resident in HBM before the timed region starts.

Prints ONE JSON line with the throughput (tokens/s), the roofline of the
dominant kernel (the gate+up product) measured with HIP events on the stream
it runs on, and the CPU oracle timed on a bounded sample of the same work.

Usage: python bench.py [--gpus 1] [--steps 256] [--warmup 8] [--no-cpu-baseline]
       python bench.py --config 3|4|5   (the other workloads, one JSON line each:
       3 small-batch GEMM sweep on the 8B shapes, 4 Llama-3-70B-shaped resident
       decode, 5 the same 70B weights streamed from pinned host memory)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5])
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-runs", type=int, default=5,
                    help="single-core oracle runs (one token each) for the CPU baseline")
    ap.add_argument("--step-mode", type=int, default=None, choices=[0, 1, 2, 3],
                    help="decode step implementation: 0 four kernels per layer, 1 persistent, "
                         "2 streaming persistent, 3 streaming workgroups per product "
                         "(default: the library's choice)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the configured step and its roofline (no quantize, verify or "
                         "attention legs), e.g. for counter runs")
    ap.add_argument("--no-attention", action="store_true",
                    help="skip the extra measurement of the step with attention over "
                         "4096-row KV caches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for "
                         "hardware byte counters)")
    ap.add_argument("--counter-sample", action="store_true",
                    help="with --config 3: only a short sample for counter runs (a 1 GiB "
                         "copy, then the 28672 x 4096 product at B = 16 on the matrix "
                         "cores and at B = 1, four launches each)")
    return ap.parse_args()


def layer_bytes(dims):
    """Algorithmic bytes of one layer: packed codes + binary16 scales of the
    four matrices (0.5625 bytes per weight)."""
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    shapes = [((H + 2 * Hkv) * hd, d), (d, H * hd), (2 * dff, d), (d, dff)]
    return sum(N * K // 2 + N * (K // 32) * 2 for N, K in shapes), shapes


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; there is no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import int4_weight_streaming_q4_amd as q4
    from int4_weight_streaming_q4_amd import inputs

    torch.cuda.set_device(0)
    if args.config == 3:
        return bench_gemm(args, q4, inputs, torch)
    if args.config == 4:
        return bench_70b_resident(args, q4, inputs, torch)
    if args.config == 5:
        return bench_70b_offload(args, q4, inputs, torch)
    dims = {k: v for k, v in inputs.MODEL_DIMS["8b"].items() if k != "n_layers"}
    n_layers = inputs.MODEL_DIMS["8b"]["n_layers"]
    CONFIG = 2
    layers = [inputs.layer_weights(dims, CONFIG, l, device="cuda") for l in range(n_layers)]
    per_layer, shapes = layer_bytes(dims)
    bytes_per_token = per_layer * n_layers
    total_tokens = args.warmup + args.steps
    h0 = torch.stack([inputs.residual_f32(dims["d"], inputs.seed_of(CONFIG, t, 9),
                                          device="cuda") for t in range(total_tokens)])
    h = torch.zeros(dims["d"], dtype=torch.float32, device="cuda")
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers), dtype=torch.uint8, device="cuda")
    dec = q4.Decoder(dims, layers, h, ws)
    if args.step_mode is not None:
        dec.set_persistent(args.step_mode)
    stream = torch.cuda.Stream()
    if args.copy_calibration:
        # 1 GiB read + 1 GiB written by one plain copy kernel
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    ctx_len = 512
    torch.cuda.synchronize()

    def token(t):
        h.copy_(h0[t], non_blocking=True)
        dec.step_graph(ctx_len, stream)

    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            token(t)
        stream.synchronize()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        start.record(stream)
        for t in range(args.warmup, total_tokens):
            token(t)
        end.record(stream)
        stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    tokens_per_s = 1000.0 / ms_per_step

    # Per-kernel durations, each kernel launched back to back between two
    # events on the decode stream, cycling through the 32 layers (the
    # dominant one, gate+up, gives the roofline line).
    reps = 3 * n_layers
    names = ["qkv", "o", "gate_up", "down"]
    with torch.cuda.stream(stream):
        for k in range(4):  # first launches load the kernels; keep them out
            dec.kernel_time_us(k, 2, stream)
        kern_us = [dec.kernel_time_us(k, reps, stream) for k in range(4)]
    kbytes = kernel_bytes(dims)
    gu_us = kern_us[2]
    achieved = kbytes[2] / (gu_us * 1e-6) / 1e9
    traffic = recorded_traffic()
    gemv1 = single_gemv(q4, inputs, torch)
    gemv1["traffic"] = recorded_traffic(PMC_SUMMARY_GEMV1)

    result = {
        "metric": "INT4 GEMV HBM GB/s (% of peak) + 8B-shape batch-1 decode tokens/s",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights (group-32 fp16 scales), fp16 activations, fp32 accumulate",
        "data": "synthetic (seeded random INT4 weights and N(0,1) activations)",
        "config": {"workload": "llama3-8b-shaped INT4 decode step, batch 1, 32 layers, "
                               "graph-captured, context bucket 512",
                   "global_batch": 1, "layers": n_layers, "d_model": dims["d"],
                   "d_ff": dims["dff"], "parallelism": "single GPU"},
        "hbm_gbps_step": round(bytes_per_token * tokens_per_s / 1e9, 1),
        "hbm_frac_step": round(bytes_per_token * tokens_per_s / 1e9 / HBM_PEAK_GBS, 4),
        "us_per_layer": round(ms_per_step * 1000.0 / n_layers, 3),
        "wall_s_timed": round(wall, 4),
        "kernels": {n: {"us": round(u, 3), "GB/s": round(b / u / 1e3, 1)}
                    for n, u, b in zip(names, kern_us, kbytes)},
        "gemv_4096x4096": gemv1,
        "roofline": {"bound": "hbm",
                     "kernel": "gate_up product 28672x4096 (RMSNorm prologue, SiLU-gate epilogue)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": kbytes[2], "avg_launch_us": round(gu_us, 3)},
    }

    if not args.no_extras:
        result["quantize"] = quantize_rate(q4, torch)
        result["verify_step"] = verify_rates(q4, inputs, torch, dims, layers, ms_per_step)
    if not (args.no_attention or args.no_extras):
        dec.close()
        del ws
        wa = attention_step(args, q4, inputs, torch, dims, layers, h0)
        # in-graph cost of attention: the replayed step over 4096-row caches
        # against the configured step (whose one-token attention is the V
        # gather in the QKV epilogue), per layer
        wa["graph_delta_us_per_layer"] = round(
            (wa["ms_per_step"] - ms_per_step) * 1000.0 / n_layers, 3)
        result["with_attention"] = wa
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers, dims, h0, args.cpu_runs)
    print(json.dumps(result), flush=True)


def verify_rates(q4, inputs, torch, dims, layers, decode_ms, reps=20):
    """Verify step of a speculative draft (B token columns through the 32
    layers together, graph-captured) at B = 1, 2, 3, 4, 8, 9, 16: ms per step
    and the tokens it checks per second, next to B single-token steps."""
    mb = 16
    h = torch.zeros(dims["d"], dtype=torch.float32, device="cuda")
    hb = torch.stack([inputs.residual_f32(dims["d"], inputs.seed_of(2, t, 9), device="cuda")
                      for t in range(mb)])
    ws = torch.zeros(q4.workspace_bytes(dims, len(layers), max_batch=mb), dtype=torch.uint8,
                     device="cuda")
    dec = q4.Decoder(dims, layers, h, ws, max_batch=mb, h_batch=hb)
    stream = torch.cuda.Stream()
    out = {}
    for B in (1, 2, 3, 4, 8, 9, 16):
        with torch.cuda.stream(stream):
            dec.verify_graph(B, stream)
            dec.verify_graph(B, stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                dec.verify_graph(B, stream)
            e1.record(stream)
        stream.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"B{B}"] = {"ms": round(ms, 4), "tokens_checked_per_s": round(B * 1000.0 / ms, 1),
                        "vs_B_decode_steps": round(B * decode_ms / ms, 3)}
    dec.close()
    return out


def quantize_rate(q4, torch, N=28672, K=4096, reps=10):
    """q4_quantize on the gate+up shape from binary32 and binary16 weights
    (N(0,1) values): average us over `reps` back-to-back launches and the
    algorithmic bytes moved per second (weights read, codes and scales
    written)."""
    out = {}
    g = torch.Generator(device="cuda").manual_seed(11)
    w32 = torch.randn(N, K, generator=g, device="cuda")
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(N, K // 32, dtype=torch.int16, device="cuda")
    stream = torch.cuda.Stream()
    for name, w in (("f32", w32), ("f16", w32.half())):
        with torch.cuda.stream(stream):
            q4.q4_quantize(w, packed, scales, stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                q4.q4_quantize(w, packed, scales, stream)
            e1.record(stream)
        stream.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / reps
        nbytes = N * K * w.element_size() + N * K // 2 + N * (K // 32) * 2
        out[f"{name}_{N}x{K}"] = {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1)}
    del w32
    return out


def attention_step(args, q4, inputs, torch, dims, layers, h0, max_ctx=4096):
    """The same 8B step with decode attention over binary16 KV caches of
    max_ctx rows: the last warmup + steps tokens of a 4096-token context
    (all in the 4096 bucket), rows before the first of them prefilled with
    N(0,1) binary16 values standing in for earlier tokens.  Returns
    tokens/s and the attention kernels' share, timed per kernel with
    events around the attention launches of one eager step at the final
    context length (those events also hold the host's launch gaps of an
    eager step; the caller adds the in-graph difference per layer)."""
    n_layers = len(layers)
    total = args.warmup + args.steps
    first = max_ctx - total + 1
    kv = inputs.act_f16((q4.kv_cache_elems(dims, n_layers, max_ctx),),
                        inputs.seed_of(2, 0, 8), device="cuda")
    h = torch.zeros(dims["d"], dtype=torch.float32, device="cuda")
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers, max_ctx=max_ctx), dtype=torch.uint8,
                     device="cuda")
    dec = q4.Decoder(dims, layers, h, ws, kv_cache=kv, max_ctx=max_ctx)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for t in range(args.warmup):
            h.copy_(h0[t], non_blocking=True)
            dec.step_graph(first + t, stream)
        stream.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for t in range(args.warmup, total):
            h.copy_(h0[t], non_blocking=True)
            dec.step_graph(first + t, stream)
        end.record(stream)
        stream.synchronize()
        ms = start.elapsed_time(end) / args.steps
        dec.set_context(max_ctx, stream)
        dec.step_profiled(stream)  # first profiled pass creates events; keep it out
        prof = dec.step_profiled(stream)
    attn_ms = sum(prof[1::5]) / n_layers
    step_ms = sum(prof) / n_layers
    # K and V rows read per layer at the final context, binary16
    kv_bytes = 2 * dims["Hkv"] * max_ctx * dims["hd"] * 2
    dec.close()
    del ws
    # verify step of nine draft tokens at positions 4086..4094, same caches
    mb = 9
    hb = h0[:mb].clone()
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers, max_ctx=max_ctx, max_batch=mb),
                     dtype=torch.uint8, device="cuda")
    dec = q4.Decoder(dims, layers, h, ws, kv_cache=kv, max_ctx=max_ctx, max_batch=mb,
                     h_batch=hb)
    with torch.cuda.stream(stream):
        dec.set_context(max_ctx - mb, stream)
        dec.verify_graph(mb, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dec.verify_graph(mb, stream)
        e1.record(stream)
    stream.synchronize()
    vms = e0.elapsed_time(e1) / 10
    dec.close()
    return {"context": [first, max_ctx], "tokens_per_s": round(1000.0 / ms, 2),
            "verify_B9_ms": round(vms, 4), "verify_B9_tokens_checked_per_s": round(9000.0 / vms, 1),
            "ms_per_step": round(ms, 5),
            "attention_us_per_layer_at_4096": round(attn_ms * 1000.0, 3),
            "attention_share_of_layer": round(attn_ms / step_ms, 4),
            "attention_kv_GBps": round(kv_bytes / (attn_ms * 1e-3) / 1e9, 1)}


def kernel_bytes(dims):
    """Algorithmic bytes of each decode kernel: packed codes and binary16
    scales once, the activation read (fp32 residual for the two kernels
    that normalise it, binary16 otherwise) and the output written."""
    d, H, Hkv, hd, dff = (dims[k] for k in ("d", "H", "Hkv", "hd", "dff"))
    nqkv = (H + 2 * Hkv) * hd
    w = lambda N, K: N * K // 2 + N * (K // 32) * 2
    return [w(nqkv, d) + 4 * d + 4 * nqkv + 2 * H * hd,     # qkv: h in, qkv f32 + o_in f16 out
            w(d, H * hd) + 2 * H * hd + 8 * d,               # o: o_in in, h read + written
            w(2 * dff, d) + 4 * d + 2 * dff,                 # gate+up: h in, gated f16 out
            w(d, dff) + 2 * dff + 8 * d]                     # down: gated in, h read + written


_CSRC = "int4_weight_streaming_q4_amd/csrc/"
# Source files of the kernels whose counters are committed: the 8B gate+up
# (K = 4096) runs the row-per-wave kernel, the 70B gate+up (K = 8192) the
# pipelined product kernel.
KERNEL_SOURCES_8B = [_CSRC + f for f in ("q4_gemv_row.hip", "q4_gemv_core.h", "q4_lanes.h",
                                         "q4_internal.h")]
KERNEL_SOURCES_70B = [_CSRC + f for f in ("q4_gemv.hip", "q4_gemv_core.h", "q4_internal.h")]
KERNEL_SOURCES_GEMM = [_CSRC + f for f in ("q4_gemm.hip", "q4_internal.h")]
PMC_SUMMARY = "profiles/gate_up_8b_decode_pmc.md"
PMC_SUMMARY_GEMV1 = "profiles/gemv_4096_config1_pmc.md"
PMC_SUMMARY_GEMM = "profiles/small_batch_gate_up_counters.md"
PMC_SUMMARY_70B = "profiles/gate_up_70b_decode_pmc.md"


def kernel_source_hash(files=KERNEL_SOURCES_8B):
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(root, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(summary=PMC_SUMMARY, files=KERNEL_SOURCES_8B):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, summary)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("    ") and ":" in line:
            k, v = line.strip().split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(files):
        return None
    try:
        return int(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def single_gemv(q4, inputs, torch):
    """The 4096 x 4096 single product: 64 distinct weight copies (605 MB, more
    than the 256 MB last-level cache) launched round-robin inside one
    captured graph, replayed; average per launch."""
    N = K = 4096
    copies = 64
    Ws = [(inputs.random_bytes(N, K, inputs.seed_of(1, i, 0), device="cuda"),
           inputs.scales(N, K, inputs.seed_of(1, i, 1), device="cuda")) for i in range(copies)]
    x = inputs.act_f16(K, inputs.seed_of(1, 0, 2), device="cuda")
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for p, sc in Ws:  # warm the launch-shape cache outside the capture
            q4.q4_gemv(p, sc, x, y, stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for p, sc in Ws:
            q4.q4_gemv(p, sc, x, y, stream=s)
    reps = 20
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):  # replay and events on the same stream
        g.replay()
        s.synchronize()
        e0.record(s)
        for _ in range(reps):
            g.replay()
        e1.record(s)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1000.0 / (reps * copies)
    nbytes = N * K // 2 + N * (K // 32) * 2 + 2 * K + 4 * N
    gbs = nbytes / us / 1e3
    return {"us": round(us, 3), "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": nbytes}


def graph_avg_us(torch, launches, stream, reps=10):
    """Average microseconds per launch of the callables in `launches`,
    captured once into a graph on `stream` and replayed `reps` times."""
    with torch.cuda.stream(stream):
        for f in launches:
            f(stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in launches:
            f(stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        stream.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / (reps * len(launches))


def base_result(metric, value, unit, steps, warmup, workload, extra=None):
    r = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps,
         "warmup": warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
         "dtype": "int4 weights (group-32 fp16 scales), fp16 activations, fp32 accumulate",
         "data": "synthetic (seeded random INT4 weights and N(0,1) activations)",
         "config": {"workload": workload, "parallelism": "single GPU"}}
    if extra:
        r.update(extra)
    return r


def gemm_counter_sample(q4, inputs, torch):
    """A few launches to read hardware counters on: one plain 1 GiB device
    copy (calibration), then the 28672 x 4096 product on four weight copies
    at B = 16 through the library's small-batch path (matrix cores) and at
    B = 1 (the GEMV)."""
    N, K, copies = 28672, 4096, 4
    Ws = [(inputs.random_bytes(N, K, inputs.seed_of(3, i, 0), device="cuda"),
           inputs.scales(N, K, inputs.seed_of(3, i, 1), device="cuda")) for i in range(copies)]
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    X = inputs.act_f16((16, K), inputs.seed_of(3, 0, 2) + 16, device="cuda")
    Y = torch.empty(16, N, dtype=torch.float32, device="cuda")
    for p, sc in Ws:
        q4.q4_gemm_smallbatch(p, sc, X, Y)
    x = inputs.act_f16(K, inputs.seed_of(3, 0, 2) + 1, device="cuda")
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    for p, sc in Ws:
        q4.q4_gemv(p, sc, x, y)
    torch.cuda.synchronize()
    print(json.dumps({"counter_sample": "gate_up 28672x4096, B=16 and B=1, 4 launches each",
                      "weight_bytes_per_launch": N * K // 2 + N * (K // 32) * 2}), flush=True)


def bench_gemm(args, q4, inputs, torch):
    """Small-batch product on the four 8B matrix shapes, B in {1, 2, 3, 4,
    8, 16}: distinct weight copies (> 512 MB per shape) launched round-robin
    inside a captured graph; GB/s and effective TFLOP/s = 2NKB / t for the
    library's choice of kernel, plus both paths side by side (vector-ALU
    batch kernel where its columns fit, matrix-core kernel) to show the
    crossover in B."""
    shapes = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096),
              "down": (4096, 14336)}
    if args.counter_sample:
        return gemm_counter_sample(q4, inputs, torch)
    stream = torch.cuda.Stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    table = {}
    for name, (N, K) in shapes.items():
        wbytes = N * K // 2 + N * (K // 32) * 2
        copies = max(2, -(-600_000_000 // wbytes))
        Ws = [(inputs.random_bytes(N, K, inputs.seed_of(3, i, 0), device="cuda"),
               inputs.scales(N, K, inputs.seed_of(3, i, 1), device="cuda"))
              for i in range(copies)]
        for B in (1, 2, 3, 4, 8, 16):
            X = inputs.act_f16((B, K), inputs.seed_of(3, 0, 2) + B, device="cuda")
            Y = torch.empty(B, N, dtype=torch.float32, device="cuda")
            nbytes = wbytes + 2 * B * K + 4 * B * N

            def rate(us):
                return {"us": round(us, 3), "GB/s": round(nbytes / us / 1e3, 1),
                        "TFLOP/s": round(2 * N * K * B / us / 1e6, 2)}
            launches = [(lambda st, p=p, sc=sc: q4.q4_gemm_smallbatch(p, sc, X, Y, stream=st))
                        for p, sc in Ws]
            table[f"{name}_B{B}"] = rate(graph_avg_us(torch, launches, stream))
            if B > 1:
                # the two paths side by side (the matrix-core kernel at the
                # library's own launch shape is q4_gemm_tuned's default here)
                tiles, cap, rt = (N + 15) // 16, (2 if B <= 2 else 4), 1
                while rt * 2 <= cap and tiles // (rt * 2) >= cus * 3 // 4:
                    rt *= 2
                mf = [(lambda st, p=p, sc=sc: q4.q4_gemm_tuned(p, sc, X, Y, rt, 4, stream=st))
                      for p, sc in Ws]
                table[f"{name}_B{B}"]["mfma_us"] = round(graph_avg_us(torch, mf, stream), 3)
                if B in (2, 3, 4, 8) and B * K * 2 <= 65536:
                    va = [(lambda st, p=p, sc=sc: q4.q4_gemm_valu(p, sc, X, Y, stream=st))
                          for p, sc in Ws]
                    table[f"{name}_B{B}"]["valu_us"] = round(graph_avg_us(torch, va, stream), 3)
        del Ws
        torch.cuda.empty_cache()
    top = table["gate_up_B16"]
    res = base_result("INT4 small-batch GEMM effective TFLOP/s (8B shapes, B=1..16)",
                      top["TFLOP/s"], "TFLOP/s", 10, 1,
                      "speculative-verify small-batch INT4 GEMM on Llama-3-8B layer shapes; "
                      "value = gate+up 28672x4096 at B=16",
                      {"shapes": table,
                       "roofline": {"bound": "hbm", "kernel": "gate+up 28672x4096, B=16",
                                    "achieved": top["GB/s"], "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": round(top["GB/s"] / HBM_PEAK_GBS, 4),
                                    "traffic": recorded_traffic(PMC_SUMMARY_GEMM,
                                                                KERNEL_SOURCES_GEMM)}})
    print(json.dumps(res), flush=True)


def make_70b(q4, inputs, torch, device="cuda"):
    dims = {k: v for k, v in inputs.MODEL_DIMS["70b"].items() if k != "n_layers"}
    n_layers = inputs.MODEL_DIMS["70b"]["n_layers"]
    return dims, n_layers


def bench_70b_resident(args, q4, inputs, torch):
    dims, n_layers = make_70b(q4, inputs, torch)
    steps = args.steps if args.steps != 256 else 64
    warmup = args.warmup if args.warmup != 8 else 4
    layers = [inputs.layer_weights(dims, 4, l, device="cuda") for l in range(n_layers)]
    per_layer, _ = layer_bytes(dims)
    total = steps + warmup
    h0 = torch.stack([inputs.residual_f32(dims["d"], inputs.seed_of(4, t, 9), device="cuda")
                      for t in range(total)])
    h = torch.zeros(dims["d"], dtype=torch.float32, device="cuda")
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers), dtype=torch.uint8, device="cuda")
    dec = q4.Decoder(dims, layers, h, ws)
    if args.step_mode is not None:
        dec.set_persistent(args.step_mode)
    stream = torch.cuda.Stream()
    if args.copy_calibration:
        # 1 GiB read + 1 GiB written by one plain copy kernel
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for t in range(warmup):
            h.copy_(h0[t], non_blocking=True)
            dec.step_graph(2048, stream)
        stream.synchronize()
        e0.record(stream)
        for t in range(warmup, total):
            h.copy_(h0[t], non_blocking=True)
            dec.step_graph(2048, stream)
        e1.record(stream)
        stream.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tps = 1000.0 / ms
    with torch.cuda.stream(stream):
        for k in range(4):
            dec.kernel_time_us(k, 2, stream)
        kern_us = [dec.kernel_time_us(k, n_layers, stream) for k in range(4)]
    kb = kernel_bytes(dims)
    gbs = per_layer * n_layers * tps / 1e9
    res = base_result("70B-shape batch-1 decode tokens/s (HBM-resident INT4)", round(tps, 2),
                      "tokens/s", steps, warmup,
                      "llama3-70b-shaped INT4 decode step, batch 1, 80 layers (38.5 GB resident), "
                      "graph-captured, context bucket 2048",
                      {"ms_per_step": round(ms, 4), "us_per_layer": round(ms * 1000 / n_layers, 2),
                       "hbm_gbps_step": round(gbs, 1), "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
                       "kernels": {n: {"us": round(u, 3), "GB/s": round(b / u / 1e3, 1)}
                                   for n, u, b in zip(["qkv", "o", "gate_up", "down"], kern_us, kb)},
                       "roofline": {"bound": "hbm", "kernel": "gate_up 57344x8192",
                                    "achieved": round(kb[2] / kern_us[2] / 1e3, 1),
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(kb[2] / kern_us[2] / 1e3 / HBM_PEAK_GBS, 4),
                                    "traffic": recorded_traffic(PMC_SUMMARY_70B, KERNEL_SOURCES_70B),
                                    "bytes_per_launch": kb[2],
                                    "avg_launch_us": round(kern_us[2], 3)}})
    print(json.dumps(res), flush=True)


def bench_70b_offload(args, q4, inputs, torch):
    """70B weights in 80 pinned host blobs (one merged blob per layer),
    streamed through two device slots on a copy stream while the compute
    stream runs each layer.  Reports the host->device link peak (best pinned
    copy of one blob), achieved H2D GB/s, tokens/s and the overlap fraction
    (sum T_copy + sum T_compute - T_wall) / min(sum T_copy, sum T_compute):
    T_copy from timing events the weight stream records where each copy
    starts (after the wait for its slot) and ends (their union: the time the
    copy streams were busy), T_compute the 80 layers computed alone from
    resident slots, T_wall the streamed tokens (1 = compute fully hidden
    behind the copies, 0 = serial).  q4_decode_token_streamed keeps the host
    one token ahead of the device at most."""
    dims, n_layers = make_70b(q4, inputs, torch)
    steps = args.steps if args.steps != 256 else 64
    warmup = args.warmup if args.warmup != 8 else 2
    offs, blob_bytes = q4.layer_blob_layout(dims)
    blobs = []
    for l in range(n_layers):
        L = inputs.layer_weights(dims, 4, l, device="cuda")
        dev = torch.empty(blob_bytes, dtype=torch.uint8, device="cuda")
        for i, name in enumerate(("qkv", "o", "gate_up", "down")):
            p, sc = L[name]
            pb = p.reshape(-1).view(torch.uint8)
            sb = sc.reshape(-1).view(torch.uint8)
            dev[offs[2 * i]:offs[2 * i] + pb.numel()].copy_(pb)
            dev[offs[2 * i + 1]:offs[2 * i + 1] + sb.numel()].copy_(sb)
        hb = torch.empty(blob_bytes, dtype=torch.uint8, pin_memory=True)
        hb.copy_(dev)
        blobs.append(hb)
        del L, dev
    torch.cuda.synchronize()
    print(f"[config 5] {n_layers} pinned blobs of {blob_bytes} bytes ready", file=sys.stderr,
          flush=True)
    slots = [torch.empty(blob_bytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    copy_s = torch.cuda.Stream()
    comp_s = torch.cuda.Stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # link peak: best single pinned blob copy
    best = 1e30
    with torch.cuda.stream(copy_s):
        for i in range(10):
            e0.record(copy_s)
            slots[i % 2].copy_(blobs[i % n_layers], non_blocking=True)
            e1.record(copy_s)
            copy_s.synchronize()
            best = min(best, e0.elapsed_time(e1))
    link_gbs = blob_bytes / (best * 1e-3) / 1e9
    # copies alone, back to back
    with torch.cuda.stream(copy_s):
        e0.record(copy_s)
        for l in range(n_layers):
            slots[l % 2].copy_(blobs[l], non_blocking=True)
        e1.record(copy_s)
        copy_s.synchronize()
    t_copy_b2b = e0.elapsed_time(e1)
    h = torch.zeros(dims["d"], dtype=torch.float32, device="cuda")
    ws = torch.zeros(q4.workspace_bytes(dims, n_layers), dtype=torch.uint8, device="cuda")
    dec = q4.Decoder(dims, None, h, ws, n_layers=n_layers)
    # compute alone: the 80 layers from the two resident slots (after one
    # untimed pass, so first-launch costs are not counted)
    slot_layers = [q4.layer_from_blob(dims, s.data_ptr()) for s in slots]
    h.copy_(inputs.residual_f32(dims["d"], inputs.seed_of(4, 0, 9), device="cuda"))
    torch.cuda.synchronize()
    with torch.cuda.stream(comp_s):
        for l in range(n_layers):
            dec.layer(slot_layers[l % 2], comp_s)
        e0.record(comp_s)
        for l in range(n_layers):
            dec.layer(slot_layers[l % 2], comp_s)
        e1.record(comp_s)
        comp_s.synchronize()
    t_compute = e0.elapsed_time(e1)
    print(f"[config 5] link peak {link_gbs:.1f} GB/s, copies alone {t_copy_b2b:.1f} ms, "
          f"compute alone {t_compute:.2f} ms", file=sys.stderr, flush=True)
    h0 = [inputs.residual_f32(dims["d"], inputs.seed_of(4, t, 9), device="cuda")
          for t in range(steps + warmup)]

    def streamed(ws_obj, n_tok, n_timed_tok=0):
        """(ms per token over n_tok timed tokens, overlap figures or None)."""
        with torch.cuda.stream(comp_s):
            for t in range(warmup):
                h.copy_(h0[t % len(h0)], non_blocking=True)
                dec.token_streamed(ws_obj, comp_s)
            comp_s.synchronize()
            copy_s.synchronize()
            e0.record(comp_s)
            for t in range(n_tok):
                h.copy_(h0[(warmup + t) % len(h0)], non_blocking=True)
                dec.token_streamed(ws_obj, comp_s)
            e1.record(comp_s)
            comp_s.synchronize()
        ms = e0.elapsed_time(e1) / n_tok
        ov = None
        if n_timed_tok:
            # instrumented tokens: per-copy start and end events
            n_str = sum(1 for b in ws_obj._keep[0] if b is not None)
            ws_obj.set_timing(n_str * n_timed_tok + 1)
            with torch.cuda.stream(comp_s):
                e0.record(comp_s)
                for t in range(n_timed_tok):
                    h.copy_(h0[t % len(h0)], non_blocking=True)
                    dec.token_streamed(ws_obj, comp_s)
                e1.record(comp_s)
                comp_s.synchronize()
            starts, ends = ws_obj.copy_times(n_str * n_timed_tok + 1)
            ws_obj.set_timing(0)
            wall = e0.elapsed_time(e1)
            # the copies that belong to these tokens: the first was begun by
            # the token before them (prefetch), the last begins the next token
            k = n_str * n_timed_tok
            # time the copy streams were busy: the union of the copies'
            # intervals (with two copy streams a layer's pieces and the next
            # layer's overlap in time), and the idle gaps between them
            merged = []
            for s0, e0_ in sorted(zip(starts[:k], ends[:k])):
                if merged and s0 <= merged[-1][1]:
                    merged[-1][1] = max(merged[-1][1], e0_)
                else:
                    merged.append([s0, e0_])
            sum_copy = sum(e - s for s, e in merged)
            sum_comp = t_compute * n_timed_tok  # every layer streamed here
            gaps = sorted(merged[i + 1][0] - merged[i][1] for i in range(len(merged) - 1))
            ov = {"tokens": n_timed_tok, "wall_ms": round(wall, 3),
                  "sum_copy_ms": round(sum_copy, 3),
                  "sum_compute_ms": round(sum_comp, 3),
                  "overlap_fraction": round((sum_copy + sum_comp - wall) /
                                            min(sum_copy, sum_comp), 4),
                  "copy_ms_median": round(sorted(e - s for s, e in zip(starts[:k], ends[:k]))[k // 2], 4),
                  "copy_busy_intervals": len(merged),
                  "copy_gap_us_median": round(1000 * gaps[len(gaps) // 2], 2) if gaps else None,
                  "copy_gap_us_max": round(1000 * gaps[-1], 2) if gaps else None}
        torch.cuda.synchronize()
        return ms, ov

    wstream = q4.WeightStream(blobs, slots, copy_s)
    t0 = time.perf_counter()
    t_wall, ov1 = streamed(wstream, steps, n_timed_tok=4)
    wall = time.perf_counter() - t0
    wstream.close()
    tps = 1000.0 / t_wall
    h2d = blob_bytes * n_layers * tps / 1e9
    res = base_result("70B-shape offload decode tokens/s (pinned host -> 2-slot HBM pool)",
                      round(tps, 4), "tokens/s", steps, warmup,
                      "llama3-70b-shaped INT4 decode, batch 1, 80 layers streamed per token "
                      "from 80 pinned host blobs of 481 MB into two device slots",
                      {"ms_per_step": round(t_wall, 3), "wall_s_timed": round(wall, 3),
                       "h2d_gbps": round(h2d, 2), "link_peak_gbps": round(link_gbs, 2),
                       "frac_of_link_peak": round(h2d / link_gbs, 4),
                       "t_copy_back_to_back_ms": round(t_copy_b2b, 3),
                       "t_compute_ms": round(t_compute, 3),
                       "overlap_fraction": ov1["overlap_fraction"],
                       "overlap": ov1,
                       "roofline": {"bound": "host-to-device link", "kernel": "H2D layer copies",
                                    "achieved": round(h2d, 2), "peak": round(link_gbs, 2),
                                    "unit": "GB/s", "frac": round(h2d / link_gbs, 4),
                                    "traffic": None}})
    print(f"[config 5] one copy stream: {t_wall:.2f} ms/token, {h2d:.2f} GB/s, "
          f"overlap {ov1}", file=sys.stderr, flush=True)

    # the same stream in 32 MB pieces alternating over two copy streams
    copy2_s = torch.cuda.Stream()
    chunk = 32 << 20
    ws2 = q4.WeightStream(blobs, slots, copy_s, copy2=copy2_s, chunk_bytes=chunk)
    ms2, ov2 = streamed(ws2, max(4, steps // 4), n_timed_tok=2)
    ws2.close()
    variants = {"one_copy_stream_whole_blobs": {"ms_per_token": round(t_wall, 3),
                                                "tokens_per_s": round(tps, 4),
                                                "h2d_gbps": round(h2d, 2)},
                "two_copy_streams_32MB_pieces": {
                    "ms_per_token": round(ms2, 3), "tokens_per_s": round(1000.0 / ms2, 4),
                    "h2d_gbps": round(blob_bytes * n_layers / ms2 / 1e6, 2), "overlap": ov2}}
    # partial residency: a budget of 40 layer blobs of HBM, placed by
    # q4_offload_plan (two slots + 38 resident layers spread over the depth)
    budget = 40 * blob_bytes
    mask = q4.offload_plan(n_layers, blob_bytes, budget)
    resident = [blobs[l].to("cuda") if m else None for l, m in enumerate(mask)]
    torch.cuda.synchronize()
    ws3 = q4.WeightStream([None if m else b for b, m in zip(blobs, mask)], slots, copy_s,
                          resident=resident)
    ms3, _ = streamed(ws3, max(4, steps // 4))
    ws3.close()
    n_str = n_layers - sum(mask)
    variants[f"resident_{sum(mask)}_of_{n_layers}_budget_40_blobs"] = {
        "ms_per_token": round(ms3, 3), "tokens_per_s": round(1000.0 / ms3, 4),
        "h2d_gbps": round(blob_bytes * n_str / ms3 / 1e6, 2), "streamed_layers": n_str}
    del resident
    res["variants"] = variants
    dec.close()
    print(json.dumps(res), flush=True)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layers, dims, h0, runs=5):
    """The fp64 oracle, single-threaded and pinned to one core, on a bounded
    sample of the same workload: one token through the 32 layers per run,
    median of `runs` runs (about 20 s), plus the 4096 x 4096 product as ns per
    weight (median of 5).  Beside it, labelled as a baseline and not as the
    oracle: the same loops from the oracle's source built with OpenMP
    (product rows in parallel) on every core this process may use."""
    import statistics

    import numpy as np
    import oracle
    from int4_weight_streaming_q4_amd import inputs

    host = [{k: (p.cpu().numpy(), inputs.to_numpy_u16(s)) for k, (p, s) in L.items()}
            for L in layers]
    N = K = 4096
    gp = inputs.random_bytes(N, K, inputs.seed_of(1, 0, 0)).numpy()
    gs = inputs.to_numpy_u16(inputs.scales(N, K, inputs.seed_of(1, 0, 1)))
    gx = inputs.to_numpy_u16(inputs.act_f16(K, inputs.seed_of(1, 0, 2)))
    h0s = [h.cpu().numpy().astype(np.float64) for h in h0[:runs]]

    def product_s(all_cores):
        ts = []
        for _ in range(5):
            t0 = time.perf_counter()
            oracle.gemv(gp, gs, gx, all_cores=all_cores)
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    def token_s(all_cores, n):
        ts = []
        for r in range(n):
            hh = h0s[r % len(h0s)].copy()
            t0 = time.perf_counter()
            for L in host:
                oracle.decode_layer(L, dims, hh, all_cores=all_cores)
            ts.append(time.perf_counter() - t0)
        return ts

    allowed = sorted(os.sched_getaffinity(0))
    pin = allowed[0]
    os.sched_setaffinity(0, {pin})
    try:
        g1 = product_s(False)
        tok = token_s(False, runs)
    finally:
        os.sched_setaffinity(0, set(allowed))
    threads = min(len(allowed), int(os.environ.get("OMP_NUM_THREADS", len(allowed))))
    g1_all = product_s(True)
    tok_all = token_s(True, 3)
    med = statistics.median(tok)
    return {"value": round(1.0 / med, 5), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"one token x {len(host)} layers of the same 8B-shaped model per run, "
                      f"median of {runs} runs; fp64 single-threaded C pinned to cpu {pin}",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "cpus_allowed": len(allowed),
            "pinned_cpu": pin, "s_per_token_runs": [round(t, 3) for t in tok],
            "config1_gemv_4096x4096": {"ms_median_of_5": round(1000 * g1, 3),
                                       "ns_per_weight": round(1e9 * g1 / (N * K), 3)},
            "all_cores": {"label": "baseline, not the oracle: the oracle's source built with "
                                   "OpenMP, product rows in parallel",
                          "threads": threads,
                          "tokens_per_s": round(1.0 / statistics.median(tok_all), 4),
                          "config1_ns_per_weight": round(1e9 * g1_all / (N * K), 4)}}


if __name__ == "__main__":
    main()

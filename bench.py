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
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=3)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for "
                         "hardware byte counters)")
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
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import int4_weight_streaming_q4_amd as q4
    from int4_weight_streaming_q4_amd import inputs

    torch.cuda.set_device(0)
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
    ws = torch.zeros(q4.workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    dec = q4.Decoder(dims, layers, h, ws)
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
        kern_us = [dec.kernel_time_us(k, reps, stream) for k in range(4)]
    kbytes = kernel_bytes(dims)
    gu_us = kern_us[2]
    achieved = kbytes[2] / (gu_us * 1e-6) / 1e9
    traffic = recorded_traffic()
    gemv1 = single_gemv(q4, inputs, torch)

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

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers, dims, h0, args.cpu_tokens)
    print(json.dumps(result), flush=True)


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


KERNEL_SOURCES = ["int4_weight_streaming_q4_amd/csrc/q4_gemv.hip",
                  "int4_weight_streaming_q4_amd/csrc/q4_internal.h"]
PMC_SUMMARY = "profiles/gate_up_8b_decode_pmc.md"


def kernel_source_hash():
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(root, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per gate+up launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, PMC_SUMMARY)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("    ") and ":" in line:
            k, v = line.strip().split(":", 1)
            rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
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


def cpu_baseline(layers, dims, h0, n_tokens):
    """The fp64 oracle (single thread) on a bounded sample: n_tokens tokens of
    the same 32-layer model, same weights and inputs."""
    import numpy as np
    import oracle
    from int4_weight_streaming_q4_amd import inputs

    host = [{k: (p.cpu().numpy(), inputs.to_numpy_u16(s)) for k, (p, s) in L.items()}
            for L in layers]
    t0 = time.perf_counter()
    for t in range(n_tokens):
        hh = h0[t].cpu().numpy().astype(np.float64)
        for L in host:
            oracle.decode_layer(L, dims, hh)
    dt = time.perf_counter() - t0
    return {"value": round(n_tokens / dt, 5), "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n_tokens} token(s) x {len(host)} layers of the same 8B-shaped "
                      f"model, fp64 single-threaded C, {dt:.1f} s"}


if __name__ == "__main__":
    main()

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
    ap.add_argument("--profiled-steps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1)
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

    # dominant kernel: gate+up, timed with events around every kernel of an
    # eager step on the same stream
    prof = []
    with torch.cuda.stream(stream):
        for _ in range(args.profiled_steps):
            prof.append(dec.step_profiled(stream))
    prof = np.array(prof)  # [steps, 6 * n_layers]
    per_kernel = prof.reshape(prof.shape[0], n_layers, 6).mean(axis=(0, 1))  # ms
    names = ["norm1", "qkv", "o", "norm2", "gate_up", "down"]
    gu_N, gu_K = shapes[2]
    gu_bytes = gu_N * gu_K // 2 + gu_N * (gu_K // 32) * 2 + gu_K * 2 + (gu_N // 2) * 2
    gu_ms = float(per_kernel[4])
    achieved = gu_bytes / (gu_ms * 1e-3) / 1e9

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
        "kernel_us_eager": {n: round(float(v) * 1000.0, 3) for n, v in zip(names, per_kernel)},
        "roofline": {"bound": "hbm", "kernel": "gate_up product 28672x4096 (SiLU-gated epilogue)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_ms * 1000.0, 3)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers, dims, h0, args.cpu_tokens)
    print(json.dumps(result), flush=True)


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

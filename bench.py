"""Benchmark of the routed-expert MoE decode step on one MI355X.

A step is one qs_moe_decode call through every layer of the workload (the
residual chain x_{l+1} = x_l + MoE_l(x_l)) for one batch of T tokens.  The
inputs rotate through 64 seeded batches already resident in HBM, so picks
change from step to step.  Throughput is tokens/s; the weight-read rate is
the algorithmic bytes of a step (router, shared expert and each distinct
selected expert once per layer, plus activations in and out) over the step
time, against the 8 TB/s HBM peak.

Prints one JSON line.  --gpus above 1 is refused: this path is measured on
one GPU.
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
N_BATCHES = 64


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="a3b_stack40_zipf")
    p.add_argument("--tokens", default="1,4,16", help="batch sizes; the first is the headline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=6, help="layers in the oracle sample")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    p.add_argument("--multikernel", action="store_true", help="time the one-kernel-per-step path")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path runs on one MI355X, see DESIGN.md for how it would shard)")
        sys.exit(2)
    import torch

    import quantized_moe_decode_router_amd as qm
    import synth

    wl = synth.WORKLOADS[args.workload]
    L = args.layers or wl.n_layers
    tok_list = [int(t) for t in args.tokens.split(",")]
    maxT = max(tok_list)
    cb = synth.codebook()
    torch.cuda.init()
    log(f"[bench] workload {wl.name}: {L} layers, H={wl.hidden} E={wl.n_experts} k={wl.top_k} "
        f"F={wl.expert_ffn} Fs={wl.shared_ffn}, tokens {tok_list}")
    t0 = time.time()
    moe = qm.MoE.for_workload(wl, cb, n_layers=L, max_tokens=maxT)
    for l in range(L):
        moe.upload(l, synth.layer_weights(wl, l))
        if l % 10 == 9 or l == L - 1:
            log(f"[bench] uploaded {l + 1}/{L} layers ({time.time() - t0:.1f}s)")
    g, u, d = wl.expert_bytes()
    per_expert = g + u + d
    fixed_layer = wl.router_bytes() + wl.shared_bytes()
    stream = torch.cuda.current_stream()

    results = {}
    for T in tok_list:
        xs = torch.from_numpy(np.stack([synth.tokens(wl, T, b) for b in range(N_BATCHES)])).cuda()
        y = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
        ids = torch.empty((N_BATCHES, L, T, wl.top_k), dtype=torch.int32, device="cuda")
        # untimed pass: the experts each batch selects, for the byte count
        for b in range(N_BATCHES):
            moe.decode(xs[b], y, n_layers=L, residual=True, prenorm=True, ids_out=ids[b],
                       multikernel=args.multikernel)
        torch.cuda.synchronize()
        idn = ids.cpu().numpy()
        uniq = np.array([[len(np.unique(idn[b, l])) for l in range(L)] for b in range(N_BATCHES)])
        bytes_batch = uniq.sum(axis=1) * per_expert + L * fixed_layer + 2 * T * wl.hidden * 4
        for i in range(args.warmup):
            moe.decode(xs[i % N_BATCHES], y, n_layers=L, residual=True, prenorm=True,
                       multikernel=args.multikernel)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(args.steps):
            moe.decode(xs[i % N_BATCHES], y, n_layers=L, residual=True, prenorm=True,
                       multikernel=args.multikernel)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        step_bytes = float(np.mean([bytes_batch[i % N_BATCHES] for i in range(args.steps)]))
        gbs = step_bytes / (ms * 1e-3) / 1e9
        results[T] = {
            "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms, "bytes_per_step": step_bytes,
            "weight_read_GBps": gbs, "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
            "mean_distinct_experts_per_layer": float(uniq.mean()),
        }
        log(f"[bench] T={T}: {ms:.3f} ms/step, {T / (ms * 1e-3):.1f} tok/s, {gbs:.1f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), U={uniq.mean():.1f}")
        del xs, ids
    moe.close()

    T0 = tok_list[0]
    head = results[T0]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T0, L, args.cpu_layers)
    line = {
        "metric": "MoE decode tokens/s and weight-read GB/s as % of HBM peak, batch 1/4/16",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "arith": "2-bit weights decoded to int8, activations as 16-bit fixed point in two int8 "
                 "limbs, int32-exact dot products, fp32 scales and combine, fp64 router",
        "data": "synthetic (seeded weights and activations, 64 rotating input batches)",
        "config": {"workload": wl.name, "layers": L, "hidden": wl.hidden, "experts": wl.n_experts,
                   "top_k": wl.top_k, "expert_ffn": wl.expert_ffn, "shared_ffn": wl.shared_ffn,
                   "gate_up_format": wl.gate_up_format, "down_format": wl.down_format,
                   "tokens": T0, "zipf_s": wl.zipf_s, "parallelism": "single GPU"},
        "weight_read_GBps": head["weight_read_GBps"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "roofline": {"bound": "hbm", "kernel": "decode step (all kernels of one call)",
                     "achieved": head["weight_read_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["weight_read_GBps"] / HBM_PEAK_GBS, "traffic": None},
        "per_batch": {str(T): r for T, r in results.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(wl, T, L, n_layers_sample):
    """The oracle as it stands on a bounded sample: the first n layers of one
    step at batch T, single BLAS thread; scaled to tokens/s of a full step."""
    import synth
    from oracle import moe as om
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limit = None
    n = min(n_layers_sample, L)
    cb = synth.codebook()
    x = synth.tokens(wl, T, 0)
    layers = []
    for l in range(n):
        lw = synth.layer_weights(wl, l)
        # only the experts this sample touches are dequantised (lazily)
        layers.append(om.Layer(wl, lw, cb))
    t0 = time.perf_counter()
    cur = x
    for layer in layers:
        cur = om.moe_layer(layer, cur, residual=True, prenorm=True)["y"]
    dt = time.perf_counter() - t0
    if limit is not None:
        limit.unregister() if hasattr(limit, "unregister") else None
    step_s = dt * L / n
    log(f"[bench] oracle: {n} layers at T={T} in {dt:.2f}s -> {T / step_s:.3f} tok/s for {L} layers")
    return {"value": T / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {L} layers of one step at T={T} (numpy fp64, one thread), "
                      f"{dt:.1f}s, scaled by {L}/{n}"}


if __name__ == "__main__":
    main()

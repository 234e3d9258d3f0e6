"""Benchmark of the routed-expert MoE decode step on one MI355X.

A step is one qs_moe_decode call through every layer of the workload (the
pre-norm residual chain x_{l+1} = x_l + MoE_l(RMSNorm(x_l))) for one batch of
T tokens.  The inputs rotate through 64 seeded batches already resident in
HBM, so expert picks change from step to step.  Throughput is tokens/s; the
weight-read rate is the algorithmic bytes of a step (each layer's router,
shared expert and every distinct selected expert read once, plus the
activations in and out) over the step time, against the 8 TB/s HBM peak.

The roofline entry is for the decode kernel itself (one launch per step):
algorithmic bytes per launch over its mean duration, timed with HIP events on
the stream it is launched on.  Its "traffic" is the HBM bytes per launch that
the FETCH_SIZE / WRITE_SIZE counters recorded for the same kernel, scaled by
what the counters read for a plain copy of known size; it is read from the
committed counter summary and reported only if that summary was taken from
the current kernel sources (sha256 of csrc/ and include/), else null.

Prints one JSON line.  --gpus above 1 is refused: this path is measured on
one GPU.  `--copy-calibration MiB` instead runs a plain device copy (the
reference kernel for the counter scaling) and prints what it moved.
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
N_BATCHES = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_persist_small_a3b_stack40_zipf_T1_hbm_traffic.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="a3b_stack40_zipf")
    p.add_argument("--tokens", default="1,4,16", help="batch sizes; the first is the headline")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the other HBM-target workloads (routed-only stack, large-layer stack)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=40, help="layers in the oracle sample")
    p.add_argument("--layers", type=int, default=0, help="override the layer count (0 = workload's)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of this many MiB, 20 times")
    return p.parse_args()


# The other workloads the bench line reports beside the headline one: the
# routed-only 40-layer stack, the stack with an 8-bit shared expert, the
# headline stack with every layer's output steered, and the 8-layer
# large-layer stack, at their batch sizes, with fewer timed steps; and the
# headline stack with expert paging: 4 resident layers, the routed experts of
# the other 36 in host memory behind a cache of a quarter of them, warmed
# with the popularity hotlist.
STEERED = "+steer"
PAGED = "+paged"
PAGING = {"resident_layers": 4, "cache_fraction": 0.25}
EXTRA = (("a3b_routed40", (1, 4)), ("a3b_stack40_zipf_q8", (1, 4)), ("a3b_stack40_zipf" + STEERED, (1, 4, 16)),
         ("a3b_stack40_q4tail", (1, 4, 16)), ("flash_stack8_zipf", (1, 8, 32)), ("a3b_stack40_zipf" + PAGED, (1, 4)))
STEER_SCALE = 0.8
EXTRA_STEPS = 100


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    """sha256 over the kernel sources and the public header."""
    h = hashlib.sha256()
    dirs = [os.path.join(ROOT, "quantized_moe_decode_router_amd", "csrc"), os.path.join(ROOT, "include")]
    for d in dirs:
        for name in sorted(os.listdir(d)):
            if name.endswith((".h", ".hip", ".cpp")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str, T: int):
    """HBM bytes per launch from the committed counter summary, when it
    matches this workload, batch and the current sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith((" ", "\t", "#", "$")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if (kv.get("source_sha256") != source_digest() or kv.get("workload") != workload
                or int(kv.get("tokens", -1)) != T):
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(20):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                                           "launches": 20}}), flush=True)


def kernel_name(wl, T):
    if getattr(wl, "tail_layers", 0):
        return ("2-bit layers: " + kernel_name(synth_plain(wl), T) +
                f"; last {wl.tail_layers} layers: k_persist_big<q4k> (a second launch)")
    fmt = "cb2" if wl.gate_up_format == "cb2" else "q2k"
    # the small-batch kernel: batches up to 4 at hidden sizes up to 2048, and
    # the large-layer shape's fixed instantiation at one token
    small = T <= 4 and (wl.hidden <= 2048 or (T == 1 and wl.hidden == 4096 and wl.top_k == 6
                                                and wl.expert_ffn == 2048 and wl.shared_ffn == 2048))
    return ("k_persist_small" if small else "k_persist_big") + f"<{fmt}> (one launch = the whole decode call)"


def synth_plain(wl):
    """The workload without its Q4_K-style tail (for naming the 2-bit kernel)."""
    import dataclasses
    return dataclasses.replace(wl, tail_layers=0)


def run_workload(qm, wl, L, tok_list, steps, warmup, steer=False, paging=None):
    """Time `steps` decode calls through all L layers at each batch size
    (with steer: every layer's output steered along a seeded unit direction;
    with paging: expert paging as PAGING describes); returns {T: figures}."""
    import torch
    import synth
    cb = synth.codebook()
    tag = (STEERED if steer else "") + (PAGED if paging else "")
    log(f"[bench] workload {wl.name}{tag}: {L} layers, H={wl.hidden} E={wl.n_experts} k={wl.top_k} "
        f"F={wl.expert_ffn} Fs={wl.shared_ffn}, tokens {list(tok_list)}")
    t0 = time.time()
    kw = {}
    if paging:
        R = paging["resident_layers"]
        kw = dict(resident_layers=R, cache_slots=int(paging["cache_fraction"] * (L - R) * wl.n_experts))
    moe = qm.MoE.for_workload(wl, cb, n_layers=L, max_tokens=max(tok_list), **kw)
    for l in range(L):
        moe.upload(l, synth.layer_weights(wl, l))
        if l % 10 == 9 or l == L - 1:
            log(f"[bench] uploaded {l + 1}/{L} layers ({time.time() - t0:.1f}s)")
    if paging:
        moe.cache_preload(synth.hotlist(wl, range(kw["resident_layers"], L)))
        log(f"[bench] paging: {kw}, preloaded {moe.cache_stats()['preloaded']} experts")
    if steer:
        dirs = np.random.default_rng(12).standard_normal((L, wl.hidden))
        moe.set_steering((dirs / np.linalg.norm(dirs, axis=1, keepdims=True)).astype(np.float32), STEER_SCALE)
    # bytes of one expert in each layer (the Q4_K-style tail layers' are larger)
    per_expert = np.array([sum(wl.expert_bytes(l)) for l in range(L)], dtype=np.float64)
    fixed_layer = wl.router_bytes() + wl.shared_bytes() + (wl.hidden * 4 if steer else 0)
    # decode() launches on torch's current stream; every event below is
    # recorded on that same stream
    stream = torch.cuda.current_stream()

    # the bench runs nothing else on the device: exclusive launches (the same
    # kernel dispatched without the cooperative launch's serialisation); the
    # cooperative launch is timed as well
    def step(x, y, ids=None, exclusive=True):
        moe.decode(x, y, n_layers=L, residual=True, prenorm=True, ids_out=ids, stream=stream, steer=steer,
                   exclusive=exclusive)

    results = {}
    for T in tok_list:
        xs = torch.from_numpy(np.stack([synth.tokens(wl, T, b) for b in range(N_BATCHES)])).cuda()
        y = torch.empty((T, wl.hidden), dtype=torch.float32, device="cuda")
        ids = torch.empty((N_BATCHES, L, T, wl.top_k), dtype=torch.int32, device="cuda")
        # untimed pass: the experts each batch selects, for the byte count
        for b in range(N_BATCHES):
            step(xs[b], y, ids[b])
        moe.sync_status(stream)
        idn = ids.cpu().numpy()
        uniq = np.array([[len(np.unique(idn[b, l])) for l in range(L)] for b in range(N_BATCHES)])
        bytes_batch = uniq @ per_expert + L * fixed_layer + 2 * T * wl.hidden * 4
        for i in range(warmup):
            step(xs[i % N_BATCHES], y)
        torch.cuda.synchronize()
        if paging:
            moe.cache_sync(stream)
            c0 = moe.cache_stats()
        # whole timed region: K steps back to back
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for i in range(steps):
            step(xs[i % N_BATCHES], y)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        cache = None
        if paging:   # the cache over the timed steps (their uses applied after the region)
            moe.cache_sync(stream)
            c1 = moe.cache_stats()
            d = {n: c1[n] - c0[n] for n in ("hits", "misses", "admissions", "evictions")}
            exp_b = float(np.mean(per_expert[kw["resident_layers"]:]))
            cache = dict(kw, **d, hit_rate=d["hits"] / max(1, d["hits"] + d["misses"]),
                         expert_bytes=exp_b, host_bytes=c1["host_bytes"],
                         pcie_bytes_per_step=(d["misses"] + d["admissions"]) * exp_b / steps,
                         pcie_GBps=(d["misses"] + d["admissions"]) * exp_b / (ms * 1e-3 * steps) / 1e9)
            log(f"[bench] cache over the timed steps: hit rate {cache['hit_rate']:.3f}, "
                f"{d['misses'] / steps:.1f} misses and {d['admissions'] / steps:.1f} admissions per step, "
                f"PCIe {cache['pcie_GBps']:.1f} GB/s")
        # the same steps with cooperative launches
        start.record(stream)
        for i in range(steps):
            step(xs[i % N_BATCHES], y, exclusive=False)
        end.record(stream)
        torch.cuda.synchronize()
        coop_ms = start.elapsed_time(end) / steps
        # per launch: an event pair around each decode call (one kernel
        # launch), same stream, same inputs
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record(stream)
            step(xs[i % N_BATCHES], y)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        moe.sync_status(stream)          # no timed call gave up a wait
        launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
        step_bytes = float(np.mean([bytes_batch[i % N_BATCHES] for i in range(steps)]))
        gbs = step_bytes / (ms * 1e-3) / 1e9
        achieved = step_bytes / (launch_ms.mean() * 1e-3) / 1e9
        results[T] = {
            "tokens_per_s": T / (ms * 1e-3), "ms_per_step": ms, "bytes_per_step": step_bytes,
            "cooperative_ms_per_step": coop_ms, "cooperative_tokens_per_s": T / (coop_ms * 1e-3),
            "weight_read_GBps": gbs, "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
            "mean_distinct_experts_per_layer": float(uniq.mean()),
            "launch_ms_mean": float(launch_ms.mean()), "launch_ms_p10": float(np.percentile(launch_ms, 10)),
            "launch_ms_p90": float(np.percentile(launch_ms, 90)),
            "roofline": {"bound": "hbm", "achieved": achieved,
                         "kernel": kernel_name(wl, T).replace("k_persist_small", "k_persist_small_paged").replace(
                             "k_persist_big", "k_persist_big_paged") if paging else kernel_name(wl, T),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS},
        }
        if cache:
            results[T]["cache"] = cache
        log(f"[bench] {wl.name}{tag} T={T}: {ms:.3f} ms/step, {T / (ms * 1e-3):.1f} tok/s, {gbs:.1f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s), U={uniq.mean():.1f}, "
            f"launch {launch_ms.mean():.3f} ms (p10 {np.percentile(launch_ms, 10):.3f}, "
            f"p90 {np.percentile(launch_ms, 90):.3f}); cooperative launches {coop_ms:.3f} ms/step")
        del xs, ids
    moe.close()
    return results


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode step "
              "runs and is measured on a single MI355X (the design notes say how it would shard)")
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch

    import quantized_moe_decode_router_amd as qm
    import synth

    torch.cuda.init()
    wl = synth.WORKLOADS[args.workload]
    L = args.layers or wl.n_layers
    tok_list = [int(t) for t in args.tokens.split(",")]
    results = run_workload(qm, wl, L, tok_list, args.steps, args.warmup)
    others = {}
    if not args.no_extra and not args.layers:
        for name, toks in EXTRA:
            if name == wl.name:
                continue
            steer, paged = name.endswith(STEERED), name.endswith(PAGED)
            w2 = synth.WORKLOADS[name.split("+")[0]]
            r = run_workload(qm, w2, w2.n_layers, toks, min(args.steps, EXTRA_STEPS), args.warmup, steer=steer,
                             paging=PAGING if paged else None)
            others[name] = {"layers": w2.n_layers, "per_batch": {str(T): v for T, v in r.items()}}

    T0 = tok_list[0]
    head = results[T0]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, T0, L, args.cpu_layers)
    traffic = None if args.layers else committed_traffic(wl.name, T0)
    roof = dict(head["roofline"])
    roof.update({"algorithmic_bytes_per_launch": head["bytes_per_step"], "launch_ms": head["launch_ms_mean"],
                 "traffic": traffic})
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
        "launch": "QS_DECODE_EXCLUSIVE (the persistent kernel as an ordinary dispatch; the bench runs nothing "
                  "else on the device); per_batch.*.cooperative_ms_per_step times the cooperative launch",
        "config": {"workload": wl.name, "layers": L, "hidden": wl.hidden, "experts": wl.n_experts,
                   "top_k": wl.top_k, "expert_ffn": wl.expert_ffn, "shared_ffn": wl.shared_ffn,
                   "gate_up_format": wl.gate_up_format, "down_format": wl.down_format,
                   "tokens": T0, "zipf_s": wl.zipf_s, "parallelism": "single GPU"},
        "weight_read_GBps": head["weight_read_GBps"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "roofline": roof,
        "per_batch": {str(T): r for T, r in results.items()},
        "other_workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    if limit is not None and hasattr(limit, "unregister"):
        limit.unregister()
    step_s = dt * L / n
    log(f"[bench] oracle: {n} layers at T={T} in {dt:.2f}s -> {T / step_s:.4f} tok/s for {L} layers")
    return {"value": T / step_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cpu": cpu_model(), "host_nproc": os.cpu_count(),
            "sample": (f"all {L} layers" if n == L else f"first {n} of {L} layers, scaled by {L}/{n},")
                      + f" of one step at T={T} (numpy fp64 with one BLAS thread, dequantising each"
                      f" touched expert): {dt:.1f}s"}


if __name__ == "__main__":
    main()

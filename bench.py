"""Benchmark of the RouteRelay routing pass on one MI355X.

One step = the whole routing pass over the batched-heads workload (32 heads, 1024 query and
key chunks per head, d = 64, bf16, 32 layers, anchors at layers 0/8/16/24, k = 12, m = 12,
r = 8): the RouteRelay chain (anchor layers + relay layers) and, as the comparator, full
routing at every layer (top-12 only).  Inputs for all 32 layers are resident in HBM before
timing starts.

Headline: relay-layer query-row routes per second = heads * nq * (relay layers) / (time spent
in relay layers), timed with HIP events on the launch stream around every layer call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--graph]
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

from long_context_prefill_anchor_amd import rr, synth, workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def upload_layers(w):
    import torch
    qs, ks, sig = [], [], []
    for li in synth.generate(w):
        qs.append(torch.from_numpy(li.q.view(np.int16)).cuda())
        ks.append(torch.from_numpy(li.k.view(np.int16)).cuda())
        sig.append(li.sigma)
    torch.cuda.synchronize()
    return qs, ks, sig


def run_relay_chain(w, led, qs, ks, outs=None, ev=None):
    """Anchor or relay per layer; optional per-layer events (start, end) lists."""
    for l in range(w.layers):
        if ev is not None:
            ev[l][0].record()
        if w.is_anchor(l):
            led.anchor(qs[l], ks[l], l)
        else:
            led.relay(qs[l], ks[l], l, outs[l] if outs is not None else None)
        if ev is not None:
            ev[l][1].record()


def run_full_chain(w, full, qs, ks, ev=None):
    for l in range(w.layers):
        if ev is not None:
            ev[l][0].record()
        full.anchor(qs[l], ks[l], l)
        if ev is not None:
            ev[l][1].record()


def quality_pass(w, led, full, qs, ks):
    """Untimed: recall of the relayed routes against full routing, rerouted fraction,
    evaluated score-pair fraction (Section 5 metrics)."""
    import torch
    H, n = w.heads, w.n
    outs = [led.alloc_outputs(with_scores=False) if not w.is_anchor(l) else None for l in range(w.layers)]
    recall_sum, rows_rerouted, relay_flags, pairs = 0.0, 0, [], 0
    for l in range(w.layers):
        if w.is_anchor(l):
            led.anchor(qs[l], ks[l], l)
            rows_rerouted += H * n
            pairs += H * n * n
        else:
            led.relay(qs[l], ks[l], l, outs[l])
        full.anchor(qs[l], ks[l], l)
        torch.cuda.synchronize()
        used = led.get()[0].cpu().numpy().reshape(-1, w.k)
        exact = full.get()[0].cpu().numpy().reshape(-1, w.k)
        # recall per row: |used & exact| / |exact| (routes are ascending; n >= k so no padding)
        inter = (used[:, :, None] == exact[:, None, :]).any(axis=2).sum(axis=1)
        recall_sum += float((inter / w.k).mean())
        if not w.is_anchor(l):
            nf = int(outs[l].n_rows.cpu().numpy()[0])
            relay_flags.append(nf / (H * n))
            rows_rerouted += nf
            pairs += H * n * w.c + nf * n
    L = w.layers
    return dict(recall=recall_sum / L, reroute_fraction=rows_rerouted / (H * n * L),
                relay_rho_mean=float(np.mean(relay_flags)), relay_rho_per_layer=[round(x, 4) for x in relay_flags],
                pair_fraction=pairs / (H * n * n * L))


def cpu_baseline(w, max_seconds=20.0):
    """The oracle, unmodified, on a bounded sample: the first heads of the same workload, as
    many chain layers as fit in ~max_seconds; single-threaded BLAS."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    heads = 4
    cfg = O.RouteConfig(heads=heads, nq=w.n, nk=w.n, d=w.d, k=w.k, m=w.m, r=w.r, gamma=w.gamma,
                        causal=w.causal, seed=w.seed, dtype=w.dtype)
    t_relay = t_anchor = 0.0
    n_relay = n_anchor = 0
    led = None
    t_start = time.perf_counter()
    with threadpool_limits(limits=1):
        for li in synth.generate(w, slice(0, heads)):
            t0 = time.perf_counter()
            if led is None or w.is_anchor(li.layer):
                led = O.anchor_layer(cfg, li.q, li.k, li.layer)
                t_anchor += time.perf_counter() - t0
                n_anchor += 1
            else:
                led = O.relay_layer(cfg, li.q, li.k, li.layer, led).ledger
                t_relay += time.perf_counter() - t0
                n_relay += 1
            if time.perf_counter() - t_start > max_seconds and n_relay >= 2:
                break
    rows = heads * w.n
    return {"value": rows * n_relay / t_relay, "unit": "relay-layer query-row routes/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {w.heads} heads, layers 0-{n_anchor + n_relay - 1} "
                      f"({n_anchor} anchor, {n_relay} relay), single-threaded NumPy",
            "full_routing_value": rows * n_anchor / t_anchor if n_anchor else None,
            "relay_over_full_time": (t_relay / n_relay) / (t_anchor / n_anchor) if n_anchor else None}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); heads shard across GPUs "
              "with no exchange, so run one process per GPU on its own heads.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    rr.lib()
    w = W.batched_heads()
    H, n = w.heads, w.n
    log(f"[bench] generating + uploading {w.layers} layers of {H}x{n}x{w.d} bf16 Q and K")
    qs, ks, _ = upload_layers(w)
    led = rr.Ledger(H, n, n, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed)
    full = rr.Ledger(H, n, n, w.d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)

    log("[bench] quality pass (recall, reroute fraction, pair fraction)")
    q = quality_pass(w, led, full, qs, ks)
    log(f"[bench] recall={q['recall']:.6f} reroute={q['reroute_fraction']:.4f} "
        f"relay_rho={q['relay_rho_mean']:.4f} pairs={q['pair_fraction']:.4f}")

    L = w.layers
    relay_layers = [l for l in range(L) if not w.is_anchor(l)]
    anchor_layers = [l for l in range(L) if w.is_anchor(l)]

    def step(evr=None, evf=None):
        run_relay_chain(w, led, qs, ks, None, evr)
        run_full_chain(w, full, qs, ks, evf)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    evs = [([[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)],
            [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)])
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s][0], evs[s][1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    relay_ms = np.array([[evs[s][0][l][0].elapsed_time(evs[s][0][l][1]) for l in range(L)]
                         for s in range(args.steps)])
    full_ms = np.array([[evs[s][1][l][0].elapsed_time(evs[s][1][l][1]) for l in range(L)]
                        for s in range(args.steps)])
    t_relay_layers = relay_ms[:, relay_layers].sum()          # ms over all timed steps
    t_full_layers = full_ms.sum()
    rows_relay = H * n * len(relay_layers) * args.steps
    value = rows_relay / (t_relay_layers / 1e3)
    full_value = H * n * L * args.steps / (t_full_layers / 1e3)
    relay_layer_us = float(np.median(relay_ms[:, relay_layers]) * 1e3)
    anchor_layer_us = float(np.median(relay_ms[:, anchor_layers]) * 1e3)
    full_layer_us = float(np.median(full_ms) * 1e3)
    speedup = (t_full_layers / (L * args.steps)) / (t_relay_layers / (len(relay_layers) * args.steps))

    # Dominant kernel: full routing of a whole layer (the anchor / comparator route kernel),
    # bound by MFMA: algorithmic flops per launch = 2 * d * heads * nq * nk.
    flops = 2.0 * w.d * H * n * n
    achieved_tflops = flops / (full_layer_us * 1e-6) / 1e12
    roofline = {"kernel": "k_route (full routing, k=12)", "bound": "mfma",
                "achieved": round(achieved_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": None,
                "per_launch": {"flops": flops, "avg_us": round(full_layer_us, 2)}}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu_baseline: oracle on a bounded sample")
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": "relay-layer query-row routes/sec at Nk=1024 + speedup vs full routing; top-k recall",
        "value": round(value, 1),
        "unit": "query-row routes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "batched_heads", "heads": H, "nq": n, "nk": n, "d": w.d,
                   "layers": L, "anchors": list(w.anchors), "k": w.k, "m": w.m, "r": w.r,
                   "gamma": w.gamma, "causal": w.causal, "drift": "sigma_l ~ U[0.01, 0.06), relative",
                   "parallelism": "single GPU"},
        "speedup_vs_full": round(float(speedup), 4),
        "recall": round(q["recall"], 6),
        "reroute_fraction": round(q["reroute_fraction"], 4),
        "relay_rho_mean": round(q["relay_rho_mean"], 4),
        "pair_fraction": round(q["pair_fraction"], 4),
        "full_routing_routes_per_s": round(full_value, 1),
        "relay_layer_us_median": round(relay_layer_us, 2),
        "anchor_layer_us_median": round(anchor_layer_us, 2),
        "full_layer_us_median": round(full_layer_us, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    led.close()
    full.close()


if __name__ == "__main__":
    main()

"""Benchmark of the RouteRelay routing pass on one MI355X.

One step = the whole routing pass over the batched-heads workload (32 heads, 1024 query and
key chunks per head, d = 64, bf16, 32 layers, anchors at layers 0/8/16/24, k = 12, m = 12,
r = 8): the RouteRelay chain (anchor layers + relay layers) and, as the comparator, full
routing at every layer (top-12 only).  Inputs for all 32 layers are resident in HBM before
timing starts.

Headline: relay-layer query-row routes per second = heads * nq * (relay layers) / (time spent
in relay layers), timed with HIP events on the launch stream around every layer call.  Each
kernel is also timed on its own, in a second timed region of the same steps (events the
library records around its launches), and set against its roofline: the reroute kernel (dominant in relay layers) and full routing against
the bf16 MFMA peak on algorithmic flops, the rescore kernel against HBM bandwidth on
algorithmic bytes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--calib-copy]
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

from long_context_prefill_anchor_amd import rr, synth, workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
# the routing kernels' source and the headers it includes
KERNEL_SRCS = tuple(os.path.join(ROOT, "long_context_prefill_anchor_amd", "csrc", f)
                    for f in ("rr_kernels.hip", "rr_device.h", "rr_internal.h"))
BUILD_SCRIPT = os.path.join(ROOT, "long_context_prefill_anchor_amd", "build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_route_reroute_batched_heads.txt")
CALIB_BYTES = 256 << 20         # plain copy used to calibrate the HBM byte counters


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def upload_layers(w):
    import torch
    qs, ks = [], []
    for li in synth.generate(w):
        qs.append(torch.from_numpy(li.q.view(np.int16)).cuda())
        ks.append(torch.from_numpy(li.k.view(np.int16)).cuda())
    torch.cuda.synchronize()
    return qs, ks


def run_relay_chain(w, led, qs, ks, ev=None):
    """Anchor or relay per layer; optional per-layer events (start, end) lists."""
    for l in range(w.layers):
        if ev is not None:
            ev[l][0].record()
        if w.is_anchor(l):
            led.anchor(qs[l], ks[l], l)
        else:
            led.relay(qs[l], ks[l], l)
        if ev is not None:
            ev[l][1].record()


def run_full_chain(w, full, qs, ks, ev=None):
    for l in range(w.layers):
        if ev is not None:
            ev[l][0].record()
        full.anchor(qs[l], ks[l], l)
        if ev is not None:
            ev[l][1].record()


def route_recall(used, exact):
    """Mean over rows of |used & exact| / |exact| for [rows, k] int arrays; -1 padding in
    `exact` is not counted (a row with no exact entries counts as 0)."""
    hit = ((used[:, :, None] == exact[:, None, :]) & (exact[:, None, :] >= 0)).any(axis=1).sum(axis=1)
    return float((hit / np.maximum((exact >= 0).sum(axis=1), 1)).mean())


def stride_reuse_routes(exact_per_layer, stride=4):
    """The fixed-stride baseline: every row refreshed at layers divisible by `stride`, the
    route reused unchecked in between."""
    out, stale = [], None
    for l, exact in enumerate(exact_per_layer):
        if l % stride == 0:
            stale = exact
        out.append(stale)
    return out


def quality_pass(w, led, full, qs, ks):
    """Untimed: recall of the relayed routes against full routing, rerouted fraction,
    evaluated score-pair fraction (Section 5 metrics), flagged rows per relay layer; also the
    recall of the pages' fixed-stride baseline (every row refreshed each 4th layer, the route
    reused unchecked in between), which needs no kernel of its own."""
    import torch
    H, n = w.heads, w.nq
    n_i = (np.arange(n) + 1) if w.causal else np.full(n, w.nk)       # allowed keys per row
    c_i = np.minimum(w.c, n_i)                                          # candidates per row
    out = led.alloc_outputs(with_scores=False)
    recall_sum, rows_rerouted, flagged, pairs, relay_pairs = 0.0, 0, {}, 0, 0
    stride4_sum, stale = 0.0, None
    for l in range(w.layers):
        if w.is_anchor(l):
            led.anchor(qs[l], ks[l], l)
            rows_rerouted += H * n
            pairs += H * int(n_i.sum())
        else:
            led.relay(qs[l], ks[l], l, out)
        full.anchor(qs[l], ks[l], l)
        torch.cuda.synchronize()
        used = led.get()[0].cpu().numpy().reshape(-1, w.k)
        exact = full.get()[0].cpu().numpy().reshape(-1, w.k)
        recall_sum += route_recall(used, exact)
        if l % 4 == 0:
            stale = exact                                    # same rule as stride_reuse_routes
        stride4_sum += route_recall(stale, exact)
        if not w.is_anchor(l):
            nf = int(out.n_rows.cpu().numpy()[0])
            rows = out.rows.cpu().numpy()[:nf] % n
            flagged[l] = nf
            rows_rerouted += nf
            lp = H * int(c_i.sum()) + int(n_i[rows].sum())
            pairs += lp
            relay_pairs += lp
    L = w.layers
    relay_rho = [flagged[l] / (H * n) for l in sorted(flagged)]
    return dict(recall=recall_sum / L, reroute_fraction=rows_rerouted / (H * n * L),
                relay_rho_mean=float(np.mean(relay_rho)), relay_rho_per_layer=[round(x, 4) for x in relay_rho],
                pair_fraction=pairs / (H * int(n_i.sum()) * L), flagged=flagged, relay_pairs=relay_pairs,
                stride4_recall=stride4_sum / L)


def time_chains(w, led, full, qs, ks, steps, warmup):
    """`warmup` untimed passes, then `steps` timed passes of the relay chain and the full-routing
    chain, each layer call bracketed by events on the launch stream; returns the per-layer
    times (ms) of both chains and the wall time of the timed passes."""
    import torch
    L = w.layers
    for _ in range(warmup):
        run_relay_chain(w, led, qs, ks)
        run_full_chain(w, full, qs, ks)
    torch.cuda.synchronize()
    evs = [([[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)],
            [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L)])
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        run_relay_chain(w, led, qs, ks, evs[s][0])
        run_full_chain(w, full, qs, ks, evs[s][1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    relay_ms = np.array([[evs[s][0][l][0].elapsed_time(evs[s][0][l][1]) for l in range(L)] for s in range(steps)])
    full_ms = np.array([[evs[s][1][l][0].elapsed_time(evs[s][1][l][1]) for l in range(L)] for s in range(steps)])
    return relay_ms, full_ms, wall


def graph_chains(w, led, full, qs, ks, reps=10):
    """Both 32-layer chains captured once as HIP graphs (through torch's graph capture on the
    library's stream argument) and replayed `reps` times; returns mean ms per chain and whether
    the replayed relay chain leaves the same ledger as an eager run."""
    import torch
    torch.cuda.synchronize()
    run_relay_chain(w, led, qs, ks)
    torch.cuda.synchronize()
    eager = [t.cpu() for t in led.get()]
    res = {}
    for name, fn in (("relay_chain_ms", lambda: run_relay_chain(w, led, qs, ks)),
                     ("full_chain_ms", lambda: run_full_chain(w, full, qs, ks))):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / reps, 4)
        if name == "relay_chain_ms":
            replayed = [t.cpu() for t in led.get()]
            res["replay_matches_eager"] = all(bool(torch.equal(a, b)) for a, b in zip(eager, replayed))
        del g
    res["speedup_vs_full_chain"] = round(res["full_chain_ms"] / res["relay_chain_ms"], 4)
    return res


def secondary_causal(steps=3, warmup=1):
    """The 64-head, 4096-chunk causal workload: relay vs full routing (reported beside the
    headline, which is the 32-head 1024-chunk workload)."""
    w = W.causal_large()
    log(f"[bench] secondary: {w.name} {w.heads}x{w.n} causal, {w.layers} layers")
    return relay_vs_full(w, steps, warmup)


def drift_sweep_batched(sigmas=(0.01, 0.03, 0.06), steps=2, warmup=1):
    """The batched-heads shape (32 x 1024, bf16) at fixed per-layer drift: where relay layers
    stand against full routing as the rerouted fraction grows (the headline draws each layer's
    drift from [0.01, 0.06))."""
    out = []
    for s in sigmas:
        w = W.batched_heads().with_(name=f"batched_heads_drift{s:g}", drift=(s, s))
        log(f"[bench] drift sweep: {w.name}")
        r = relay_vs_full(w, steps, warmup)
        out.append({"sigma": s, **{k: r[k] for k in ("relay_layer_us_median", "full_layer_us_median",
                                                      "speedup_vs_full", "recall", "reroute_fraction",
                                                      "relay_rho_mean", "fixed_stride4_recall")}})
    return out


def sentinel_ablation(seeds=5):
    """Sentinel mixes on the pages' ablation setting (1 x 256 chunks, fp32, 24 layers, drift
    0.003, k = 12; anchors every 8 layers, as in the other chains): mean recall against full
    routing, rerouted fraction and score-pair fraction over the seeds.  The 24-wide near-miss
    row runs on the one-wave-per-row kernel (k + m = 36); the 48-wide row needs c = 72 ledger
    entries, past this library's 64, so 40 near-miss + 12 random (c = 64) stands nearest.  The
    last mix trades three random sentinels for the mandatory kind (Section 3.1, item 3: one
    sink chunk, two recent chunks); the synthetic walk gives those chunks no special role,
    and a pair count of c per row is an upper bound when one of them is already routed."""
    import torch
    mixes = [("random only", 0, 12, 0, 0), ("near-miss only", 12, 0, 0, 0),
             ("12 near-miss + 12 random", 12, 12, 0, 0), ("12 near-miss + 8 random", 12, 8, 0, 0),
             ("12 near-miss + 1 sink + 2 recent + 5 random", 12, 5, 1, 2),
             ("24 near-miss + 12 random", 24, 12, 0, 0), ("40 near-miss + 12 random", 40, 12, 0, 0)]
    out = []
    for name, m, r, sink, recent in mixes:
        acc = np.zeros(3)
        for seed in range(seeds):
            w = W.drift_sweep(0.003, seed).with_(name=f"ablation_{m}nm_{r}rnd_{sink}s{recent}r_seed{seed}",
                                                 layers=24, anchors=W.stride_anchors(24, 8), m=m, r=r,
                                                 sink=sink, recent=recent)
            qs, ks = upload_layers(w)
            led = rr.Ledger(w.heads, w.n, w.n, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed,
                            sink=w.sink, recent=w.recent)
            full = rr.Ledger(w.heads, w.n, w.n, w.d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)
            q = quality_pass(w, led, full, qs, ks)
            acc += [q["recall"], q["reroute_fraction"], q["pair_fraction"]]
            led.close()
            full.close()
        acc /= seeds
        out.append({"sentinels": name, "m": m, "r": r, "sink": sink, "recent": recent,
                    "recall": round(float(acc[0]), 6),
                    "reroute_fraction": round(float(acc[1]), 4), "pair_fraction": round(float(acc[2]), 4)})
    torch.cuda.empty_cache()
    return out


def preferred_chunks_sweep(sigmas=(0.01, 0.03, 0.06, 0.1), seeds=10):
    """The cross-layer stability setting (Section 5.1, Table 2, Figure 2): 1 head, 384 query
    rows, 192 key chunks, 32 fp32 layers, persistent preferred chunks with layer-local drift
    (generator in synth.py; its preference strength and the anchor schedule are this build's
    choices), 12 + 24 near-miss + 12 random.  Means over the seeds of relay recall, rerouted
    fraction and the fixed-stride-4 baseline's recall."""
    import torch
    out = []
    for sigma in sigmas:
        acc = np.zeros(3)
        for seed in range(seeds):
            w = W.preferred_chunks(sigma, seed)
            qs, ks = upload_layers(w)
            led = rr.Ledger(w.heads, w.nq, w.nk, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed)
            full = rr.Ledger(w.heads, w.nq, w.nk, w.d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)
            q = quality_pass(w, led, full, qs, ks)
            acc += [q["recall"], q["reroute_fraction"], q["stride4_recall"]]
            led.close()
            full.close()
        acc /= seeds
        out.append({"drift": sigma, "recall": round(float(acc[0]), 6),
                    "reroute_fraction": round(float(acc[1]), 4),
                    "fixed_stride4_recall": round(float(acc[2]), 6)})
    torch.cuda.empty_cache()
    return out


def sparse_attention_measure(reps=20, causal=False):
    """The routes' consumer (Section 2.1 token expansion, Eq. 3): sparse online-softmax
    attention of every query token over the tokens of its chunk's route, at the headline
    shape (32 heads x 1024 chunks of 64 tokens = 65,536 tokens per head, d = 64, bf16), or
    with ``causal`` at the causal workload's shape (64 heads x 4096 chunks = 262,144 tokens
    per head), with the routes of an anchor ledger on the workload's first layer and seeded
    synthetic token Q, K, V drawn on the device.  Reported against both bounds: MFMA flops of
    the two products (causal: of the unmasked pairs), and the bytes a gather moves when
    nothing is reused (Q, each routed chunk's K and V per query chunk, O)."""
    import torch
    w = (W.causal_large() if causal else W.batched_heads()).with_(layers=1)
    H, n, T, d = w.heads, w.n, 64, w.d
    qs, ks = upload_layers(w)
    led = rr.Ledger(H, n, n, d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed)
    led.anchor(qs[0], ks[0], 0)
    routes = led.get()[0]
    torch.cuda.synchronize()
    g = torch.Generator(device="cuda").manual_seed(2024)
    qt = (torch.randn((H, n * T, d), generator=g, device="cuda") / 8).to(torch.bfloat16)
    kt = (torch.randn((H, n * T, d), generator=g, device="cuda") / 8).to(torch.bfloat16)
    vt = (torch.randn((H, n * T, d), generator=g, device="cuda") / 8).to(torch.bfloat16)
    vt = vt.view(H, n, T, d).transpose(2, 3).contiguous()
    out = torch.empty((H, n * T, d), dtype=torch.float32, device="cuda")
    for _ in range(3):
        rr.rr_sparse_attention(qt, kt, vt, routes, H, n, n, w.k, out, causal=causal)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        rr.rr_sparse_attention(qt, kt, vt, routes, H, n, n, w.k, out, causal=causal)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / reps
    valid = int((routes >= 0).sum().item())
    pairs = float(valid) * T * T
    if causal:                                   # the diagonal chunk keeps T (T + 1) / 2 pairs
        own = (routes == torch.arange(n, device=routes.device).view(1, n, 1)).sum().item()
        pairs -= float(own) * T * (T - 1) / 2
    flops = pairs * d * 2 * 2
    gathered = float(H * n * T * d * 2 + valid * T * d * 2 * 2 + H * n * T * d * 4)
    unique = float(H * n * T * d * (2 * 3 + 4))
    ach_f = flops / (us * 1e-6) / 1e12
    ach_b = gathered / (us * 1e-6) / 1e9
    led.close()
    del qs, ks, qt, kt, vt, out
    torch.cuda.empty_cache()
    return {"kernel": f"k_sparse_attn<{str(causal).lower()}>",
            "workload": f"{w.name} tokens ({H} heads x {n} chunks x {T} tokens)",
            "chunk_tokens": T, "route_k": w.k, "routed_chunks": valid, "avg_us": round(us, 2), "reps": reps,
            "mfma": {"flops": flops, "achieved": round(ach_f, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach_f / MFMA_BF16_PEAK_TFLOPS, 4)},
            "hbm_gathered": {"bytes": gathered, "achieved": round(ach_b, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ach_b / HBM_PEAK_GBS, 4)},
            "unique_bytes": unique}


class LedgerGroup:
    """Width-bucket ledgers driven as one: each call goes to every bucket in turn."""

    def __init__(self, leds):
        self.leds = leds

    def anchor(self, q, k, layer):
        for led in self.leds:
            led.anchor(q, k, layer)

    def relay(self, q, k, layer, out=None):
        for led in self.leds:
            led.relay(q, k, layer)


def width_buckets(steps=3, warmup=1):
    """Query-dependent route widths through width-bucketed ledgers (Sections 4.3-4.4) on the
    headline chain: even query rows route with k = 8 (m = 12, r = 8), odd rows with k = 16
    (m = 12, r = 4); the comparator routes every row in full at its own width.  Recall is
    against each row's own exact top-k."""
    import torch
    w = W.batched_heads()
    H, n = w.heads, w.n
    qs, ks = upload_layers(w)
    specs = [(tuple(range(0, n, 2)), 8, 12, 8), (tuple(range(1, n, 2)), 16, 12, 4)]
    leds = [rr.Ledger(H, n, n, w.d, k, m, r, w.gamma, w.causal, w.dtype, w.seed, q_rows=rows)
            for rows, k, m, r in specs]
    fulls = [rr.Ledger(H, n, n, w.d, k, 0, 0, w.gamma, w.causal, w.dtype, w.seed, q_rows=rows)
             for rows, k, _, _ in specs]
    outs = [led.alloc_outputs(with_scores=False) for led in leds]
    recall, rerouted = 0.0, 0
    for l in range(w.layers):
        for led, full, o in zip(leds, fulls, outs):
            if w.is_anchor(l):
                led.anchor(qs[l], ks[l], l)
            else:
                led.relay(qs[l], ks[l], l, o)
            full.anchor(qs[l], ks[l], l)
        torch.cuda.synchronize()
        for led, full, o in zip(leds, fulls, outs):
            used = led.get()[0].cpu().numpy().reshape(-1, led.k)
            exact = full.get()[0].cpu().numpy().reshape(-1, led.k)
            recall += route_recall(used, exact) * led.nq / n
            rerouted += H * led.nq if w.is_anchor(l) else int(o.n_rows.cpu().numpy()[0])
    relay_ms, full_ms, _ = time_chains(w, LedgerGroup(leds), LedgerGroup(fulls), qs, ks, steps, warmup)
    relay_layers = [l for l in range(w.layers) if not w.is_anchor(l)]
    t_relay, t_full = relay_ms[:, relay_layers].sum(), full_ms.sum()
    out = {"workload": "batched_heads, two width buckets",
           "buckets": [{"rows": "even query rows", "k": 8, "m": 12, "r": 8},
                       {"rows": "odd query rows", "k": 16, "m": 12, "r": 4}],
           "recall": round(recall / w.layers, 6), "reroute_fraction": round(rerouted / (H * n * w.layers), 4),
           "relay_routes_per_s": round(H * n * len(relay_layers) * steps / (t_relay / 1e3), 1),
           "speedup_vs_full": round(float((t_full / (w.layers * steps)) / (t_relay / (len(relay_layers) * steps))), 4),
           "relay_layer_us_median": round(float(np.median(relay_ms[:, relay_layers]) * 1e3), 2),
           "full_layer_us_median": round(float(np.median(full_ms) * 1e3), 2), "steps": steps}
    for x in leds + fulls:
        x.close()
    del qs, ks
    torch.cuda.empty_cache()
    return out


def relay_vs_full(w, steps, warmup):
    import torch
    H, n = w.heads, w.n
    qs, ks = upload_layers(w)
    led = rr.Ledger(H, n, n, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed,
                    sink=w.sink, recent=w.recent, min_reuse=w.min_reuse, gamma_extra=w.gamma_extra)
    full = rr.Ledger(H, n, n, w.d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)
    q = quality_pass(w, led, full, qs, ks)
    relay_ms, full_ms, _ = time_chains(w, led, full, qs, ks, steps, warmup)
    relay_layers = [l for l in range(w.layers) if not w.is_anchor(l)]
    t_relay = relay_ms[:, relay_layers].sum()
    t_full = full_ms.sum()
    out = {"workload": w.name, "heads": H, "nq": n, "nk": n, "causal": w.causal, "layers": w.layers,
           "k": w.k, "m": w.m, "r": w.r, "sink": w.sink, "recent": w.recent,
           "min_reuse": w.min_reuse, "gamma_extra": w.gamma_extra,
           "relay_routes_per_s": round(H * n * len(relay_layers) * steps / (t_relay / 1e3), 1),
           "full_routing_routes_per_s": round(H * n * w.layers * steps / (t_full / 1e3), 1),
           "speedup_vs_full": round(float((t_full / (w.layers * steps)) / (t_relay / (len(relay_layers) * steps))), 4),
           "relay_layer_us_median": round(float(np.median(relay_ms[:, relay_layers]) * 1e3), 2),
           "full_layer_us_median": round(float(np.median(full_ms) * 1e3), 2),
           "recall": round(q["recall"], 6), "reroute_fraction": round(q["reroute_fraction"], 4),
           "relay_rho_mean": round(q["relay_rho_mean"], 4), "pair_fraction": round(q["pair_fraction"], 4),
           "fixed_stride4_recall": round(q["stride4_recall"], 6),
           "steps": steps}
    led.close()
    full.close()
    del qs, ks
    torch.cuda.empty_cache()
    return out


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


def kernel_build_hash():
    """sha256 of the kernel source and its headers, followed by the build script (its compiler
    flags)."""
    h = hashlib.sha256()
    for path in (*KERNEL_SRCS, BUILD_SCRIPT):
        h.update(open(path, "rb").read())
    return h.hexdigest()


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` (reroute / rescore / route) from the committed counter
    summary, if it was taken on the kernel source and build script as they are now (else None)."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("kernel_build_sha256") != kernel_build_hash():
        return None
    try:
        return float(fields[f"{kernel}_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calib_copy():
    """A plain device copy of known size (CALIB_BYTES read + written), for counter calibration."""
    import torch
    a = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the side measurements (64-head 4096-chunk causal; fixed-drift sweep; sentinel ablation)")
    ap.add_argument("--only-attention", action="store_true",
                    help="measure only the sparse attention over routed chunks and print its JSON")
    ap.add_argument("--calib-copy", action="store_true",
                    help=f"run one plain {CALIB_BYTES >> 20} MiB device copy first (counter calibration)")
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
    if args.calib_copy:
        calib_copy()
    if args.only_attention:
        print(json.dumps({"sparse_attention": sparse_attention_measure()}), flush=True)
        return
    w = W.batched_heads()
    H, n, d = w.heads, w.n, w.d
    log(f"[bench] generating + uploading {w.layers} layers of {H}x{n}x{d} bf16 Q and K")
    qs, ks = upload_layers(w)
    led = rr.Ledger(H, n, n, d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed)
    full = rr.Ledger(H, n, n, d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)

    log("[bench] quality pass (recall, reroute fraction, pair fraction)")
    q = quality_pass(w, led, full, qs, ks)
    log(f"[bench] recall={q['recall']:.6f} reroute={q['reroute_fraction']:.4f} "
        f"relay_rho={q['relay_rho_mean']:.4f} pairs={q['pair_fraction']:.4f}")

    L = w.layers
    relay_layers = [l for l in range(L) if not w.is_anchor(l)]
    anchor_layers = [l for l in range(L) if w.is_anchor(l)]

    def step():
        run_relay_chain(w, led, qs, ks)
        run_full_chain(w, full, qs, ks)

    log(f"[bench] warmup {args.warmup} steps, timing {args.steps} steps")
    relay_ms, full_ms, wall = time_chains(w, led, full, qs, ks, args.steps, args.warmup)

    log("[bench] chains as graph replays")
    graph = graph_chains(w, led, full, qs, ks)

    # Second timed region, same steps, with the library's per-kernel launch events on (kept
    # out of the headline region: each extra event record adds a gap between kernels).
    log(f"[bench] timing {args.steps} steps with per-kernel events")
    led.profile(True)
    full.profile(True)
    for s in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt_led = led.kernel_times()
    kt_full = full.kernel_times()
    led.profile(False)
    full.profile(False)

    t_relay_layers = relay_ms[:, relay_layers].sum()          # ms over all timed steps
    t_full_layers = full_ms.sum()
    rows_relay = H * n * len(relay_layers) * args.steps
    value = rows_relay / (t_relay_layers / 1e3)
    full_value = H * n * L * args.steps / (t_full_layers / 1e3)
    relay_layer_us = float(np.median(relay_ms[:, relay_layers]) * 1e3)
    anchor_layer_us = float(np.median(relay_ms[:, anchor_layers]) * 1e3)
    full_layer_us = float(np.median(full_ms) * 1e3)
    speedup = (t_full_layers / (L * args.steps)) / (t_relay_layers / (len(relay_layers) * args.steps))
    pairs_per_s = q["relay_pairs"] * args.steps / (t_relay_layers / 1e3)

    # Per-kernel averages from the library's own launch events (same stream as the kernels).
    def avg_us(kt, kind):
        nl, ms = kt[kind]
        return (ms * 1e3 / nl) if nl else None, nl
    t_resc, n_resc = avg_us(kt_led, rr.RR_KERNEL_RESCORE)
    t_rer, n_rer = avg_us(kt_led, rr.RR_KERNEL_REROUTE)
    t_anc, n_anc = avg_us(kt_led, rr.RR_KERNEL_ROUTE)
    t_full, n_full = avg_us(kt_full, rr.RR_KERNEL_ROUTE)

    # Algorithmic work per launch.
    #   reroute: 2*d*nk flops per flagged row (its full row is scored), averaged over the
    #            relay layers (every timed step repeats the same flags);
    #   full routing: 2*d*nq*nk per head;
    #   rescore: bytes read once — Q, K (K counted once per head), the c ledger IDs per row —
    #            plus one flag byte written per row.
    reroute_flops = 2.0 * d * n * float(np.mean([q["flagged"][l] for l in relay_layers]))
    full_flops = 2.0 * d * H * n * n
    rescore_bytes = float(H * (n * d * 2 + n * d * 2 + n * w.c * 4 + n))

    def mfma_line(name, flops, us, nl):
        ach = flops / (us * 1e-6) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "per_launch": {"flops": flops, "avg_us": round(us, 2), "launches": nl}}

    rer = mfma_line("k_route<bf16, reroute> (flagged rows)", reroute_flops, t_rer, n_rer)
    rer["traffic"] = recorded_traffic("reroute")
    ach_resc = rescore_bytes / (t_resc * 1e-6) / 1e9
    kernels = {
        "rescore": {"kernel": "k_rescore<bf16, 1>", "bound": "hbm", "achieved": round(ach_resc, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach_resc / HBM_PEAK_GBS, 4),
                    "per_launch": {"bytes": rescore_bytes, "avg_us": round(t_resc, 2), "launches": n_resc},
                    "traffic": recorded_traffic("rescore")},
        "reroute": rer,
        "full_routing": mfma_line("k_route<bf16, full> (k=12, m=r=0)", full_flops, t_full, n_full),
        "anchor": mfma_line("k_route<bf16, full> (k=12, m=12, r=8)", full_flops, t_anc, n_anc),
    }
    roofline = dict(rer)

    led.close()
    full.close()
    del qs, ks
    torch.cuda.empty_cache()
    secondary = None if args.no_secondary else secondary_causal()
    drift_sweep = None if args.no_secondary else drift_sweep_batched()
    ablation = None if args.no_secondary else sentinel_ablation()
    preferred = None if args.no_secondary else preferred_chunks_sweep()
    buckets = None if args.no_secondary else width_buckets()
    wide = None
    if not args.no_secondary:
        log("[bench] batched heads with a 24-wide near-miss set (k + m = 36: one-wave-per-row kernel)")
        wide = relay_vs_full(W.batched_heads().with_(name="batched_heads_nm24", m=24, r=8), steps=2, warmup=1)
    attention, attention_causal = None, None
    if not args.no_secondary:
        log("[bench] sparse attention over the routes (token expansion, Eq. 3)")
        attention = sparse_attention_measure()
        attention["routing_relay_layer_us"] = round(relay_layer_us, 2)
        attention["routing_share_of_layer"] = round(relay_layer_us / (relay_layer_us + attention["avg_us"]), 4)
        log("[bench] causal sparse attention at the 64 x 4096 shape")
        attention_causal = sparse_attention_measure(reps=5, causal=True)
        if secondary is not None:
            attention_causal["routing_relay_layer_us"] = secondary["relay_layer_us_median"]
            attention_causal["routing_share_of_layer"] = round(
                secondary["relay_layer_us_median"] / (secondary["relay_layer_us_median"] + attention_causal["avg_us"]), 4)
    # Hysteresis (Section 3.2): a one-layer reuse horizon after each relay refresh, alone and
    # with a post-refresh guard of 0.005, on the headline chain.
    hysteresis = None
    if not args.no_secondary:
        hysteresis = []
        for mr, ge in ((1, 0.0), (1, 0.005)):
            log(f"[bench] batched heads with hysteresis (min_reuse {mr}, gamma_extra {ge})")
            hysteresis.append(relay_vs_full(W.batched_heads().with_(name="batched_heads_hysteresis",
                                                                    min_reuse=mr, gamma_extra=ge),
                                            steps=3, warmup=1))
    # The headline workload with mandatory sentinels (one sink, two recent) in place of three
    # random ones: same c = 32, same kernels.
    mandatory = None
    if not args.no_secondary:
        log("[bench] batched heads with mandatory sentinels (sink 1, recent 2, r 5)")
        mandatory = relay_vs_full(W.batched_heads().with_(name="batched_heads_mandatory", sink=1,
                                                          recent=2, r=5), steps=3, warmup=1)

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
        "config": {"workload": "batched_heads", "heads": H, "nq": n, "nk": n, "d": d,
                   "layers": L, "anchors": list(w.anchors), "k": w.k, "m": w.m, "r": w.r,
                   "gamma": w.gamma, "causal": w.causal, "drift": "sigma_l ~ U[0.01, 0.06), relative",
                   "parallelism": "single GPU"},
        "speedup_vs_full": round(float(speedup), 4),
        "recall": round(q["recall"], 6),
        "reroute_fraction": round(q["reroute_fraction"], 4),
        "relay_rho_mean": round(q["relay_rho_mean"], 4),
        "pair_fraction": round(q["pair_fraction"], 4),
        "fixed_stride4_recall": round(q["stride4_recall"], 6),
        "relay_score_pairs_per_s": round(pairs_per_s, 1),
        "full_routing_routes_per_s": round(full_value, 1),
        "relay_layer_us_median": round(relay_layer_us, 2),
        "anchor_layer_us_median": round(anchor_layer_us, 2),
        "full_layer_us_median": round(full_layer_us, 2),
        "roofline": roofline,
        "kernels": kernels,
        "graph": graph,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "drift_sweep": drift_sweep,
        "sentinel_ablation": ablation,
        "mandatory_sentinels": mandatory,
        "preferred_chunks": preferred,
        "hysteresis": hysteresis,
        "width_buckets": buckets,
        "wide_near_miss": wide,
        "sparse_attention": attention,
        "sparse_attention_causal": attention_causal,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

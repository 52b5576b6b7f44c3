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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_batched_heads.txt")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_batched_heads.txt")
CALIB_BYTES = 256 << 20         # plain copy used to calibrate the HBM byte counters
# MI355X: 32 shader engines of 8 compute units, 4 SIMDs each; the SQ busy counter is per engine.
SIMDS_PER_SE = 32
L2_REQUEST_BYTES = 128          # one L1 -> L2 read request moves a 128-byte line
# Kernel symbols (as the profiler names them) -> keys of the profile summaries and the bench line,
# with the mangled name the build's resource report uses.
PROFILE_KERNELS = {"k_relay<rr::bf16_t, false>": "relay", "k_route<rr::bf16_t, false, false>": "route",
                   "k_route<rr::bf16_t, false, true>": "reroute", "k_rescore<rr::bf16_t, 1, 1>": "rescore",
                   "k_compact_out": "list"}
PROFILE_SYMBOLS = {"relay": "k_relayINS_6bf16_tELb0E", "route": "k_routeINS_6bf16_tELb0ELb0E",
                   "reroute": "k_routeINS_6bf16_tELb0ELb1E", "rescore": "k_rescoreINS_6bf16_tELi1ELi1E",
                   "list": "k_compact_out"}


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


RHO_BINS = ((0.0, 0.35), (0.35, 0.5), (0.5, 0.65), (0.65, 0.8), (0.8, 1.0))


def rho_breakdown(rho_per_layer, relay_ms, full_ms):
    """Relay against full routing layer by layer, grouped by the layer's flagged fraction rho
    (the chain's layers differ in drift): per bin the number of relay layers, their mean rho,
    and the mean over those layers of each layer's median relay and full-routing time (us)."""
    rows = [(rho, float(np.median(relay_ms[:, j])) * 1e3, float(np.median(full_ms[:, j])) * 1e3)
            for j, rho in enumerate(rho_per_layer)]
    out = []
    for lo, hi in RHO_BINS:
        sel = [x for x in rows if lo <= x[0] < hi or (hi == 1.0 and x[0] == 1.0)]
        if not sel:
            continue
        r = float(np.mean([x[1] for x in sel]))
        f = float(np.mean([x[2] for x in sel]))
        out.append({"rho": [lo, hi], "layers": len(sel), "rho_mean": round(float(np.mean([x[0] for x in sel])), 3),
                    "relay_layer_us": round(r, 2), "full_layer_us": round(f, 2), "speedup_vs_full": round(f / r, 4)})
    return out


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


def quality_only(w):
    """Untimed quality pass of one workload (relay chain and full-routing comparator)."""
    led = rr.Ledger(w.heads, w.nq, w.nk, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed,
                    sink=w.sink, recent=w.recent, min_reuse=w.min_reuse, gamma_extra=w.gamma_extra)
    full = rr.Ledger(w.heads, w.nq, w.nk, w.d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)
    qs, ks = upload_layers(w)
    q = quality_pass(w, led, full, qs, ks)
    led.close()
    full.close()
    return q


def drift_sweep_table2(sigmas=(0.01, 0.03, 0.06), seeds=10):
    """The drift-sweep workload as stated (1 head x 256 chunks, fp32, 16 layers, anchor stride 8,
    k = 12, m = 12, r = 8, ten seeds): per drift, the means over the seeds of the rerouted
    fraction and the recall against full routing (all layers and relay layers' rho), the
    analogue of the page's Table 2; relay and full-routing layer times at seed 0 (one head
    of 256 rows: launch-bound)."""
    import torch
    out = []
    for sigma in sigmas:
        acc = np.zeros(5)
        for seed in range(seeds):
            q = quality_only(W.drift_sweep(sigma, seed))
            acc += [q["recall"], q["reroute_fraction"], q["relay_rho_mean"], q["pair_fraction"],
                    q["stride4_recall"]]
        acc /= seeds
        t = relay_vs_full(W.drift_sweep(sigma, 0), steps=5, warmup=2)
        out.append({"sigma": sigma, "seeds": seeds, "recall": round(float(acc[0]), 6),
                    "reroute_fraction": round(float(acc[1]), 4), "relay_rho_mean": round(float(acc[2]), 4),
                    "pair_fraction": round(float(acc[3]), 4), "fixed_stride4_recall": round(float(acc[4]), 6),
                    "relay_layer_us_median_seed0": t["relay_layer_us_median"],
                    "full_layer_us_median_seed0": t["full_layer_us_median"],
                    "speedup_vs_full_seed0": t["speedup_vs_full"]})
    torch.cuda.empty_cache()
    return out


def scale_sweep_table4(ns=(128, 256, 512, 1024), seeds=3):
    """The scale-sweep workload as stated (1 head, n in {128, 256, 512, 1024} chunks, bf16,
    32 layers, drift 0.03, anchor stride 8, k = 12, m = 12, r = 8), seeds 0-2 like the page's
    three seeds: per n, the means of the fraction of full-routing score pairs evaluated, the
    recall, the rerouted fraction and relay rho (the analogue of the page's Table 4); relay
    routes/s, layer times and speedup against the same GPU's full routing at seed 0."""
    import torch
    out = []
    for n in ns:
        acc = np.zeros(4)
        for seed in range(seeds):
            q = quality_only(W.scale_sweep(n, seed))
            acc += [q["pair_fraction"], q["recall"], q["reroute_fraction"], q["relay_rho_mean"]]
        acc /= seeds
        t = relay_vs_full(W.scale_sweep(n, 0), steps=5, warmup=2)
        out.append({"n": n, "seeds": seeds, "pair_fraction": round(float(acc[0]), 4),
                    "recall": round(float(acc[1]), 6), "reroute_fraction": round(float(acc[2]), 4),
                    "relay_rho_mean": round(float(acc[3]), 4),
                    "relay_routes_per_s_seed0": t["relay_routes_per_s"],
                    "full_routing_routes_per_s_seed0": t["full_routing_routes_per_s"],
                    "relay_layer_us_median_seed0": t["relay_layer_us_median"],
                    "full_layer_us_median_seed0": t["full_layer_us_median"],
                    "speedup_vs_full_seed0": t["speedup_vs_full"]})
    torch.cuda.empty_cache()
    return out


def sentinel_ablation(seeds=5):
    """Sentinel mixes on the pages' ablation setting (1 x 256 chunks, fp32, 24 layers, drift
    0.003, k = 12; anchors every 8 layers, as in the other chains): mean recall against full
    routing, rerouted fraction and score-pair fraction over the seeds.  The 24- and 48-wide
    near-miss rows run on the one-wave-per-row kernel (k + m = 36 and 60; the 48-wide row keeps
    c = 72 ledger entries per row).  The
    last mix trades three random sentinels for the mandatory kind (Section 3.1, item 3: one
    sink chunk, two recent chunks); the synthetic walk gives those chunks no special role,
    and a pair count of c per row is an upper bound when one of them is already routed."""
    import torch
    mixes = [("random only", 0, 12, 0, 0), ("near-miss only", 12, 0, 0, 0),
             ("12 near-miss + 12 random", 12, 12, 0, 0), ("12 near-miss + 8 random", 12, 8, 0, 0),
             ("12 near-miss + 1 sink + 2 recent + 5 random", 12, 5, 1, 2),
             ("24 near-miss + 12 random", 24, 12, 0, 0), ("48 near-miss + 12 random", 48, 12, 0, 0)]
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
            # every byte moved once (Q, K, V, O): the bound a perfect reuse of routed chunks would meet
            "hbm_unique": {"bytes": unique, "achieved": round(unique / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": round(unique / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "gathered_over_unique": round(gathered / unique, 2)},
            "unique_bytes": unique}


def width_buckets(steps=3, warmup=1):
    """Query-dependent route widths through width-bucketed ledgers (Sections 4.3-4.4) on the
    headline chain: even query rows route with k = 8 (m = 12, r = 8), odd rows with k = 16
    (m = 12, r = 4); the comparator routes every row in full at its own width.  Both advance
    their buckets together (rr_anchor_route_group / rr_relay_layer_group: one launch per layer
    for all buckets).  Recall is against each row's own exact top-k."""
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
    group, full_group = rr.LedgerGroup(leds), rr.LedgerGroup(fulls)
    recall, rerouted = 0.0, 0
    for l in range(w.layers):
        if w.is_anchor(l):
            group.anchor(qs[l], ks[l], l)
        else:
            group.relay(qs[l], ks[l], l, outs)
        full_group.anchor(qs[l], ks[l], l)
        torch.cuda.synchronize()
        for led, full, o in zip(leds, fulls, outs):
            used = led.get()[0].cpu().numpy().reshape(-1, led.k)
            exact = full.get()[0].cpu().numpy().reshape(-1, led.k)
            recall += route_recall(used, exact) * led.nq / n
            rerouted += H * led.nq if w.is_anchor(l) else int(o.n_rows.cpu().numpy()[0])
    relay_ms, full_ms, _ = time_chains(w, group, full_group, qs, ks, steps, warmup)
    relay_layers = [l for l in range(w.layers) if not w.is_anchor(l)]
    t_relay, t_full = relay_ms[:, relay_layers].sum(), full_ms.sum()
    out = {"workload": "batched_heads, two width buckets",
           "buckets": [{"rows": "even query rows", "k": 8, "m": 12, "r": 8},
                       {"rows": "odd query rows", "k": 16, "m": 12, "r": 4}],
           "launch": "one grid per layer for both buckets (grouped calls)",
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


def relay_vs_full(w, steps, warmup, mode="auto", with_quality=True):
    import torch
    H, n = w.heads, w.n
    qs, ks = upload_layers(w)
    led = rr.Ledger(H, n, n, w.d, w.k, w.m, w.r, w.gamma, w.causal, w.dtype, w.seed,
                    sink=w.sink, recent=w.recent, min_reuse=w.min_reuse, gamma_extra=w.gamma_extra)
    led.set_relay_mode(mode)
    full = rr.Ledger(H, n, n, w.d, w.k, 0, 0, w.gamma, w.causal, w.dtype, w.seed)
    q = quality_pass(w, led, full, qs, ks) if with_quality else None
    relay_ms, full_ms, _ = time_chains(w, led, full, qs, ks, steps, warmup)
    relay_layers = [l for l in range(w.layers) if not w.is_anchor(l)]
    t_relay = relay_ms[:, relay_layers].sum()
    t_full = full_ms.sum()
    out = {"workload": w.name, "heads": H, "nq": n, "nk": n, "causal": w.causal, "layers": w.layers,
           "k": w.k, "m": w.m, "r": w.r, "sink": w.sink, "recent": w.recent,
           "min_reuse": w.min_reuse, "gamma_extra": w.gamma_extra, "relay_mode": mode,
           "relay_routes_per_s": round(H * n * len(relay_layers) * steps / (t_relay / 1e3), 1),
           "full_routing_routes_per_s": round(H * n * w.layers * steps / (t_full / 1e3), 1),
           "speedup_vs_full": round(float((t_full / (w.layers * steps)) / (t_relay / (len(relay_layers) * steps))), 4),
           "relay_layer_us_median": round(float(np.median(relay_ms[:, relay_layers]) * 1e3), 2),
           "full_layer_us_median": round(float(np.median(full_ms) * 1e3), 2),
           "steps": steps}
    if q is not None:
        out.update({"recall": round(q["recall"], 6), "reroute_fraction": round(q["reroute_fraction"], 4),
                    "relay_rho_mean": round(q["relay_rho_mean"], 4), "pair_fraction": round(q["pair_fraction"], 4),
                    "fixed_stride4_recall": round(q["stride4_recall"], 6)})
    led.close()
    full.close()
    del qs, ks
    torch.cuda.empty_cache()
    return out


CPU_WORKERS_MAX = 16             # the GPU machine's CPU share for one GPU


def _cpu_head_chain(args):
    """One worker of cpu_baseline: the oracle, unmodified, on one head of the workload (its own
    seeded layers), for as many chain layers as fit in `budget` seconds (at least two relay
    layers), with single-threaded BLAS.  Returns (anchor layers, their seconds, relay layers,
    their seconds)."""
    w, h, budget = args
    import oracle as O
    from threadpoolctl import threadpool_limits
    cfg = O.RouteConfig(heads=1, nq=w.n, nk=w.n, d=w.d, k=w.k, m=w.m, r=w.r, gamma=w.gamma,
                        causal=w.causal, seed=w.seed, dtype=w.dtype)
    t_relay = t_anchor = 0.0
    n_relay = n_anchor = 0
    led = None
    t_start = time.perf_counter()
    with threadpool_limits(limits=1):
        for li in synth.generate(w, slice(h, h + 1)):
            t0 = time.perf_counter()
            if led is None or w.is_anchor(li.layer):
                led = O.anchor_layer(cfg, li.q, li.k, li.layer)
                t_anchor += time.perf_counter() - t0
                n_anchor += 1
            else:
                led = O.relay_layer(cfg, li.q, li.k, li.layer, led).ledger
                t_relay += time.perf_counter() - t0
                n_relay += 1
            if time.perf_counter() - t_start > budget and n_relay >= 2:
                break
    return n_anchor, t_anchor, n_relay, t_relay


def cpu_baseline(w, max_seconds=20.0):
    """The oracle, unmodified, on a bounded sample of the same workload, on the host's cores:
    one worker process per core (at most CPU_WORKERS_MAX), each running one head's chain with
    single-threaded BLAS for ~max_seconds; heads are independent, so the workers' rates add up.
    Call it before the GPU is initialised: the workers are started as fresh interpreters."""
    import multiprocessing as mp
    cores = max(1, min(len(os.sched_getaffinity(0)), CPU_WORKERS_MAX, w.heads))
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_cpu_head_chain, [(w, h, max_seconds) for h in range(cores)])
    rows = w.n
    relay_rate = sum(rows * nr / tr for _, _, nr, tr in res)
    full_rate = sum(rows * na / ta for na, ta, _, _ in res)
    per_relay = float(np.mean([tr / nr for _, _, nr, tr in res]))
    per_anchor = float(np.mean([ta / na for na, ta, _, _ in res]))
    n_rel = [nr for _, _, nr, _ in res]
    n_anc = [na for na, _, _, _ in res]
    return {"value": relay_rate, "unit": "relay-layer query-row routes/s",
            "cores": cores, "kind": "oracle",
            "sample": f"heads 0-{cores - 1} of {w.heads}, one head per worker process (single-threaded "
                      f"NumPy each), {min(n_anc)}-{max(n_anc)} anchor and {min(n_rel)}-{max(n_rel)} relay "
                      f"layers per head from layer 0 (~{max_seconds:g} s per worker); value = sum of the "
                      f"workers' relay-layer rates",
            "full_routing_value": full_rate,
            "relay_over_full_time": per_relay / per_anchor}


def kernel_build_hash():
    """sha256 of the kernel source and its headers, followed by the build script (its compiler
    flags)."""
    h = hashlib.sha256()
    for path in (*KERNEL_SRCS, BUILD_SCRIPT):
        h.update(open(path, "rb").read())
    return h.hexdigest()


def _summary_fields(path):
    """key: value lines of a committed profile summary, or None when it is missing or was taken
    on another kernel source or build script than the current one."""
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    return fields if fields.get("kernel_build_sha256") == kernel_build_hash() else None


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` (relay / route / rescore / reroute) from the committed
    counter summary, if it was taken on the kernel source and build script as they are now (else
    None)."""
    fields = _summary_fields(TRAFFIC_FILE)
    try:
        return float(fields[f"{kernel}_hbm_bytes_per_launch"]) if fields else None
    except (KeyError, ValueError):
        return None


def recorded_counters(kernel):
    """Measured utilisation of `kernel` from the committed counter summary (same validity rule
    as recorded_traffic): VALU and MFMA busy fractions of the SIMD cycles, LDS bank-conflict
    share of LDS cycles, L1 -> L2 read bytes per launch."""
    fields = _summary_fields(COUNTERS_FILE)
    if not fields:
        return None
    out = {}
    for name in ("valu_busy", "mfma_busy", "lds_bank_conflict_frac", "l2_read_bytes_per_launch",
                 "valu_insts_per_wave", "vgprs"):
        try:
            out[name] = float(fields[f"{kernel}_{name}"])
        except (KeyError, ValueError):
            pass
    return out or None


def _pmc_medians(csv_path):
    """{profile key: {counter: median over the run's dispatches}} from one rocprofv3 counter
    collection file.  "calib_copy": the largest value any device copy dispatch shows for each
    counter (the run's one 256 MiB copy, bench.py --calib-copy, is its largest copy)."""
    import csv
    vals, calib = {}, {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            value = float(row["Counter_Value"])
            if "copyBuffer" in name and "Rect" not in name:
                calib[row["Counter_Name"]] = max(calib.get(row["Counter_Name"], 0.0), value)
                continue
            key = next((v for k, v in PROFILE_KERNELS.items() if k in name), None)
            if key is None:
                continue
            vals.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(value)
    out = {k: {c: float(np.median(v)) for c, v in d.items()} for k, d in vals.items()}
    if calib:
        out["calib_copy"] = calib
    return out


def summarize_profiles(out_dir, cmd_line):
    """Write profiles/traffic_batched_heads.txt and profiles/counters_batched_heads.txt from the
    counter runs under `out_dir` (rocprofv3 --pmc, one pass per run, each under
    <out_dir>/<schedule>_<pass>/, schedules auto and compacted, passes util, mem, fetch, write;
    see the command lines written into the files)."""
    import glob
    runs = {}
    for f in sorted(glob.glob(os.path.join(out_dir, "*", "*counter_collection.csv"))):
        tag = os.path.basename(os.path.dirname(f))
        runs[tag] = _pmc_medians(f)
    med = {}
    for tag, per_kernel in runs.items():
        for key, cs in per_kernel.items():
            med.setdefault(key, {}).update(cs)
    h = kernel_build_hash()
    try:
        import json
        from long_context_prefill_anchor_amd import build as B
        resources = json.load(open(B.RESOURCES))
    except (OSError, ValueError):
        resources = {}
    calib = med.get("calib_copy", {})
    fetch_scale = (CALIB_BYTES / 1024) / calib["FETCH_SIZE"] if calib.get("FETCH_SIZE") else None
    write_scale = (CALIB_BYTES / 1024) / calib["WRITE_SIZE"] if calib.get("WRITE_SIZE") else None
    head = [f"# Command (rocprofv3 under {cmd_line.split()[0]}): one run per counter pass and relay schedule,",
            f"#   {cmd_line}",
            "# Values are medians over every dispatch of the kernel in the run; valid only for the kernel",
            "# source and build script with the hash below (sha256 of rr_kernels.hip, rr_device.h and",
            "# rr_internal.h, followed by build.py).",
            f"kernel_build_sha256: {h}"]
    t = ["# HBM traffic per launch, batched-heads workload (32 heads x 1024 chunks, d = 64, bf16).",
         f"# Calibration: one plain {CALIB_BYTES >> 20} MiB device copy (bench.py --calib-copy) reads and",
         "# writes that many bytes; its FETCH_SIZE / WRITE_SIZE (KiB as counted) give the scales that",
         "# turn counted KiB into bytes moved."] + head
    t.append(f"fetch_scale: {fetch_scale:.4f}" if fetch_scale else "fetch_scale: none")
    t.append(f"write_scale: {write_scale:.4f}" if write_scale else "write_scale: none")
    c = ["# Utilisation per kernel, batched-heads workload (32 heads x 1024 chunks, d = 64, bf16).",
         "# valu_busy  = SQ_ACTIVE_INST_VALU * 4 / (SQ_BUSY_CYCLES * 32): VALU issue cycles over SIMD",
         "#              cycles (the active-instruction counter is in quad-cycles summed over waves, the",
         "#              busy counter is per shader engine of 32 SIMDs);",
         "# mfma_busy  = SQ_VALU_MFMA_BUSY_CYCLES / (SQ_BUSY_CYCLES * 32);",
         "# lds_bank_conflict_frac = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS;",
         "# l2_read_bytes_per_launch = TCP_TCC_READ_REQ_sum * 128 (L1 -> L2 read requests of one line);",
         "# vgprs, scratch and occupancy from the build's resource report (librr.resources.json);",
         "# wait_frac = SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave time spent waiting on memory, LDS or barriers)."] + head
    for key in ("relay", "route", "rescore", "reroute", "list"):
        cs = med.get(key)
        if not cs:
            continue
        if fetch_scale and "FETCH_SIZE" in cs and write_scale and "WRITE_SIZE" in cs:
            rd, wr = cs["FETCH_SIZE"] * 1024 * fetch_scale, cs["WRITE_SIZE"] * 1024 * write_scale
            t += [f"{key}_fetch_kib_counted: {cs['FETCH_SIZE']:.1f}", f"{key}_write_kib_counted: {cs['WRITE_SIZE']:.1f}",
                  f"{key}_hbm_read_bytes_per_launch: {rd:.0f}", f"{key}_hbm_write_bytes_per_launch: {wr:.0f}",
                  f"{key}_hbm_bytes_per_launch: {rd + wr:.0f}"]
        busy = cs.get("SQ_BUSY_CYCLES")
        if busy:
            c.append(f"{key}_valu_busy: {cs['SQ_ACTIVE_INST_VALU'] * 4 / (busy * SIMDS_PER_SE):.4f}")
            c.append(f"{key}_mfma_busy: {cs['SQ_VALU_MFMA_BUSY_CYCLES'] / (busy * SIMDS_PER_SE):.4f}")
        if cs.get("SQ_WAVES"):
            c.append(f"{key}_valu_insts_per_wave: {cs['SQ_INSTS_VALU'] / cs['SQ_WAVES']:.0f}")
            if cs.get("SQ_INSTS_LDS") is not None:
                c.append(f"{key}_lds_insts_per_wave: {cs['SQ_INSTS_LDS'] / cs['SQ_WAVES']:.0f}")
        if cs.get("SQ_ACTIVE_INST_LDS"):
            c.append(f"{key}_lds_bank_conflict_frac: {cs['SQ_LDS_BANK_CONFLICT'] / cs['SQ_ACTIVE_INST_LDS']:.4f}")
        if cs.get("TCP_TCC_READ_REQ_sum") is not None:
            c.append(f"{key}_l2_read_bytes_per_launch: {cs['TCP_TCC_READ_REQ_sum'] * L2_REQUEST_BYTES:.0f}")
        if cs.get("SQ_WAVE_CYCLES") and cs.get("SQ_WAIT_ANY") is not None:
            c.append(f"{key}_wait_frac: {cs['SQ_WAIT_ANY'] / cs['SQ_WAVE_CYCLES']:.4f}")
        res = next((u for sym, u in resources.items() if PROFILE_SYMBOLS[key] in sym), None)
        if res:
            c.append(f"{key}_vgprs: {res.get('VGPRs')}")
            c.append(f"{key}_scratch_bytes_per_lane: {res.get('ScratchSize [bytes/lane]')}")
            c.append(f"{key}_occupancy_waves_per_simd: {res.get('Occupancy [waves/SIMD]')}")
        for name in sorted(cs):
            c.append(f"{key}.{name}: {cs[name]:.1f}")
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(t) + "\n")
    with open(COUNTERS_FILE, "w") as f:
        f.write("\n".join(c) + "\n")
    print(TRAFFIC_FILE)
    print(COUNTERS_FILE)


def calib_copy():
    """A plain device copy of known size (CALIB_BYTES read + written), for counter calibration."""
    import torch
    a = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b


# Phase-trace slots (see RR_STAMP in csrc/rr_kernels.hip): what each stamp follows.
PHASE_SLOTS = {0: "start", 1: "keys staged (relay) / first pass done (route)", 2: "rescored (relay) / threshold set (route)",
               3: "flags ready (relay)", 4: "compacted (relay)", 5: "streaming pass done", 6: "final drain done",
               7: "drain barrier", 8: "lists exchanged", 9: "quad merge done", 10: "merge barrier",
               13: "bitmap built", 14: "random draws done", 15: "segments sorted", 11: "ledger written",
               12: "end barrier"}


def phase_trace():
    """Per-phase durations of the route and relay kernels at the batched-heads shape, from the
    measurement build (python -m long_context_prefill_anchor_amd.build --phase-trace): the first
    lane of every wave stamps the 100 MHz real-time counter at fixed points; per phase, the
    median and 90th percentile over all waves of one launch (us), the spread of each block's
    waves at each stamp, and the waves' mid-stream drain counts."""
    import ctypes
    import torch
    L = rr.lib()
    L.rr_debug_phase_trace.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t]
    NB, NW, NS = 4096, 8, 16

    def trace(fn, nblocks, nw, chain, nflag=None):
        assert L.rr_debug_phase_clear() == 0
        torch.cuda.synchronize()
        fn()
        torch.cuda.synchronize()
        st = np.zeros(NB * NW * NS, np.uint64)
        dr = np.zeros(NB * NW, np.uint32)
        assert L.rr_debug_phase_trace(st.ctypes.data, st.size, dr.ctypes.data, dr.size) == 0
        t = st.reshape(NB, NW, NS)[:nblocks, :nw].astype(np.int64)
        live = t[:, 0, 0] > 0
        bidx = np.nonzero(live)[0]
        t, dr = t[live], dr.reshape(NB, NW)[:nblocks, :nw][live]
        out = {"blocks": int(live.sum())}
        phases = {}
        for a, b in zip(chain[:-1], chain[1:]):
            m = (t[:, :, a] > 0) & (t[:, :, b] > 0)
            d = (t[:, :, b] - t[:, :, a])[m] / 100.0
            if d.size:
                phases[f"{PHASE_SLOTS[a]} -> {PHASE_SLOTS[b]}"] = [round(float(np.median(d)), 2),
                                                                   round(float(np.percentile(d, 90)), 2)]
        out["phase_us_median_p90"] = phases
        end = t[:, :, chain[-1]]
        ok = (end > 0).all(axis=1)
        chains = (end[ok].max(axis=1) - t[ok, :, 0].min(axis=1)) / 100.0
        out["block_chain_us_median"] = round(float(np.median(chains)), 2)
        # spread of the blocks' chains, and of their start and end times over the launch (the
        # launch lasts from the first start to the last end)
        starts, ends = t[ok, :, 0].min(axis=1), end[ok].max(axis=1)
        t0 = starts.min()
        out["block_chain_us_p10_p90_max"] = [round(float(np.percentile(chains, 10)), 2),
                                             round(float(np.percentile(chains, 90)), 2), round(float(chains.max()), 2)]
        out["block_start_us_p90_max"] = [round(float(np.percentile((starts - t0) / 100.0, 90)), 2),
                                         round(float((starts.max() - t0) / 100.0), 2)]
        out["launch_span_us"] = round(float((ends.max() - t0) / 100.0), 2)
        out["drains_per_wave"] = {int(k): int(c) for k, c in zip(*np.unique(dr, return_counts=True))}
        if nflag is not None:
            # Fused relay blocks by their flagged rows: one reroute slice (<= 64) or two.
            nf = nflag[bidx[ok]]
            out["flagged_rows_per_block_mean"] = round(float(nf.mean()), 1)
            for name, sel in (("one_slice", nf <= 64), ("two_slices", nf > 64)):
                c = chains[sel]
                out[f"{name}_blocks"] = int(sel.sum())
                if c.size:
                    out[f"{name}_chain_us_median_max"] = [round(float(np.median(c)), 2), round(float(c.max()), 2)]
            if nf.std() > 0 and chains.std() > 0:
                out["chain_vs_flagged_corr"] = round(float(np.corrcoef(nf, chains)[0, 1]), 3)
        return out

    w = W.batched_heads()
    gen = synth.generate(w)
    l0, l1 = next(gen), next(gen)
    H, n = w.heads, w.n
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()  # noqa: E731
    q0, k0, q1, k1 = up(l0.q), up(l0.k), up(l1.q), up(l1.k)
    led = rr.Ledger(H, n, n, 64, w.k, w.m, w.r, 0.0, False, "bf16", w.seed)
    full = rr.Ledger(H, n, n, 64, w.k, 0, 0, 0.0, False, "bf16", w.seed)
    for _ in range(3):
        led.anchor(q0, k0, 0)
        full.anchor(q0, k0, 0)
    route = [0, 1, 2, 5, 6, 7, 8, 9, 10, 13, 14, 15, 11, 12]
    res = {"workload": "batched_heads, layers 0 (anchor) and 1 (relay)"}
    res["full_routing"] = trace(lambda: full.anchor(q1, k1, 1), H * 16, 4, route)
    res["anchor"] = trace(lambda: led.anchor(q0, k0, 0), H * 16, 4, route)
    led.set_relay_mode("fused")
    led.anchor(q0, k0, 0)
    led.relay(q1, k1, 1)
    led.anchor(q0, k0, 0)
    res["relay_fused"] = trace(lambda: led.relay(q1, k1, 1), H * 8, 8, [0, 1, 2, 3, 4] + route[3:])
    led.set_relay_mode("compacted")
    led.anchor(q0, k0, 0)
    res["reroute_compacted"] = trace(lambda: led.relay(q1, k1, 1), H * 16, 4, [0, 2] + route[3:])
    led.close()
    # The fused relay layer at fixed drifts (layer 1 after an anchor at layer 0), with each
    # block's chain set against its flagged rows, beside full routing of the same layer.
    by_drift = []
    for sigma in (0.01, 0.03, 0.06):
        wd = w.with_(name=f"phase_drift{sigma:g}", drift=(sigma, sigma))
        g = synth.generate(wd)
        a0, a1 = next(g), next(g)
        qa, ka, qb, kb = up(a0.q), up(a0.k), up(a1.q), up(a1.k)
        ld = rr.Ledger(H, n, n, 64, w.k, w.m, w.r, 0.0, False, "bf16", w.seed)
        ld.set_relay_mode("fused")
        outs = ld.alloc_outputs(with_scores=False)
        ld.anchor(qa, ka, 0)
        ld.relay(qb, kb, 1, outs)
        torch.cuda.synchronize()
        # flagged rows of each 128-row fused block, in the kernel's block order (h * n/128 + g)
        nflag = outs.flags.cpu().numpy().astype(np.int64).reshape(H, n // 128, 128).sum(axis=2).reshape(-1)
        ld.anchor(qa, ka, 0)
        r = trace(lambda: ld.relay(qb, kb, 1), H * 8, 8, [0, 1, 2, 3, 4] + route[3:], nflag=nflag)
        f = trace(lambda: full.anchor(qb, kb, 1), H * 16, 4, route)
        by_drift.append({"sigma": sigma, "rho": round(float(nflag.sum()) / (H * n), 4),
                         "relay_fused": {k: v for k, v in r.items() if k != "phase_us_median_p90"},
                         "full_routing": {k: f[k] for k in ("block_chain_us_median", "block_chain_us_p10_p90_max",
                                                            "launch_span_us")}})
        ld.close()
    res["relay_fused_by_drift"] = by_drift
    full.close()
    return res


def side(fn, *a, **kw):
    """A side measurement: its result, or {"error": ...} if it fails (the headline stands)."""
    try:
        return fn(*a, **kw)
    except Exception as e:                               # noqa: BLE001 - recorded in the line
        log(f"[bench] side measurement {fn.__name__} failed: {e!r}")
        return {"error": f"{type(e).__name__}: {e}"}


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
    ap.add_argument("--relay-mode", default="auto", choices=list(rr.RELAY_MODES),
                    help="relay schedule of the headline chain (include/rr.h, rr_ledger_set_relay_mode)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ counter summaries from rocprofv3 --pmc runs under DIR and exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summaries")
    ap.add_argument("--phase-trace", action="store_true",
                    help="per-phase kernel durations from the measurement build "
                         "(python -m long_context_prefill_anchor_amd.build --phase-trace); prints its JSON")
    ap.add_argument("--calib-copy", action="store_true",
                    help=f"run one plain {CALIB_BYTES >> 20} MiB device copy first (counter calibration)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.profile_command or "rocprofv3 --pmc <counters> -- python3 bench.py")
        return
    if args.phase_trace:
        from long_context_prefill_anchor_amd import build as B
        if not os.path.exists(B.PHASE_LIB):
            print(f"{B.PHASE_LIB} is missing: python -m long_context_prefill_anchor_amd.build --phase-trace",
                  file=sys.stderr)
            sys.exit(2)
        rr.LIB_PATH = B.PHASE_LIB
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); heads shard across GPUs "
              "with no exchange, so run one process per GPU on its own heads.", file=sys.stderr)
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline and not args.only_attention:
        # before the GPU is initialised: the oracle's worker processes start from a clean parent
        log("[bench] cpu_baseline: oracle on a bounded sample, on the host cores")
        cpu = cpu_baseline(W.batched_heads(), args.cpu_seconds)
        log(f"[bench] cpu_baseline: {cpu['value']:.1f} routes/s on {cpu['cores']} cores")

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    rr.lib()
    if args.phase_trace:
        print(json.dumps({"phase_trace": phase_trace()}), flush=True)
        return
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
    led.set_relay_mode(args.relay_mode)
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
    relay_vs_rho = rho_breakdown(q["relay_rho_per_layer"], relay_ms[:, relay_layers], full_ms[:, relay_layers])

    # Per-kernel averages from the library's own launch events (same stream as the kernels).
    def avg_us(kt, kind):
        nl, ms = kt[kind]
        return (ms * 1e3 / nl) if nl else None, nl
    t_resc, n_resc = avg_us(kt_led, rr.RR_KERNEL_RESCORE)
    t_rer, n_rer = avg_us(kt_led, rr.RR_KERNEL_REROUTE)
    t_rel, n_rel = avg_us(kt_led, rr.RR_KERNEL_RELAY)
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

    # rescoring flops: 2*d per candidate of every row (the fused kernel's first phase)
    rescore_flops = 2.0 * d * H * n * w.c
    kernels = {
        "full_routing": mfma_line("k_route<bf16, full> (k=12, m=r=0)", full_flops, t_full, n_full),
        "anchor": mfma_line("k_route<bf16, full> (k=12, m=12, r=8)", full_flops, t_anc, n_anc),
    }
    # Measured utilisation beside the roofline fractions (committed counter summary; the route
    # kernel's figures are medians over its full-routing and anchor launches, 32 of them full
    # routing for every 4 anchors).
    kernels["full_routing"]["counters"] = recorded_counters("route")
    kernels["full_routing"]["traffic"] = recorded_traffic("route")
    roofline = None
    if n_rel:
        # fused relay layer: the rescoring of every row plus the full scoring of the flagged rows
        rel = mfma_line("k_relay<bf16> (rescore + compaction + reroute of flagged rows)",
                        rescore_flops + reroute_flops, t_rel, n_rel)
        ach_b = rescore_bytes / (t_rel * 1e-6) / 1e9
        rel["rescore_bytes"] = {"bytes": rescore_bytes, "achieved": round(ach_b, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(ach_b / HBM_PEAK_GBS, 4)}
        rel["traffic"] = recorded_traffic("relay")
        rel["counters"] = recorded_counters("relay")
        kernels["relay"] = rel
        roofline = dict(rel)
    if n_resc:
        ach_resc = rescore_bytes / (t_resc * 1e-6) / 1e9
        kernels["rescore"] = {"kernel": "k_rescore<bf16, 1>", "bound": "hbm", "achieved": round(ach_resc, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach_resc / HBM_PEAK_GBS, 4),
                              "per_launch": {"bytes": rescore_bytes, "avg_us": round(t_resc, 2), "launches": n_resc},
                              "traffic": recorded_traffic("rescore"), "counters": recorded_counters("rescore")}
        ctr = kernels["rescore"]["counters"]
        if ctr and "l2_read_bytes_per_launch" in ctr:
            # the gathers' L1 -> L2 bytes beside the algorithmic HBM bytes
            ach_l2 = ctr["l2_read_bytes_per_launch"] / (t_resc * 1e-6) / 1e9
            kernels["rescore"]["l2_read"] = {"bytes": ctr["l2_read_bytes_per_launch"], "achieved": round(ach_l2, 1),
                                             "unit": "GB/s"}
    if n_rer:
        rer = mfma_line("k_route<bf16, reroute> (flagged rows)", reroute_flops, t_rer, n_rer)
        rer["traffic"] = recorded_traffic("reroute")
        rer["counters"] = recorded_counters("reroute")
        kernels["reroute"] = rer
        if roofline is None:
            roofline = dict(rer)

    led.close()
    full.close()
    del qs, ks
    torch.cuda.empty_cache()
    secondary = None if args.no_secondary else side(secondary_causal)
    relay_modes = None
    if not args.no_secondary:
        # the fused schedule needs a head's keys in 128 KB of LDS: the 1024-chunk workload only
        relay_modes = []
        for wl, modes in ((W.batched_heads(), ("fused", "compacted")), (W.causal_large(), ("compacted",))):
            for mode in modes:
                log(f"[bench] relay schedule {mode}: {wl.name}")
                r = side(relay_vs_full, wl, steps=3, warmup=1, mode=mode, with_quality=False)
                relay_modes.append({k: r[k] for k in ("workload", "relay_mode", "relay_layer_us_median",
                                                      "full_layer_us_median", "speedup_vs_full",
                                                      "relay_routes_per_s")} if "error" not in r else r)
    drift_sweep = None if args.no_secondary else side(drift_sweep_batched)
    drift_t2 = scale_t4 = None
    if not args.no_secondary:
        log("[bench] drift sweep workload (1 x 256 fp32, ten seeds per drift)")
        drift_t2 = side(drift_sweep_table2)
        log("[bench] scale sweep workload (1 x {128 .. 1024} bf16, three seeds per size)")
        scale_t4 = side(scale_sweep_table4)
    ablation = None if args.no_secondary else side(sentinel_ablation)
    preferred = None if args.no_secondary else side(preferred_chunks_sweep)
    buckets = None if args.no_secondary else side(width_buckets)
    wide = None
    if not args.no_secondary:
        log("[bench] batched heads with a 24-wide near-miss set (k + m = 36: one-wave-per-row kernel)")
        wide = side(relay_vs_full, W.batched_heads().with_(name="batched_heads_nm24", m=24, r=8), steps=2, warmup=1)
    attention, attention_causal = None, None
    if not args.no_secondary:
        log("[bench] sparse attention over the routes (token expansion, Eq. 3)")
        attention = side(sparse_attention_measure)
        if "error" not in attention:
            attention["routing_relay_layer_us"] = round(relay_layer_us, 2)
            attention["routing_share_of_layer"] = round(relay_layer_us / (relay_layer_us + attention["avg_us"]), 4)
        log("[bench] causal sparse attention at the 64 x 4096 shape")
        attention_causal = side(sparse_attention_measure, reps=5, causal=True)
        if secondary is not None and "error" not in secondary and "error" not in attention_causal:
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
            hysteresis.append(side(relay_vs_full, W.batched_heads().with_(name="batched_heads_hysteresis",
                                                                          min_reuse=mr, gamma_extra=ge),
                                   steps=3, warmup=1))
    # The headline workload with mandatory sentinels (one sink, two recent) in place of three
    # random ones: same c = 32, same kernels.
    mandatory = None
    if not args.no_secondary:
        log("[bench] batched heads with mandatory sentinels (sink 1, recent 2, r 5)")
        mandatory = side(relay_vs_full, W.batched_heads().with_(name="batched_heads_mandatory", sink=1,
                                                                recent=2, r=5), steps=3, warmup=1)

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
                   "relay_schedule": args.relay_mode, "parallelism": "single GPU"},
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
        "relay_vs_rho": relay_vs_rho,
        "roofline": roofline,
        "kernels": kernels,
        "graph": graph,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "relay_modes": relay_modes,
        "drift_sweep": drift_sweep,
        "drift_sweep_1x256": drift_t2,
        "scale_sweep": scale_t4,
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

"""Chain statistics against the page's reported directions.

The page's generator (Section 5.1, "persistent preferred chunks together with
layer-local Gaussian drift") is not specified, so recall / reroute / pair values
are parity unpinned; only the directions the page reports are checked.  The
``preferred_chunks`` workload is this build's reading of that generator.
"""
import numpy as np
import pytest

import oracle as O
from long_context_prefill_anchor_amd import synth, workloads as W


def chain_stats(w, with_stride4=False):
    cfg = O.RouteConfig(heads=w.heads, nq=w.nq, nk=w.nk, d=w.d, k=w.k, m=w.m, r=w.r,
                        gamma=w.gamma, causal=w.causal, seed=w.seed, dtype=w.dtype)
    recs = O.run_chain(cfg, synth.generate(w), w.anchors)
    kinds = [x.kind for x in recs]
    flags = [x.flags for x in recs]
    rho = O.reroute_fraction(kinds, flags, w.heads * w.nq)
    recall = float(np.mean([O.route_recall(x.used_route, x.exact_route) for x in recs]))
    n_row = np.array([O.n_allowed(i, cfg) for i in range(w.nq)])
    ev, full = O.pair_counts(kinds, w.heads, n_row, flags, [x.cand_count for x in recs])
    if not with_stride4:
        return rho, recall, ev / full
    # fixed stride 4 (Section 5.1): exact routes at layers 0, 4, 8, ... reused in between
    stale = [recs[4 * (x.layer // 4)].exact_route for x in recs]
    s4 = float(np.mean([O.route_recall(st, x.exact_route) for st, x in zip(stale, recs)]))
    return rho, recall, ev / full, s4


def test_reroute_fraction_rises_with_drift():
    """Table 2 / Section 5.1: more drift, more rerouted rows."""
    rhos = [chain_stats(W.drift_sweep(s, seed=0))[0] for s in (0.01, 0.03, 0.06)]
    assert rhos[0] < rhos[1] < rhos[2]


def test_preferred_chunks_generator_layout():
    """Persistent preferred chunks with layer-local drift: shapes nq x nk; the drift does not
    accumulate (layer 31 is as close to layer 1 as layer 2 is); each row's preferred chunks
    score above the rest on average."""
    w = W.preferred_chunks(0.06, seed=3)
    layers = list(synth.generate(w))
    assert len(layers) == 32 and layers[0].q.shape == (1, 384, 64) and layers[0].k.shape == (1, 192, 64)
    d12 = np.std(layers[2].q - layers[1].q)
    d31 = np.std(layers[31].q - layers[1].q)
    step = 0.06 / 8
    assert abs(d12 / (step * np.sqrt(2)) - 1) < 0.05 and abs(d31 / d12 - 1) < 0.05
    s = layers[0].q[0] @ layers[0].k[0].T
    top = np.sort(s, axis=1)[:, -12:].mean()
    assert top - s.mean() > 0.3             # preferred chunks stand out (gain 1.0 / sqrt(12) ~ 0.29 + the tail)


def test_preferred_chunks_directions():
    """Table 2 / Figure 2 directions on the persistent-preferred-chunk workload: the rerouted
    fraction rises with drift, relay keeps recall above 0.9999, and fixed-stride-4 reuse loses
    recall as drift grows, staying below relay."""
    stats = [chain_stats(W.preferred_chunks(s, seed=0), with_stride4=True) for s in (0.01, 0.03, 0.06)]
    rho = [x[0] for x in stats]
    assert rho[0] < rho[1] < rho[2]
    for x in stats:
        assert x[1] > 0.9999 and x[3] < x[1]
    assert stats[0][3] > stats[1][3] > stats[2][3]


def test_near_miss_sentinels_carry_recall():
    """Table 3: random sentinels alone lose recall and reroute fewer rows; near-miss
    sentinels recover full recall; adding random ones to them changes nothing here."""
    base = W.Workload("ablation", heads=1, layers=24, n=256, d=64, dtype="f32",
                      drift=(0.003, 0.003), drift_scale="relative", anchors=(0,))
    rnd = chain_stats(base.with_(m=0, r=12))
    near = chain_stats(base.with_(m=24, r=0))
    both = chain_stats(base.with_(m=12, r=12))
    assert rnd[1] < near[1] and near[1] == 1.0
    assert rnd[0] < near[0]
    assert both[0] == near[0] and both[1] == near[1]


def test_pair_fraction_falls_with_chunk_count():
    """Table 4 / Section 5.3: the fixed-width candidate set gets relatively cheaper as
    the number of key chunks grows (checked between 128 and 512 chunks)."""
    p128 = chain_stats(W.scale_sweep(128).with_(layers=16))[2]
    p512 = chain_stats(W.scale_sweep(512).with_(layers=16))[2]
    assert p512 < p128

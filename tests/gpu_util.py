"""Helpers for the GPU parity tests: upload inputs, run the C-ABI path, compare with the oracle.

Comparison rule: route / sentinel / anchor IDs, refresh flags and the compacted row list
must be bit-equal, except rows whose oracle score gap at a decision boundary is below
``tol`` (1e-5 absolute; 0 for integer-valued inputs, whose scores are exact on both sides),
which are excluded and counted.  Scores (alpha, beta, candidate scores) must agree within
``rel`` * (|s_ref| + rms of the row's candidate scores): 1e-5 for fp32 inputs, 1e-3 for bf16.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np

import oracle as O
from long_context_prefill_anchor_amd import rr

GAP_TOL = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upload(x: np.ndarray):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def oracle_cfg(led: rr.Ledger, dtype: str, gamma=0.0, causal=False, seed=0):
    return O.RouteConfig(heads=led.heads, nq=led.nq, nk=led.nk, d=64, k=led.k, m=led.m, r=led.r,
                         gamma=gamma, causal=causal, seed=seed, dtype=dtype, sink=led.sink,
                         recent=led.recent, min_reuse=led.min_reuse, gamma_extra=led.gamma_extra,
                         q_rows=led.q_rows, nq_q=led.nq_q)


def ledger_np(led: rr.Ledger):
    route, sent, anchor = led.get()
    refreshed = led.get_refreshed()
    import torch
    torch.cuda.synchronize()
    return route.cpu().numpy(), sent.cpu().numpy(), anchor.cpu().numpy(), refreshed.cpu().numpy()


def set_ledger(led: rr.Ledger, ol: O.Ledger, last_layer: int):
    import torch
    led.set(torch.from_numpy(ol.route).cuda(), torch.from_numpy(ol.sent).cuda(),
            torch.from_numpy(ol.anchor).cuda(), last_layer)
    led.set_refreshed(torch.from_numpy(np.ascontiguousarray(ol.refreshed)).cuda())


def oracle_scores(cfg: O.RouteConfig, q, k) -> np.ndarray:
    Q, K = O.decode(q, cfg.dtype), O.decode(k, cfg.dtype)
    return np.stack([O.score_rows(O.query_rows(cfg, Q[h]), K[h]) for h in range(cfg.heads)])


def selection_excluded(cfg: O.RouteConfig, S: np.ndarray, tol: float, rows=None) -> np.ndarray:
    """bool [H, nq]: rows whose route / near-miss boundary gap is below tol."""
    ex = np.zeros((cfg.heads, cfg.nq), bool)
    if tol <= 0:
        return ex
    it = rows if rows is not None else [(h, i) for h in range(cfg.heads) for i in range(cfg.nq)]
    for h, i in it:
        ex[h, i] = O.selection_gap(S[h, i], O.n_allowed(i, cfg), cfg.k, cfg.m) < tol
    return ex


@dataclass
class Report:
    rows: int = 0
    excluded: int = 0
    max_score_err: float = 0.0
    notes: list = field(default_factory=list)


def compare_ledgers(gpu, ora: O.Ledger, mask: np.ndarray, what: str):
    """Bit-equality of route / sent / anchor / hysteresis state on rows where mask is True."""
    g_route, g_sent, g_anchor, g_ref = gpu
    for name, g, o in (("route", g_route, ora.route), ("sent", g_sent, ora.sent),
                       ("anchor", g_anchor, ora.anchor), ("refreshed", g_ref, ora.refreshed)):
        gm, om = g[mask], o[mask]
        if not np.array_equal(gm, om):
            bad = np.argwhere(mask)[np.flatnonzero((gm != om).reshape(len(gm), -1).any(axis=1))]
            h, i = bad[0]
            raise AssertionError(f"{what}: {name} differs on {len(bad)} rows, first (h={h}, i={i}): "
                                 f"gpu={g[h, i]} oracle={o[h, i]}")


def check_scores(got, ref, rel, rms, what):
    """|got - ref| <= rel * (|ref| + rms) where the oracle value is finite; where it is NaN
    (no ID) or +-inf (beta of a row without sentinels) the GPU value must be the same
    NaN / infinity.  Returns the largest error over the finite oracle values."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.broadcast_to(np.asarray(rms, np.float64), np.broadcast_shapes(got.shape, ref.shape))
    got, ref = np.broadcast_arrays(got, ref)
    fin = np.isfinite(ref)
    special_ok = (np.isnan(ref) & np.isnan(got)) | (np.isinf(ref) & (got == ref))
    err = np.zeros(got.shape)
    err[fin] = np.abs(got[fin] - ref[fin])
    lim = np.zeros(got.shape)
    lim[fin] = rel * (np.abs(ref[fin]) + rms[fin])
    ok = np.where(fin, np.isfinite(got) & (err <= lim), special_ok)
    if not ok.all():
        idx = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} values out of tolerance, first {idx}: "
                             f"gpu={got[idx]} oracle={ref[idx]}")
    return float(err[fin].max()) if fin.any() else 0.0


def check_compaction(g_rows, g_counts, g_flags, res, mask, what):
    """The GPU's compacted list (Sections 4.1-4.2: ascending h*nq+i of flagged rows) and its
    per-head counts against the oracle's, on rows outside the exclusion mask: the list must be
    strictly ascending, name exactly the rows the oracle flags among the compared rows, and
    each head count must equal the oracle's plus the GPU-minus-oracle flag difference on that
    head's excluded rows."""
    H, nq = res.flags.shape
    g_rows = np.asarray(g_rows, np.int64)
    assert np.all(np.diff(g_rows) > 0), f"{what}: compacted list not strictly ascending"
    assert g_rows.size == 0 or (g_rows[0] >= 0 and g_rows[-1] < H * nq), f"{what}: list entry out of range"
    listed = np.zeros(H * nq, np.uint8)
    listed[g_rows] = 1
    listed = listed.reshape(H, nq)
    if not np.array_equal(listed[mask], res.flags[mask]):
        h, i = np.argwhere(mask & (listed != res.flags))[0]
        raise AssertionError(f"{what}: compacted list differs from the oracle's at row (h={h}, i={i}): "
                             f"gpu lists it {bool(listed[h, i])}, oracle flags it {bool(res.flags[h, i])}")
    ora_rows = set(int(x) for x in res.rows)
    cmp_rows = set(int(x) for x in np.flatnonzero(mask.reshape(-1)))
    assert (set(int(x) for x in g_rows) & cmp_rows) == (ora_rows & cmp_rows), f"{what}: compacted list"
    diff = ((np.asarray(g_flags, np.int64) - res.flags.astype(np.int64)) * (~mask)).sum(axis=1)
    expect = res.head_counts.astype(np.int64) + diff
    if not np.array_equal(np.asarray(g_counts, np.int64), expect):
        h = int(np.flatnonzero(np.asarray(g_counts) != expect)[0])
        raise AssertionError(f"{what}: head count of head {h}: gpu={g_counts[h]} oracle={res.head_counts[h]} "
                             f"(+{diff[h]} from excluded rows)")
    assert np.array_equal(np.asarray(g_counts), listed.sum(axis=1)), f"{what}: head counts vs the list"


def run_anchor(led: rr.Ledger, q, k, layer: int):
    import torch
    led.anchor(upload(q), upload(k), layer)
    torch.cuda.synchronize()
    return ledger_np(led)


def anchor_parity(led, cfg, q, k, layer, tol, rep: Report, rows=None):
    """GPU anchor layer vs oracle on all rows (or the given (h, i) sample)."""
    gpu = run_anchor(led, q, k, layer)
    if rows is None:
        S = oracle_scores(cfg, q, k)
        ora = O.anchor_layer(cfg, q, k, layer)
        mask = ~selection_excluded(cfg, S, tol)
    else:
        S = sampled_score_rows(cfg, q, k, rows)         # {(h, i): row}: no full score matrix
        ora = O.Ledger.empty(cfg)
        for h, i in rows:
            O.rebuild_row(cfg, ora, h, layer, i, S[h, i])
        mask = np.zeros((cfg.heads, cfg.nq), bool)
        for h, i in rows:
            mask[h, i] = True
        mask &= ~selection_excluded(cfg, S, tol, rows)
    total = len(rows) if rows is not None else cfg.heads * cfg.nq
    rep.rows += total
    rep.excluded += total - int(mask.sum())
    compare_ledgers(gpu, ora, mask, f"anchor layer {layer}")
    return gpu, ora


def relay_excluded(cfg, layer, ledger_in, h, i, alpha, beta, tol) -> bool:
    """Relay decision gap below tol, with the row's own guard (a relay-refreshed row past its
    reuse horizon is tested with gamma + gamma_extra; inside the horizon there is no test)."""
    ref = bool(ledger_in.refreshed[h, i])
    if ref and layer - int(ledger_in.anchor[h, i]) <= cfg.min_reuse:
        return False
    guard = float(np.float32(np.float32(cfg.gamma) + np.float32(cfg.gamma_extra))) if ref else cfg.gamma
    return O.relay_gap(alpha, beta, guard) < tol


def relay_parity(led, cfg, q, k, layer, ledger_in: O.Ledger, tol, rel, rep: Report, excluded_in=None,
                 mode="auto"):
    """GPU relay layer (started from ``ledger_in``, launched as ``mode``: auto, fused or
    compacted) vs oracle.  Returns the GPU ledger, the oracle result and the rows excluded from
    here on."""
    import torch
    led.set_relay_mode(mode)
    set_ledger(led, ledger_in, layer - 1)
    out = led.alloc_outputs()
    led.relay(upload(q), upload(k), layer, out)
    torch.cuda.synchronize()
    gpu = ledger_np(led)
    res = O.relay_layer(cfg, q, k, layer, ledger_in)
    H, nq = cfg.heads, cfg.nq
    g_flags = out.flags.cpu().numpy().reshape(H, nq)
    g_alpha = out.alpha.cpu().numpy().reshape(H, nq)
    g_beta = out.beta.cpu().numpy().reshape(H, nq)
    g_cand = out.cand_scores.cpu().numpy().reshape(H, nq, cfg.c)
    n_rows = int(out.n_rows.cpu().numpy()[0])
    g_rows = out.rows.cpu().numpy()[:n_rows]
    g_counts = out.head_counts.cpu().numpy()

    # the compacted list is exactly the GPU's own flagged rows, ascending, with matching counts
    # (and below, on the compared rows, the oracle's list and counts)
    assert np.array_equal(g_rows, np.flatnonzero(g_flags.reshape(-1))), "compacted list"
    assert np.array_equal(g_counts, g_flags.sum(axis=1)), "head counts"

    # scores: alpha, beta, and every candidate score, within tolerance
    rms = np.sqrt(np.nanmean(res.cand_scores.astype(np.float64) ** 2, axis=2))
    e1 = check_scores(g_cand, res.cand_scores, rel, rms[:, :, None], f"layer {layer} candidate scores")
    e2 = check_scores(g_alpha, res.alpha, rel, rms, f"layer {layer} alpha")
    e3 = check_scores(g_beta, res.beta, rel, rms, f"layer {layer} beta")
    rep.max_score_err = max(rep.max_score_err, e1, e2, e3)

    # exclusions: relay decision gap, then (for refreshed rows) the selection gap at this layer
    ex = np.zeros((H, nq), bool) if excluded_in is None else excluded_in.copy()
    if tol > 0:
        for h in range(H):
            for i in range(nq):
                if relay_excluded(cfg, layer, ledger_in, h, i, res.alpha[h, i], res.beta[h, i], tol):
                    ex[h, i] = True
        S = None
        for h, i in np.argwhere(res.flags == 1):
            if S is None:
                S = oracle_scores(cfg, q, k)
            if O.selection_gap(S[h, i], O.n_allowed(i, cfg), cfg.k, cfg.m) < tol:
                ex[h, i] = True
    mask = ~ex
    rep.rows += H * nq
    rep.excluded += int(ex.sum())
    if not np.array_equal(g_flags[mask], res.flags[mask]):
        bad = np.argwhere(mask & (g_flags != res.flags))[0]
        raise AssertionError(f"layer {layer}: flags differ, first {tuple(bad)}: gpu={g_flags[tuple(bad)]} "
                             f"oracle={res.flags[tuple(bad)]} alpha={res.alpha[tuple(bad)]} beta={res.beta[tuple(bad)]}")
    check_compaction(g_rows, g_counts, g_flags, res, mask, f"relay layer {layer}")
    compare_ledgers(gpu, res.ledger, mask, f"relay layer {layer}")
    return gpu, res, ex


def sampled_score_rows(cfg: O.RouteConfig, q, k, rows):
    """Oracle score rows (fp32, Eq. 1) of the given (h, i) pairs only: {(h, i): [nk]}."""
    Q, K = O.decode(q, cfg.dtype), O.decode(k, cfg.dtype)
    out = {}
    by_head = {}
    for h, i in rows:
        by_head.setdefault(h, []).append(i)
    for h, ii in by_head.items():
        S = O.score_rows(O.query_rows(cfg, Q[h])[np.asarray(ii)], K[h])
        for r, i in enumerate(ii):
            out[(h, i)] = S[r]
    return out


def relay_parity_sampled(led, cfg, q0, k0, q1, k1, rows, tol, rel, rep: Report, mode="auto"):
    """GPU anchor at layer 0 and relay at layer 1 over every row; the oracle on the sampled
    (h, i) pairs only: its own anchor ledger entries for those rows, then its relay of them
    (rows are independent, Section 3.2).  Compared on the sampled rows outside the exclusions:
    the anchor ledger, then flags, alpha, beta, candidate scores, the rerouted ledger rows and
    the compacted list; on every row: the list equals the GPU's own flags, ascending, and the
    head counts match it.  Returns (number of compared rows, flagged among them)."""
    import torch
    H, nq = cfg.heads, cfg.nq
    rows = sorted(set((int(h), int(i)) for h, i in rows))
    gpu0 = run_anchor(led, q0, k0, 0)
    S0 = sampled_score_rows(cfg, q0, k0, rows)
    ora0 = O.Ledger.empty(cfg)
    mask = np.zeros((H, nq), bool)
    for h, i in rows:
        O.rebuild_row(cfg, ora0, h, 0, i, S0[(h, i)])
        mask[h, i] = O.selection_gap(S0[(h, i)], O.n_allowed(i, cfg), cfg.k, cfg.m) >= tol
    compare_ledgers(gpu0, ora0, mask, "sampled anchor layer 0")

    out = led.alloc_outputs()
    led.set_relay_mode(mode)
    led.relay(upload(q1), upload(k1), 1, out)
    torch.cuda.synchronize()
    gpu1 = ledger_np(led)
    g_flags = out.flags.cpu().numpy().reshape(H, nq)
    g_alpha = out.alpha.cpu().numpy().reshape(H, nq)
    g_beta = out.beta.cpu().numpy().reshape(H, nq)
    g_cand = out.cand_scores.cpu().numpy().reshape(H, nq, cfg.c)
    n_rows = int(out.n_rows.cpu().numpy()[0])
    g_rows = out.rows.cpu().numpy()[:n_rows]
    g_counts = out.head_counts.cpu().numpy()
    # every row: the list is the GPU's own flagged rows, ascending; counts per head match it
    assert np.array_equal(g_rows, np.flatnonzero(g_flags.reshape(-1))), "compacted list vs flags"
    assert np.array_equal(g_counts, g_flags.sum(axis=1)), "head counts vs flags"

    res = O.relay_layer_rows(cfg, q1, k1, 1, ora0, rows)
    S1 = None
    for h, i in rows:
        if not mask[h, i]:
            continue
        if relay_excluded(cfg, 1, ora0, h, i, res.alpha[h, i], res.beta[h, i], tol):
            mask[h, i] = False
        elif res.flags[h, i]:
            if S1 is None:
                S1 = sampled_score_rows(cfg, q1, k1, [(a, b) for a, b in rows if res.flags[a, b]])
            if O.selection_gap(S1[(h, i)], O.n_allowed(i, cfg), cfg.k, cfg.m) < tol:
                mask[h, i] = False
    rep.rows += len(rows)
    rep.excluded += len(rows) - int(mask.sum())
    rms = np.sqrt(np.nanmean(res.cand_scores[mask].astype(np.float64) ** 2, axis=1))
    e1 = check_scores(g_cand[mask], res.cand_scores[mask], rel, rms[:, None], "sampled candidate scores")
    e2 = check_scores(g_alpha[mask], res.alpha[mask], rel, rms, "sampled alpha")
    e3 = check_scores(g_beta[mask], res.beta[mask], rel, rms, "sampled beta")
    rep.max_score_err = max(rep.max_score_err, e1, e2, e3)
    if not np.array_equal(g_flags[mask], res.flags[mask]):
        bad = np.argwhere(mask & (g_flags != res.flags))[0]
        raise AssertionError(f"sampled relay: flags differ at {tuple(bad)}: gpu={g_flags[tuple(bad)]} "
                             f"oracle={res.flags[tuple(bad)]}")
    listed = np.zeros(H * nq, np.uint8)
    listed[g_rows] = 1
    assert np.array_equal(listed.reshape(H, nq)[mask], res.flags[mask]), "compacted list vs oracle flags"
    compare_ledgers(gpu1, res.ledger, mask, "sampled relay layer 1")
    return int(mask.sum()), int(res.flags[mask].sum())

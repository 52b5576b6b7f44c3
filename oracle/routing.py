"""RouteRelay routing oracle: a plain, slow CPU statement of what the routing pass computes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "RouteRelay: Event-Triggered Cross-Layer Route Reuse for Efficient
Dynamic Sparse Attention" (arXiv 2609.07306).  Each function names the part of
that page it follows.  Where the page leaves a step open, the reading taken is
stated in the function's docstring.

Numbers: the page's experiments are FP32 (Section 5, Table 1), so every score
that decides an integer result (a route ID, a sentinel, a refresh flag) is an
fp32 value here: the dot product of the fp32 or bf16 inputs is evaluated in
float64 (exactly, for bf16 inputs) and rounded once to fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterable, List, Optional, Sequence

import numpy as np

from .philox import philox4x32_10

SAMPLER_DRAW_CAP = 65536


@dataclass(frozen=True)
class RouteConfig:
    heads: int
    nq: int
    nk: int
    d: int
    k: int = 12
    m: int = 12
    r: int = 8
    gamma: float = 0.0
    causal: bool = False
    seed: int = 0
    dtype: str = "f32"          # "f32" or "bf16": encoding of the Q/K arrays handed in
    sink: int = 0               # mandatory sink sentinels: chunks 0 .. sink-1
    recent: int = 0             # mandatory recent sentinels: the row's last `recent` allowed chunks
    min_reuse: int = 0          # hysteresis: layers a refreshed row is reused untested
    gamma_extra: float = 0.0    # hysteresis: extra guard of a refreshed row until it passes once
    # width bucket (Section 4.4): ledger row r holds query row q_rows[r] of a Q with nq_q rows
    # per head; None = every query row, in order
    q_rows: Optional[tuple] = None
    nq_q: int = 0

    def query_row(self, r: int) -> int:
        return r if self.q_rows is None else int(self.q_rows[r])

    @property
    def mand(self) -> int:
        return self.sink + self.recent

    @property
    def c(self) -> int:
        return self.k + self.m + self.mand + self.r


# ----------------------------------------------------------------------------- inputs

def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Chunk representations as float64.  bf16 arrays arrive as raw uint16 bits:
    a bf16 value is the top half of the fp32 with the same bits."""
    if dtype == "bf16":
        wide = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- Eq. 1, Eq. 2

def score_rows(q_rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Routing scores S = Q K^T (Section 2.1, Eq. 1): raw dot products, no 1/sqrt(d)
    (that factor belongs to the attention of Eq. 3, not to routing).
    ``q_rows`` [a, d] and ``keys`` [b, d] are float64; returns fp32 [a, b]."""
    return (q_rows @ keys.T).astype(np.float32)


def n_allowed(i: int, cfg: RouteConfig) -> int:
    """Key chunks the query chunk of ledger row i may route to: all nk, or 0..q under the
    causal chunk mask, q being the row's query chunk (the router's own masking,
    Section 4.3)."""
    return cfg.query_row(i) + 1 if cfg.causal else cfg.nk


def query_rows(cfg: RouteConfig, Qh: np.ndarray) -> np.ndarray:
    """One head's query representations of the ledger's rows, in ledger order: a width
    bucket (Section 4.4, "ledgers are bucketed by route width") holds a subset of the
    query rows; its ledger row r is query row q_rows[r]."""
    return Qh if cfg.q_rows is None else Qh[np.asarray(cfg.q_rows, dtype=np.int64)]


def preference_order(s_row: np.ndarray, n: int) -> np.ndarray:
    """Chunks 0..n-1 ordered best first: higher score first, equal scores by lower
    chunk index (the page is silent on ties; lower index wins).  -0.0 and +0.0 are
    equal scores."""
    idx = np.arange(n)
    neg = -(s_row[:n].astype(np.float64))
    return idx[np.lexsort((idx, neg))]


def select(s_row: np.ndarray, n: int, k: int, m: int):
    """Top-k route (Eq. 2) and near-miss sentinels, the m best chunks just below the
    cutoff (Section 3.1, item 1).  Rows with fewer than k + m allowed chunks keep
    what there is."""
    order = preference_order(s_row, n)
    ki = min(k, n)
    mi = min(m, n - ki)
    return order[:ki], order[ki:ki + mi]


# ----------------------------------------------------------------------------- mandatory sentinels

def mandatory_sentinels(n: int, sink: int, recent: int, covered: Sequence[int]) -> np.ndarray:
    """Mandatory global candidates (Section 3.1, item 3), ascending.

    Reading: the sink chunks are the first ``sink`` chunks 0 .. sink-1 and the recent
    chunks the row's last ``recent`` allowed chunks n-recent .. n-1 (the query chunk and
    the ones just before it under the causal mask); both are cut to the allowed range.
    A chunk that is already in the route or the near-miss set is not repeated here: as a
    sentinel it would sit on both sides of Eq. 8 (beta >= its score >= alpha for a route
    chunk), so the row could never be reused.
    """
    wanted = set(range(min(sink, n))) | set(range(max(0, n - recent), n))
    wanted -= set(int(j) for j in covered)
    return np.asarray(sorted(wanted), dtype=np.int64)


# ----------------------------------------------------------------------------- random sentinels

def random_sentinels(seed: int, h: int, layer: int, i: int, n: int,
                     excluded: Sequence[int], r: int) -> np.ndarray:
    """r chunks drawn uniformly without replacement from the omitted chunks
    (Section 3.1, item 2; the residual pool of Section 3.4, Eq. 10).

    Reading: "omitted" = allowed chunks outside route, near-miss set and mandatory
    sentinels (``excluded`` holds all three).  The page
    names no sampler; this one is deterministic so results can be compared:
      * pool size N <= r: take the whole pool;
      * else for t = 0, 1, 2, ...: u_t = word (t mod 4) of
        Philox4x32-10(counter = (t div 4, i, layer, h), key = (seed lo32, seed hi32)),
        j_t = floor(u_t * n / 2^32); j_t is accepted if it is still in the pool,
        and leaves the pool once accepted; stop at r accepted;
      * after SAMPLER_DRAW_CAP draws, fill up with the lowest-index pool members.
    """
    if r <= 0:
        return np.zeros(0, dtype=np.int64)
    in_pool = np.ones(n, dtype=bool)
    in_pool[np.asarray(excluded, dtype=np.int64)] = False
    if int(in_pool.sum()) <= r:
        return np.flatnonzero(in_pool)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    taken: List[int] = []
    words = None
    for t in range(SAMPLER_DRAW_CAP):
        if t % 4 == 0:
            words = philox4x32_10((t // 4, i, layer, h), key)
        j = (words[t % 4] * n) >> 32
        if in_pool[j]:
            in_pool[j] = False
            taken.append(j)
            if len(taken) == r:
                break
    if len(taken) < r:
        rest = np.flatnonzero(in_pool)[: r - len(taken)]
        taken.extend(int(j) for j in rest)
    return np.sort(np.asarray(taken, dtype=np.int64))


# ----------------------------------------------------------------------------- the ledger

def _pad(ids: np.ndarray, width: int) -> np.ndarray:
    out = np.full(width, -1, dtype=np.int32)
    ids = np.sort(np.asarray(ids, dtype=np.int64))
    out[: len(ids)] = ids
    return out


@dataclass
class Ledger:
    """Route ledger (Section 3.1, Eq. 4; Section 4.1): per query row the route [k],
    the sentinels [m + sink + recent + r] and the layer a of its last full routing.
    Every segment is ascending with -1 padding; sentinels hold the near-miss segment
    (width m), the mandatory segment (width sink + recent), then the random segment
    (width r)."""
    route: np.ndarray    # int32 [H, nq, k]
    sent: np.ndarray     # int32 [H, nq, c - k]
    anchor: np.ndarray   # int32 [H, nq]
    # uint8 [H, nq] hysteresis state: 1 when the row was last routed by a relay-layer
    # refresh, 0 when by an anchor layer; with hysteresis on, also 0 once the refreshed row
    # has passed a test under the post-refresh guard
    refreshed: np.ndarray = None

    def __post_init__(self):
        if self.refreshed is None:
            self.refreshed = np.zeros(self.anchor.shape, np.uint8)

    @staticmethod
    def empty(cfg: RouteConfig) -> "Ledger":
        return Ledger(np.full((cfg.heads, cfg.nq, cfg.k), -1, np.int32),
                      np.full((cfg.heads, cfg.nq, cfg.c - cfg.k), -1, np.int32),
                      np.full((cfg.heads, cfg.nq), -1, np.int32))

    def copy(self) -> "Ledger":
        return Ledger(self.route.copy(), self.sent.copy(), self.anchor.copy(), self.refreshed.copy())

    def candidates(self, h: int, i: int) -> np.ndarray:
        """Candidate set A_i = route U sentinels (Section 3.2, Eq. 5), padding dropped."""
        ids = np.concatenate([self.route[h, i], self.sent[h, i]])
        return ids[ids >= 0]


def rebuild_row(cfg: RouteConfig, ledger: Ledger, h: int, layer: int, i: int,
                s_row: np.ndarray) -> None:
    """Full routing of one row at ``layer``: new route, near-miss, mandatory and
    random sentinels, anchor layer set to ``layer`` (Section 3.2: a failing row
    computes all n_k scores, replaces its route and rebuilds its sentinels)."""
    n = n_allowed(i, cfg)
    route, near = select(s_row, n, cfg.k, cfg.m)
    mand = mandatory_sentinels(n, cfg.sink, cfg.recent, np.concatenate([route, near]))
    # the sampler's counter names the query row, so a row draws the same sentinels in any bucket
    rnd = random_sentinels(cfg.seed, h, layer, cfg.query_row(i), n,
                           np.concatenate([route, near, mand]), cfg.r)
    ledger.route[h, i] = _pad(route, cfg.k)
    ledger.sent[h, i, : cfg.m] = _pad(near, cfg.m)
    ledger.sent[h, i, cfg.m: cfg.m + cfg.mand] = _pad(mand, cfg.mand)
    ledger.sent[h, i, cfg.m + cfg.mand:] = _pad(rnd, cfg.r)
    ledger.anchor[h, i] = layer
    ledger.refreshed[h, i] = 0


# ----------------------------------------------------------------------------- anchor layer

def anchor_layer(cfg: RouteConfig, q: np.ndarray, k: np.ndarray, layer: int) -> Ledger:
    """Anchor layer (Section 4.1): the state is built from a complete score matrix;
    every row is routed in full."""
    Q, K = decode(q, cfg.dtype), decode(k, cfg.dtype)
    led = Ledger.empty(cfg)
    for h in range(cfg.heads):
        S = score_rows(query_rows(cfg, Q[h]), K[h])
        for i in range(cfg.nq):
            rebuild_row(cfg, led, h, layer, i, S[i])
    return led


# ----------------------------------------------------------------------------- relay layer

@dataclass
class RelayResult:
    ledger: Ledger            # ledger after the layer (refreshed rows rebuilt)
    flags: np.ndarray         # uint8 [H, nq]: 1 = row failed Eq. 8 and was rerouted
    alpha: np.ndarray         # fp32 [H, nq], Eq. 6
    beta: np.ndarray          # fp32 [H, nq], Eq. 7 (-inf when the row has no sentinels)
    cand_scores: np.ndarray   # fp32 [H, nq, c]: scores of the ledger's IDs in ledger order (NaN = padding)
    rows: np.ndarray          # int32: ascending h * nq + i of flagged rows (the compacted list)
    head_counts: np.ndarray   # int32 [H]


def relay_decision(cfg: RouteConfig, layer: int, anchor: int, refreshed: int,
                   alpha: np.float32, beta: np.float32) -> tuple[bool, int]:
    """Eq. 8 with the hysteresis of Section 3.2 (after Eq. 8).  Returns (refresh the row?,
    the row's hysteresis state if it is reused).

    Reading: a row refreshed at a relay layer a is reused without a test at layers
    a+1 .. a+min_reuse (its "minimum reuse horizon"); after that it is tested with the
    larger guard gamma + gamma_extra until the first layer at which it passes (its margin
    has "recovered"), and from then on with gamma.  Rows routed at an anchor layer use gamma
    throughout.  min_reuse = 0 and gamma_extra = 0 give plain Eq. 8; the state is then never
    consulted and a reused row keeps it (it only records how the row was last routed).
    beta + guard is rounded to fp32 before the strict comparison."""
    if cfg.min_reuse == 0 and cfg.gamma_extra == 0:
        return not (alpha > np.float32(beta + np.float32(cfg.gamma))), refreshed
    if refreshed and layer - anchor <= cfg.min_reuse:
        return False, 1
    guard = np.float32(np.float32(cfg.gamma) + np.float32(cfg.gamma_extra)) if refreshed \
        else np.float32(cfg.gamma)
    reuse = alpha > np.float32(beta + guard)
    return (not reuse), 0


def _relay_row(cfg: RouteConfig, qi: np.ndarray, Kh: np.ndarray, layer: int,
               ledger: Ledger, out: Ledger, h: int, i: int):
    """One row of an intermediate layer: score its candidate set A = R U C at this layer
    (Eq. 5); alpha = min over R (Eq. 6), beta = max over C (Eq. 7), -inf when C is empty;
    reuse iff alpha > beta + gamma (Eq. 8, with the hysteresis of ``relay_decision``).
    A failing row is routed in full at this layer into ``out`` and marked refreshed.
    Returns (flag, alpha, beta, candidate scores in ledger order with NaN for padding)."""
    ids = np.concatenate([ledger.route[h, i], ledger.sent[h, i]])
    valid = ids >= 0
    s = score_rows(qi[None, :], Kh[ids[valid]])[0]
    cand = np.full(cfg.c, np.nan, np.float32)
    cand[valid] = s
    n_route = int(valid[: cfg.k].sum())
    s_route, s_sent = s[:n_route], s[n_route:]
    a = np.float32(s_route.min())
    b = np.float32(s_sent.max()) if s_sent.size else np.float32(-np.inf)
    refresh, state = relay_decision(cfg, layer, int(ledger.anchor[h, i]), int(ledger.refreshed[h, i]), a, b)
    if refresh:
        rebuild_row(cfg, out, h, layer, i, score_rows(qi[None, :], Kh)[0])
        out.refreshed[h, i] = 1
    else:
        out.refreshed[h, i] = state
    return (1 if refresh else 0), a, b, cand


def relay_layer(cfg: RouteConfig, q: np.ndarray, k: np.ndarray, layer: int,
                ledger: Ledger) -> RelayResult:
    """Intermediate layer (Sections 3.2, 4.1, 4.2): every row goes through ``_relay_row``.
    Flagged rows are listed in ascending flattened order h * nq + i (the compaction of
    Section 4.1/4.2)."""
    return relay_layer_rows(cfg, q, k, layer, ledger,
                            [(h, i) for h in range(cfg.heads) for i in range(cfg.nq)])


def relay_layer_rows(cfg: RouteConfig, q: np.ndarray, k: np.ndarray, layer: int,
                     ledger: Ledger, rows) -> RelayResult:
    """The intermediate layer of ``relay_layer`` restricted to the (h, i) pairs in ``rows``
    (rows are independent, Section 3.2): flags, alpha, beta, candidate scores and ledger
    entries are those of ``relay_layer`` at those rows; every other row keeps its input
    ledger entry, flag 0, alpha = beta = 0 and NaN scores.  ``rows`` lists and head counts
    cover the given rows only."""
    Q, K = decode(q, cfg.dtype), decode(k, cfg.dtype)
    out = ledger.copy()
    H, nq, c = cfg.heads, cfg.nq, cfg.c
    flags = np.zeros((H, nq), np.uint8)
    alpha = np.zeros((H, nq), np.float32)
    beta = np.zeros((H, nq), np.float32)
    cand = np.full((H, nq, c), np.nan, np.float32)
    Qrows = {}
    for h, i in rows:
        if h not in Qrows:
            Qrows[h] = query_rows(cfg, Q[h])
        flags[h, i], alpha[h, i], beta[h, i], cand[h, i] = _relay_row(cfg, Qrows[h][i], K[h], layer,
                                                                      ledger, out, h, i)
    flat = np.flatnonzero(flags.reshape(-1)).astype(np.int32)
    return RelayResult(out, flags, alpha, beta, cand, flat, flags.sum(axis=1).astype(np.int32))


# ----------------------------------------------------------------------------- full routing every layer

def exact_routes(cfg: RouteConfig, q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Exact top-k per row at one layer ("route every layer", Section 5.1): int32
    [H, nq, k], ascending, -1 padded."""
    Q, K = decode(q, cfg.dtype), decode(k, cfg.dtype)
    out = np.full((cfg.heads, cfg.nq, cfg.k), -1, np.int32)
    for h in range(cfg.heads):
        S = score_rows(query_rows(cfg, Q[h]), K[h])
        for i in range(cfg.nq):
            route, _ = select(S[i], n_allowed(i, cfg), cfg.k, 0)
            out[h, i] = _pad(route, cfg.k)
    return out


# ----------------------------------------------------------------------------- the chain

@dataclass
class LayerRecord:
    layer: int
    kind: str                         # "anchor" or "relay"
    used_route: np.ndarray            # int32 [H, nq, k]: route handed to token expansion
    exact_route: Optional[np.ndarray]  # int32 [H, nq, k] when requested
    flags: Optional[np.ndarray]       # relay layers only
    cand_count: Optional[np.ndarray]  # int32 [H, nq]: candidates scored per row (relay layers)
    rows: Optional[np.ndarray]
    ledger_in: Optional[Ledger]       # ledger entering the layer (relay layers)
    ledger_out: Ledger


def run_chain(cfg: RouteConfig, layers: Iterable, anchors: Sequence[int],
              with_exact: bool = True, keep_ledgers: bool = False) -> List[LayerRecord]:
    """Layer-by-layer RouteRelay (Section 3.2 "Forced anchors", Section 4.1): layer 0
    and every layer in ``anchors`` route in full; every other layer relays.
    ``layers`` yields objects with ``.layer``, ``.q`` and ``.k``."""
    recs: List[LayerRecord] = []
    led: Optional[Ledger] = None
    anchor_set = set(anchors) | {0}
    for li in layers:
        ex = exact_routes(cfg, li.q, li.k) if with_exact else None
        if led is None or li.layer in anchor_set:
            led = anchor_layer(cfg, li.q, li.k, li.layer)
            recs.append(LayerRecord(li.layer, "anchor", led.route.copy(), ex, None, None, None,
                                    None, led.copy() if keep_ledgers else led))
        else:
            cnt = (led.route >= 0).sum(axis=2) + (led.sent >= 0).sum(axis=2)
            res = relay_layer(cfg, li.q, li.k, li.layer, led)
            recs.append(LayerRecord(li.layer, "relay", res.ledger.route.copy(), ex, res.flags,
                                    cnt.astype(np.int32), res.rows,
                                    led if keep_ledgers else None, res.ledger))
            led = res.ledger
    return recs


# ----------------------------------------------------------------------------- metrics (Section 5)

def route_recall(used: np.ndarray, exact: np.ndarray) -> float:
    """Top-k route recall (Table 2 caption): mean over rows of
    |used route intersect exact top-k| / |exact top-k|."""
    tot, num = 0.0, 0
    flat_u = used.reshape(-1, used.shape[-1])
    flat_e = exact.reshape(-1, exact.shape[-1])
    for u, e in zip(flat_u, flat_e):
        e = e[e >= 0]
        u = u[u >= 0]
        tot += len(np.intersect1d(u, e)) / len(e)
        num += 1
    return tot / num


def reroute_fraction(kinds: Sequence[str], flags: Sequence[Optional[np.ndarray]], rows_per_layer: int) -> float:
    """Fraction of (layer, row) pairs that run full routing; every row of an anchor
    layer counts (a fixed stride of 4 over 32 layers gives 25.0%, Table 2)."""
    full = 0
    for kind, f in zip(kinds, flags):
        full += rows_per_layer if kind == "anchor" else int(np.asarray(f).sum())
    return full / (rows_per_layer * len(kinds))


def pair_counts(kinds: Sequence[str], heads: int, n_row: np.ndarray,
                flags: Sequence[Optional[np.ndarray]],
                cand_counts: Sequence[Optional[np.ndarray]]) -> tuple[int, int]:
    """Evaluated query-key score pairs and the full-routing total (Section 3.5,
    Eq. 11-12; Table 3).  An anchor layer scores every allowed pair; a relay layer
    scores each row's candidates, plus every allowed pair of a refreshed row.
    ``n_row`` [nq] is the allowed count per row; ``flags``/``cand_counts`` are
    [H, nq] arrays for relay layers (None for anchors)."""
    per_layer_full = heads * int(np.asarray(n_row).sum())
    evaluated = 0
    for kind, f, cc in zip(kinds, flags, cand_counts):
        if kind == "anchor":
            evaluated += per_layer_full
        else:
            f = np.asarray(f, dtype=np.int64).reshape(heads, -1)
            cc = np.asarray(cc, dtype=np.int64).reshape(heads, -1)
            evaluated += int(cc.sum()) + int((f * np.asarray(n_row, dtype=np.int64)[None, :]).sum())
    return evaluated, per_layer_full * len(kinds)


def ledger_bytes(nq: int, c: int, bytes_per_id: int = 4) -> int:
    """Index storage of one ledger (Section 4.4): nq rows of c IDs."""
    return nq * c * bytes_per_id


# ----------------------------------------------------------------------------- exclusion gaps

def selection_gap(s_row: np.ndarray, n: int, k: int, m: int) -> float:
    """Smallest score gap at the decision boundaries of ``select``: between the
    route's last member and the first near-miss, and between the last near-miss
    and the best omitted chunk (only boundaries that exist).  +inf if none."""
    order = preference_order(s_row, n)
    s = s_row[order].astype(np.float64)
    ki = min(k, n)
    mi = min(m, n - ki)
    gaps = []
    if ki < n:
        gaps.append(s[ki - 1] - s[ki])
    if ki + mi < n and mi > 0:
        gaps.append(s[ki + mi - 1] - s[ki + mi])
    return min(gaps) if gaps else np.inf


def relay_gap(alpha: float, beta: float, gamma: float) -> float:
    """Distance of the Eq. 8 decision from its threshold, |alpha - beta - gamma|."""
    if np.isneginf(beta):
        return np.inf
    return abs(float(alpha) - float(beta) - float(gamma))

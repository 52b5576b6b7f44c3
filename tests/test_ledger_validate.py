"""rr_ledger_validate (and rr_ledger_set from host memory): ledger tensors made by the oracle's
anchor and relay layers pass the host check (Section 4.1's three tensors; Section 3.1's
segments), and each way of breaking a rule is refused with the offending row named.  No GPU:
the check runs on the host."""
import numpy as np
import pytest

import oracle as O
from long_context_prefill_anchor_amd import rr, synth

CASES = [
    # name, heads, nq, nk, k, m, r, sink, recent, causal, q_rows
    ("plain", 2, 40, 64, 12, 12, 8, 0, 0, False, None),
    ("causal_short_rows", 1, 48, 48, 12, 12, 8, 0, 0, True, None),
    ("mandatory", 2, 36, 50, 6, 4, 5, 2, 2, False, None),
    ("mandatory_causal", 1, 40, 40, 4, 4, 3, 1, 2, True, None),
    ("comparator", 2, 30, 64, 12, 0, 0, 0, 0, False, None),
    ("tiny_pool", 1, 20, 10, 4, 2, 6, 1, 1, False, None),
    ("bucket_causal", 1, 25, 60, 6, 6, 4, 0, 0, True, tuple(range(3, 60, 2))[:25]),
]


def chain_ledger(case):
    name, H, nq, nk, k, m, r, sink, recent, causal, q_rows = case
    nq_q = 60 if q_rows is not None else nq
    cfg = O.RouteConfig(heads=H, nq=nq, nk=nk, d=64, k=k, m=m, r=r, causal=causal, seed=5, sink=sink,
                        recent=recent, q_rows=q_rows, nq_q=nq_q if q_rows is not None else 0)
    q, kk = synth.gaussian_inputs(H, nq_q, nk, 64, seed=3)
    led = O.anchor_layer(cfg, q, kk, 0)
    q1 = synth.perturb(q, 0.05, seed=4)
    k1 = synth.perturb(kk, 0.05, seed=5)
    res = O.relay_layer(cfg, q1, k1, 1, led)
    c = rr.make_config(H, nq, nk, 64, k, m, r, 0.0, causal, "f32", 5, sink, recent)
    return c, res.ledger, q_rows, nq_q


def validate(c, route, sent, anchor, last, q_rows, nq_q):
    rr.rr_ledger_validate(c, route, sent, anchor, last, q_rows, nq_q)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_oracle_ledgers_pass(case):
    c, led, q_rows, nq_q = chain_ledger(case)
    validate(c, led.route, led.sent, led.anchor, 1, q_rows, nq_q)


def corrupt(case, what):
    c, led, q_rows, nq_q = chain_ledger(case)
    route, sent, anchor = led.route.copy(), led.sent.copy(), led.anchor.copy()
    what(route, sent, anchor)
    with pytest.raises(rr.RRError) as e:
        validate(c, route, sent, anchor, 1, q_rows, nq_q)
    assert e.value.status == rr.RR_EINVAL
    return str(e.value)


def test_repeated_chunk_is_refused():
    def f(route, sent, anchor):
        sent[0, 3, 0] = route[0, 3, 0]            # a near-miss equal to a route chunk
        sent[0, 3, :12] = np.sort(sent[0, 3, :12])
    msg = corrupt(CASES[0], f)
    assert "row 3" in msg and ("twice" in msg or "ascending" in msg)


def test_out_of_range_and_causal_violation_are_refused():
    msg = corrupt(CASES[0], lambda r, s, a: r.__setitem__((1, 5, 11), 64))
    assert "head 1 row 5" in msg and "outside" in msg

    def causal_violation(route, sent, anchor):
        route[0, 20, -1] = 21                      # row 20 may use chunks 0 .. 20 only
    msg = corrupt(CASES[1], causal_violation)
    assert "row 20" in msg and "outside the allowed chunks [0, 21)" in msg


def test_order_padding_and_counts_are_refused():
    def unsorted(route, sent, anchor):
        route[0, 2, [0, 1]] = route[0, 2, [1, 0]]
    assert "not ascending" in corrupt(CASES[0], unsorted)

    def gap(route, sent, anchor):
        x = route[0, 7].copy()
        route[0, 7, 0] = -1                        # padding before IDs
        route[0, 7, 1:] = x[1:]
    assert "after -1 padding" in corrupt(CASES[0], gap)

    def short_route(route, sent, anchor):
        route[1, 0, -1] = -1                       # 11 route IDs where the row holds 12
    assert "route" in corrupt(CASES[0], short_route)

    def anchor_late(route, sent, anchor):
        anchor[0, 0] = 2                           # past last_layer = 1
    assert "anchor layer 2" in corrupt(CASES[0], anchor_late)


def test_mandatory_rules_are_refused():
    def not_mandatory(route, sent, anchor):
        # put a middle chunk (neither sink nor recent, not already used) into the mandatory segment
        m0 = 4                                     # sentinel layout: near-miss (4), mandatory (4), random (5)
        used = set(route[0, 0].tolist()) | set(sent[0, 0].tolist())
        j = next(x for x in range(5, 40) if x not in used)
        seg = sent[0, 0, m0:m0 + 4]
        ids = sorted([v for v in seg.tolist() if v >= 0][:-1] + [j]) if (seg >= 0).any() else [j]
        sent[0, 0, m0:m0 + 4] = ids + [-1] * (4 - len(ids))
    msg = corrupt(CASES[2], not_mandatory)
    assert "neither a sink nor a recent chunk" in msg


def test_bucket_rows_follow_their_query_rows():
    """A bucket row's causal limit is its query row's: an ID allowed for ledger row r but not
    for its query row is refused."""
    case = CASES[6]
    c, led, q_rows, nq_q = chain_ledger(case)
    row = 0                                        # query row 3: chunks 0 .. 3
    assert q_rows[row] == 3
    route = led.route.copy()
    ids = route[0, row]
    assert (ids[:4] >= 0).all() and (ids[4:] == -1).all()
    with pytest.raises(rr.RRError, match="head 0 row 0"):
        bad = route.copy()
        bad[0, row, 3] = 5
        validate(c, bad, led.sent, led.anchor, 1, q_rows, nq_q)


def test_null_and_config_errors():
    c = rr.make_config(1, 4, 8, 64, 2, 0, 0)
    z = np.zeros((1, 4, 2), np.int32)
    with pytest.raises(rr.RRError, match="required"):
        rr.rr_ledger_validate(c, None, None, np.zeros((1, 4), np.int32), 0)
    with pytest.raises(rr.RRError, match="k >= 1"):
        rr.rr_ledger_validate(rr.make_config(1, 4, 8, 64, 0, 0, 0), z, None, np.zeros((1, 4), np.int32), 0)

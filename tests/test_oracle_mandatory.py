"""Pins for the oracle's mandatory sink / recent sentinels (Section 3.1, item 3).

The expected ledgers below are worked out by hand from the scores written in each test, not
computed by the oracle."""
import numpy as np
import pytest

import oracle as O
from long_context_prefill_anchor_amd import synth

# Scores of chunks 0..9 for one query row.  Best first: 1, 3, 5, 7, 8, 9, 2, 4, 0, 6.
HAND_SCORES = [0.1, 0.9, 0.3, 0.8, 0.2, 0.7, 0.0, 0.6, 0.5, 0.4]


def unit_key_inputs(scores, d=16):
    """Q, K with K = the first n unit vectors, so s_0j = scores[j] exactly as fp32."""
    n = len(scores)
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, :n] = scores
    k = np.eye(d, dtype=np.float32)[:n][None]
    return q, k


def test_hand_worked_row():
    """k = 2, m = 2, sink = 2, recent = 2, r = 4 on 10 chunks:
    route {1, 3}; near-miss {5, 7}; sink {0, 1} and recent {8, 9} minus the covered 1 give
    mandatory {0, 8, 9}; the random pool is what is left, {2, 4, 6} (3 <= r: all taken)."""
    q, k = unit_key_inputs(HAND_SCORES)
    cfg = O.RouteConfig(heads=1, nq=1, nk=10, d=16, k=2, m=2, r=4, sink=2, recent=2)
    assert cfg.c == 12
    led = O.anchor_layer(cfg, q, k, 0)
    assert led.route[0, 0].tolist() == [1, 3]
    assert led.sent[0, 0].tolist() == [5, 7, 0, 8, 9, -1, 2, 4, 6, -1]
    assert led.anchor[0, 0] == 0


def test_hand_worked_row_no_overlap():
    """sink = 1, recent = 3: {0} and {7, 8, 9}; 7 is a near-miss, so mandatory = {0, 8, 9};
    random pool {2, 4, 6}, r = 2 draws two of them (which two is the sampler's business)."""
    q, k = unit_key_inputs(HAND_SCORES)
    cfg = O.RouteConfig(heads=1, nq=1, nk=10, d=16, k=2, m=2, r=2, sink=1, recent=3, seed=5)
    led = O.anchor_layer(cfg, q, k, 3)
    sent = led.sent[0, 0].tolist()
    assert sent[:2] == [5, 7]
    assert sent[2:6] == [0, 8, 9, -1]
    rnd = sent[6:]
    assert len(set(rnd)) == 2 and set(rnd) <= {2, 4, 6} and rnd == sorted(rnd)


def test_causal_short_rows_have_nothing_left():
    """Causal row i allows chunks 0..i.  Row 2 with k = 2, m = 2: route = best two of
    {0, 1, 2}, near-miss the third; sink and recent chunks are all covered, so the mandatory
    and random segments are empty."""
    q = np.zeros((1, 3, 16), np.float32)
    q[0, 2, :3] = [0.5, 0.25, 0.75]
    k = np.eye(16, dtype=np.float32)[:3][None]
    cfg = O.RouteConfig(heads=1, nq=3, nk=3, d=16, k=2, m=2, r=2, sink=1, recent=1, causal=True)
    led = O.anchor_layer(cfg, q, k, 0)
    assert led.route[0, 2].tolist() == [0, 2]
    assert led.sent[0, 2].tolist() == [1, -1, -1, -1, -1, -1]
    # row 0: one allowed chunk, the route; everything else padding
    assert led.route[0, 0].tolist() == [0, -1]
    assert led.sent[0, 0].tolist() == [-1] * 6


def test_sink_sentinel_triggers_refresh():
    """The sink sentinel's job: at layer 1 chunk 0 (a low scorer at the anchor) becomes the
    best chunk.  With r = 0 and near-miss chunks that stay below the route, only a sink
    sentinel sees it: beta = s_0 > alpha flags the row and the refresh routes to chunk 0."""
    s0 = [0.0, 0.9, 0.8, 0.5, 0.4, 0.3, 0.2, 0.1]
    s1 = [2.0, 0.9, 0.8, 0.5, 0.4, 0.3, 0.2, 0.1]
    (q0, k), (q1, _) = unit_key_inputs(s0), unit_key_inputs(s1)
    for sink, want_flag in ((0, 0), (1, 1)):
        cfg = O.RouteConfig(heads=1, nq=1, nk=8, d=16, k=2, m=2, r=0, sink=sink)
        led = O.anchor_layer(cfg, q0, k, 0)
        assert led.route[0, 0].tolist() == [1, 2]
        res = O.relay_layer(cfg, q1, k, 1, led)
        assert int(res.flags[0, 0]) == want_flag
        assert res.alpha[0, 0] == np.float32(0.8)
        assert res.beta[0, 0] == np.float32(2.0 if sink else 0.5)
        if want_flag:
            assert res.ledger.route[0, 0].tolist() == [0, 1]
            assert res.ledger.anchor[0, 0] == 1
        else:
            assert res.ledger.route[0, 0].tolist() == [1, 2]


@pytest.mark.parametrize("causal", [False, True])
def test_segments_partition_the_covered_chunks(causal):
    """On random rows: route, near-miss, mandatory and random segments are disjoint and
    allowed; every sink / recent chunk of the row sits in exactly one of route, near-miss,
    mandatory; the random segment avoids all of them and holds min(r, pool) chunks."""
    n = 40
    q, k = synth.gaussian_inputs(2, n, n, 64, seed=11, dtype="f32")
    cfg = O.RouteConfig(heads=2, nq=n, nk=n, d=64, k=4, m=3, r=5, sink=2, recent=3,
                        causal=causal, seed=9)
    led = O.anchor_layer(cfg, q, k, 2)
    mw = cfg.mand
    for h in range(2):
        for i in range(n):
            na = O.n_allowed(i, cfg)
            R = [j for j in led.route[h, i] if j >= 0]
            NM = [j for j in led.sent[h, i, :cfg.m] if j >= 0]
            MD = [j for j in led.sent[h, i, cfg.m:cfg.m + mw] if j >= 0]
            RN = [j for j in led.sent[h, i, cfg.m + mw:] if j >= 0]
            every = R + NM + MD + RN
            assert len(every) == len(set(every)) and all(0 <= j < na for j in every)
            special = set(range(min(2, na))) | set(range(max(0, na - 3), na))
            for j in special:
                assert (j in R) + (j in NM) + (j in MD) == 1
            assert set(MD) <= special
            pool = na - len(R) - len(NM) - len(MD)
            assert len(RN) == min(cfg.r, pool)
            assert MD == sorted(MD) and RN == sorted(RN)


def test_no_mandatory_keeps_the_two_segment_layout():
    """sink = recent = 0: the sentinel row is near-miss then random, width m + r."""
    q, k = unit_key_inputs(HAND_SCORES)
    cfg = O.RouteConfig(heads=1, nq=1, nk=10, d=16, k=2, m=2, r=8)
    led = O.anchor_layer(cfg, q, k, 0)
    assert led.sent.shape == (1, 1, 10)
    assert led.sent[0, 0].tolist() == [5, 7, 0, 2, 4, 6, 8, 9, -1, -1]

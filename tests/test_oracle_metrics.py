"""Pins for the measurement definitions (Section 4.4; Section 5, Tables 2 and 3)."""
import numpy as np
import pytest

import oracle as O
from tests.conftest import read_golden


def constants():
    return {row[0]: float(row[1]) for row in read_golden("page_constants.txt")}


def test_ledger_bytes_section_4_4():
    c = constants()
    assert O.ledger_bytes(int(c["ledger_nq"]), int(c["ledger_c"])) == c["ledger_kib"] * 1024


def test_fixed_stride_rerouted_fraction_table2():
    """A fixed stride of 4 over 32 layers refreshes every row at 8 layers: 25.0%."""
    c = constants()
    L, stride = int(c["stride4_layers"]), int(c["stride4_stride"])
    kinds = ["anchor" if l % stride == 0 else "relay" for l in range(L)]
    flags = [None if kd == "anchor" else np.zeros((1, 384), np.uint8) for kd in kinds]
    assert round(100 * O.reroute_fraction(kinds, flags, 384), 1) == c["stride4_rerouted_pct"]


@pytest.mark.parametrize("row", read_golden("sentinel_ablation_table3.txt"))
def test_score_pair_accounting_reproduces_table3(row):
    """Table 3 prints, per sentinel mix, the rerouted-row fraction and the evaluated
    score-pair fraction.  With one anchor layer out of 24 and 256 x 256 chunks, a
    flag history with the printed rerouted fraction must give the printed pair fraction
    when a relay row costs its c = k + m + r candidates plus, if refreshed, all 256."""
    nm, rnd, _, rerouted_pct, pairs_pct = int(row[0]), int(row[1]), row[2], float(row[3]), float(row[4])
    L, nq, nk, k = 24, 256, 256, 12
    c = k + nm + rnd
    total_flags = round(rerouted_pct / 100 * L * nq) - nq   # flagged (relay layer, row) pairs
    kinds = ["anchor"] + ["relay"] * (L - 1)
    per = np.zeros(L - 1, dtype=int)
    per[:] = total_flags // (L - 1)
    per[: total_flags % (L - 1)] += 1
    flags, cands = [None], [None]
    for x in per:
        f = np.zeros((1, nq), np.uint8)
        f[0, :x] = 1
        flags.append(f)
        cands.append(np.full((1, nq), c, np.int32))
    assert round(100 * O.reroute_fraction(kinds, flags, nq), 1) == rerouted_pct
    ev, full = O.pair_counts(kinds, 1, np.full(nq, nk), flags, cands)
    assert abs(100 * ev / full - pairs_pct) <= 0.1


def test_pair_counts_causal_rows_use_allowed_counts():
    n_row = np.arange(1, 9)
    kinds = ["anchor", "relay"]
    f = np.zeros((2, 8), np.uint8)
    f[1, 3] = 1
    cc = np.full((2, 8), 5, np.int32)
    ev, full = O.pair_counts(kinds, 2, n_row, [None, f], [None, cc])
    assert full == 2 * 2 * 36
    assert ev == 2 * 36 + 2 * 8 * 5 + 4


def test_route_recall_on_hand_built_routes():
    exact = np.array([[[0, 1, 2, 3], [4, 5, 6, -1]]], np.int32)
    used = np.array([[[0, 1, 9, 8], [4, 5, 6, -1]]], np.int32)
    assert O.route_recall(used, exact) == pytest.approx((0.5 + 1.0) / 2)

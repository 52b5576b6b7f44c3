"""The GPU parity comparators themselves, on hand-built values (no GPU needed): a comparator
that lets a wrong value through would void every parity test that uses it."""
import numpy as np
import pytest

import oracle as O
from tests import gpu_util as U

INF = np.inf


def test_check_scores_accepts_values_within_tolerance():
    assert U.check_scores([1.0005], [1.0], 1e-3, 0.0, "x") == pytest.approx(5e-4)
    # the row rms widens the band near zero
    assert U.check_scores([1e-4], [0.0], 1e-3, 0.5, "x") == pytest.approx(1e-4)


def test_check_scores_rejects_finite_against_minus_inf():
    """beta of a row without sentinels is -inf (Eq. 7 over an empty set): the GPU must return
    -inf too, not any finite number."""
    with pytest.raises(AssertionError):
        U.check_scores([0.5], [-INF], 1e-3, 1.0, "beta")
    with pytest.raises(AssertionError):
        U.check_scores([INF], [-INF], 1e-3, 1.0, "beta")
    with pytest.raises(AssertionError):
        U.check_scores([-3e38], [-INF], 1e-3, 1.0, "beta")
    assert U.check_scores([-INF], [-INF], 1e-3, 1.0, "beta") == 0.0


def test_check_scores_rejects_nan_mismatches():
    with pytest.raises(AssertionError):
        U.check_scores([np.nan], [0.25], 1e-3, 1.0, "s")          # NaN where a score is due
    with pytest.raises(AssertionError):
        U.check_scores([0.25], [np.nan], 1e-3, 1.0, "s")          # a score where the ID is -1
    with pytest.raises(AssertionError):
        U.check_scores([INF], [0.25], 1e-3, 1.0, "s")
    assert U.check_scores([np.nan, 0.25], [np.nan, 0.25], 1e-3, 1.0, "s") == 0.0


def test_check_scores_rejects_out_of_band_and_broadcasts_rms():
    with pytest.raises(AssertionError):
        U.check_scores([1.01], [1.0], 1e-3, 0.0, "x")
    got = np.array([[1.0, 2.0], [3.0, -INF]])
    ref = np.array([[1.0, 2.0 + 1e-4], [3.0, -INF]])
    U.check_scores(got, ref, 1e-3, np.array([[1.0], [1.0]]), "x")
    with pytest.raises(AssertionError):
        U.check_scores(got, ref, 1e-5, np.array([[1.0], [1.0]]), "x")


def _res(flags):
    flags = np.asarray(flags, np.uint8)
    H, nq = flags.shape
    return O.RelayResult(ledger=None, flags=flags, alpha=np.zeros((H, nq), np.float32),
                         beta=np.zeros((H, nq), np.float32), cand_scores=None,
                         rows=np.flatnonzero(flags.reshape(-1)).astype(np.int32),
                         head_counts=flags.sum(axis=1).astype(np.int32))


def test_check_compaction_on_matching_lists():
    res = _res([[0, 1, 1, 0], [1, 0, 0, 1]])
    mask = np.ones((2, 4), bool)
    U.check_compaction([1, 2, 4, 7], [2, 2], res.flags, res, mask, "same")


def test_check_compaction_rejects_a_missing_or_extra_row():
    res = _res([[0, 1, 1, 0], [1, 0, 0, 1]])
    mask = np.ones((2, 4), bool)
    g_flags = res.flags.copy()
    with pytest.raises(AssertionError):
        U.check_compaction([1, 4, 7], [1, 2], g_flags, res, mask, "missing")
    with pytest.raises(AssertionError):
        U.check_compaction([0, 1, 2, 4, 7], [3, 2], g_flags, res, mask, "extra")
    with pytest.raises(AssertionError):
        U.check_compaction([2, 1, 4, 7], [2, 2], g_flags, res, mask, "unordered")
    with pytest.raises(AssertionError):
        U.check_compaction([1, 2, 4, 7], [3, 1], g_flags, res, mask, "wrong counts")


def test_check_compaction_allows_differences_on_excluded_rows_only():
    """A row excluded by the gap rule may be flagged by one side only; the head count must then
    differ by exactly that row."""
    res = _res([[0, 1, 1, 0], [1, 0, 0, 1]])
    mask = np.ones((2, 4), bool)
    mask[0, 0] = False                                     # excluded: the GPU flags it, the oracle does not
    g_flags = res.flags.copy()
    g_flags[0, 0] = 1
    U.check_compaction([0, 1, 2, 4, 7], [3, 2], g_flags, res, mask, "excluded extra")
    with pytest.raises(AssertionError):
        U.check_compaction([0, 1, 2, 4, 7], [2, 2], g_flags, res, mask, "count not adjusted")
    mask2 = np.ones((2, 4), bool)
    with pytest.raises(AssertionError):                     # the same difference on a compared row
        U.check_compaction([0, 1, 2, 4, 7], [3, 2], g_flags, res, mask2, "not excluded")

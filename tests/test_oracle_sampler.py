"""Pins for the random-sentinel sampler (Section 3.1 item 2; Section 3.4, Eq. 10)."""
from math import comb

import numpy as np
import pytest

import oracle as O
import oracle.routing as OR


def draw(h, layer=3, i=5, n=40, excluded=range(8), r=8, seed=0):
    return O.random_sentinels(seed, h, layer, i, n, list(excluded), r)


@pytest.mark.parametrize("h", range(50))
def test_sample_is_distinct_subset_of_pool(h):
    excluded = [1, 2, 3, 5, 8, 13, 21, 34]
    s = draw(h, excluded=excluded)
    assert len(s) == 8 and len(set(s.tolist())) == 8
    assert all(0 <= j < 40 and j not in excluded for j in s)
    assert np.all(np.diff(s) > 0)


def test_small_pool_is_taken_whole():
    # pool N = 6 <= r = 8: take all of it (read of Eq. 10 with N <= r)
    s = O.random_sentinels(0, 0, 0, 0, 10, [0, 1, 2, 3], 8)
    assert s.tolist() == [4, 5, 6, 7, 8, 9]
    s = O.random_sentinels(0, 0, 0, 0, 12, list(range(4)), 8)  # N = 8 = r
    assert s.tolist() == list(range(4, 12))
    assert O.random_sentinels(0, 0, 0, 0, 3, [0, 1, 2], 8).tolist() == []


def test_draw_cap_fills_with_lowest_pool_members(monkeypatch):
    monkeypatch.setattr(OR, "SAMPLER_DRAW_CAP", 0)
    s = O.random_sentinels(0, 0, 0, 0, 40, [0, 2, 4], 5)
    assert s.tolist() == [1, 3, 5, 6, 7]


def test_sampler_is_keyed_by_every_counter_field():
    base = draw(0).tolist()
    assert draw(1).tolist() != base or draw(2).tolist() != base
    assert O.random_sentinels(0, 0, 4, 5, 40, list(range(8)), 8).tolist() != base
    assert O.random_sentinels(0, 0, 3, 6, 40, list(range(8)), 8).tolist() != base
    assert O.random_sentinels(1, 0, 3, 5, 40, list(range(8)), 8).tolist() != base
    assert O.random_sentinels(1 << 32, 0, 3, 5, 40, list(range(8)), 8).tolist() != base


@pytest.mark.slow
def test_eq10_miss_probability_and_uniform_inclusion():
    """Over 10^5 keyed draws from a pool of N = 32 with r = 8: the chance that u = 4 given
    pool members are all missed matches C(N-u, r) / C(N, r) (Eq. 10), and every pool
    member is included with probability r / N, each within a 4-sigma binomial band."""
    n, excluded, r = 40, list(range(8)), 8
    N = n - len(excluded)
    challengers = {10, 17, 23, 39}
    trials = 100_000
    miss = 0
    incl = np.zeros(n)
    for t in range(trials):
        s = O.random_sentinels(7, t % 64, t // 64, 5, n, excluded, r)
        ss = set(s.tolist())
        miss += not (ss & challengers)
        incl[s] += 1
    p = comb(N - len(challengers), r) / comb(N, r)
    assert p <= (1 - len(challengers) / N) ** r           # the bound in Eq. 10
    band = 4 * np.sqrt(p * (1 - p) / trials)
    assert abs(miss / trials - p) < band
    q = r / N
    band_q = 4 * np.sqrt(q * (1 - q) / trials)
    assert np.all(incl[excluded] == 0)
    assert np.all(np.abs(incl[8:] / trials - q) < band_q)


def test_zero_random_sentinels():
    assert O.random_sentinels(0, 0, 0, 0, 40, [0, 1], 0).tolist() == []

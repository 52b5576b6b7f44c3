"""Pins for the oracle's counter-based generator (the random-sentinel sampler's source)."""
import numpy as np
import pytest

from oracle import philox4x32_10, philox4x64_10
from tests.conftest import read_golden


def test_philox4x32_10_known_answers():
    """Published known-answer vectors of Philox4x32-10 (Random123 distribution)."""
    rows = read_golden("philox4x32_10_kat.txt")
    assert len(rows) == 3
    for row in rows:
        vals = [int(x, 16) for x in row]
        ctr, key, want = vals[0:4], vals[4:6], vals[6:10]
        assert list(philox4x32_10(ctr, key)) == want


@pytest.mark.parametrize("key", [(0, 0), (0x1234567890ABCDEF, 0xFEDCBA0987654321), (2**64 - 1, 7)])
@pytest.mark.parametrize("ctr", [(0, 0, 0, 0), (5, 1, 2, 3), (2**64 - 2, 2**63, 11, 2**40)])
def test_philox_round_structure_matches_numpy_4x64(ctr, key):
    """numpy.random.Philox is Philox4x64-10; it increments the counter before each
    block.  The oracle's shared round function, instantiated at 64 bits, must agree."""
    g = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    got = [int(x) for x in g.random_raw(8)]
    c1 = list(ctr)
    c1[0] = (c1[0] + 1) % 2**64
    if c1[0] == 0:
        c1[1] = (c1[1] + 1) % 2**64
    c2 = list(c1)
    c2[0] = (c2[0] + 1) % 2**64
    if c2[0] == 0:
        c2[1] = (c2[1] + 1) % 2**64
    want = list(philox4x64_10(c1, key)) + list(philox4x64_10(c2, key))
    assert got == want


def test_philox4x32_outputs_look_uniform():
    """Sanity of the 32-bit instance beyond the three vectors: mean and bit balance of
    4096 words over consecutive counters."""
    words = []
    for t in range(1024):
        words.extend(philox4x32_10((t, 3, 5, 7), (11, 13)))
    w = np.array(words, dtype=np.uint64)
    u = w / 2.0**32
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / len(u))
    bits = np.array([(w >> np.uint64(b)) & np.uint64(1) for b in range(32)], dtype=np.float64)
    assert np.all(np.abs(bits.mean(axis=1) - 0.5) < 4 * 0.5 / np.sqrt(len(u)))

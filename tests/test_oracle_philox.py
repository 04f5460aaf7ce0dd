"""Pins of the oracle's Philox4x64-10 and its uniform mapping.

The pages name no generator; the counter-based Philox4x64-10 of Salmon et al.
(SC'11) is this library's reading.  The oracle's implementation is pinned to
the published known answer and to NumPy's independent implementation.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden
from np_philox import block as _numpy_block


def test_known_answer():
    kat = read_golden("philox_kat.txt")["_rows"][0]
    want = np.array([int(x, 16) for x in kat], dtype=np.uint64)
    got = oracle.philox4x64_10([0, 0, 0, 0], [0, 0])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(8))
def test_matches_numpy_philox(seed):
    r = np.random.default_rng(1234 + seed)
    for _ in range(50):
        ctr = r.integers(0, 2**64, size=4, dtype=np.uint64)
        if seed == 0:
            ctr[:] = [r.integers(0, 5), 0, 0, 0]          # small counters, including 0
        key = r.integers(0, 2**64, size=2, dtype=np.uint64)
        assert np.array_equal(oracle.philox4x64_10(ctr, key), _numpy_block(ctr, key))


def test_uniform_is_exact_map_of_first_word():
    r = np.random.default_rng(7)
    for _ in range(200):
        seed, c0, step, stream = (int(x) for x in r.integers(0, 2**63, size=4))
        w0 = int(_numpy_block([c0, step, stream, oracle.TAG_ACCEPT], [seed, 0])[0])
        want = (2 * (w0 >> 12) + 1) / 2.0**53          # exact: a 53-bit odd integer over 2^53
        u = oracle.uniform(seed, c0, step, stream, oracle.TAG_ACCEPT)
        assert u == want and 0.0 < u < 1.0


def test_uniform_moments():
    us = np.array([oracle.uniform(5, i, 0, 0, oracle.TAG_WALK) for i in range(20000)])
    n = len(us)
    assert abs(us.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n)
    assert abs(us.var() - 1 / 12) < 4 * np.sqrt(1 / 180 / n)
    # Kolmogorov-Smirnov against U(0,1)
    from scipy import stats
    assert stats.kstest(us, "uniform").pvalue > 1e-4

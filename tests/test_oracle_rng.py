"""Pins of the oracle's counter-based generator against numpy's Philox4x64-10.

numpy.random.Philox is an independent implementation of the same published
generator (Salmon et al., SC'11).  Calibrated layout: numpy increments its 256-bit
little-endian counter BEFORE producing each 4-word block, so the block numpy
returns first for counter c is the block function at c + 1.
"""
import numpy as np
import pytest

from oracle import philox

MASK = (1 << 64) - 1


def numpy_block(counter, key):
    """Philox block at `counter` via numpy (counter is given as 4 words, low word first)."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & MASK for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=words)
    return [int(v) for v in bg.random_raw(4)]


CASES = [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (1, 2)),
    ((7, 3, 0, 0), (0xDEADBEEF, 5)),
    ((MASK, MASK, MASK, MASK), (MASK, MASK)),
    ((123456789, 42, 99, 0), (1004, 0)),
    ((0, 1 << 63, 5, 1), (2 ** 40 + 3, 1)),
]


@pytest.mark.parametrize("counter,key", CASES)
def test_block_matches_numpy(counter, key):
    assert list(philox.philox4x64(counter, key)) == numpy_block(counter, key)


def test_many_random_blocks_match_numpy():
    rng = np.random.default_rng(7)
    for _ in range(200):
        counter = [int(v) for v in rng.integers(0, 2 ** 63, 4, dtype=np.uint64)]
        key = [int(v) for v in rng.integers(0, 2 ** 63, 2, dtype=np.uint64)]
        assert list(philox.philox4x64(counter, key)) == numpy_block(counter, key)


def test_uniform_contract_grid_and_range():
    us = np.array(philox.uniforms(1003, 0, 5, 16, 8), dtype=np.float64)
    assert us.shape == (16, 9)
    assert (us >= 0).all() and (us < 1).all()
    # every draw is k * 2^-24 and survives a round trip through fp32 unchanged
    k = us * 2 ** 24
    assert (k == np.floor(k)).all()
    assert (us.astype(np.float32).astype(np.float64) == us).all()
    # the contract: word 0 of the block at counter (t, b, step, 0) under key (seed, domain)
    w0 = numpy_block((3, 2, 5, 0), (1003, 0))[0]
    assert us[2, 3] == (w0 >> 40) / 2 ** 24


def test_uniform_streams_are_distinct_and_roughly_uniform():
    a = np.array(philox.uniforms(1, 0, 0, 64, 15)).ravel()
    b = np.array(philox.uniforms(1, 1, 0, 64, 15)).ravel()
    c = np.array(philox.uniforms(1, 0, 1, 64, 15)).ravel()
    assert not np.array_equal(a, b) and not np.array_equal(a, c)
    allu = np.concatenate([a, b, c])
    # 3072 draws: the mean of U(0,1) has sd 0.0052; 5 sd bound
    assert abs(allu.mean() - 0.5) < 0.027
    hist, _ = np.histogram(allu, bins=8, range=(0, 1))
    expected = len(allu) / 8
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 24.3  # chi-square, 7 dof, p = 0.001

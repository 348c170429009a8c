"""Pins for the oracle's Philox4x64-10 and its uniform mapping.

The independent known-answer source is numpy.random.Philox (Philox4x64-10).
numpy advances its 256-bit counter before producing a block, so numpy's first
block for counter c is the block at c + 1.
"""
import numpy as np
import pytest
from numpy.random import Philox


def _numpy_block(seed, ctr, key1=0):
    c = 0
    for i, w in enumerate(ctr):
        c |= int(w) << (64 * i)
    c = (c - 1) % (1 << 256)          # numpy pre-increments
    words = np.array([(c >> (64 * i)) & (2**64 - 1) for i in range(4)], dtype=np.uint64)
    g = Philox(key=np.array([seed, key1], dtype=np.uint64), counter=words)
    return g.random_raw(4)


@pytest.mark.parametrize("seed", [0, 2, 5, 4_000_000, 2**63 + 12345, 2**64 - 1])
@pytest.mark.parametrize("ctr", [(0, 0, 0, 0), (1, 0, 0, 0), (14, 63, 0, 0), (7, 0, 0, 0),
                                 (2**64 - 1, 3, 0, 0), (5, 6, 7, 8)])
def test_philox_matches_numpy(orc, seed, ctr):
    mine = orc.philox(seed, ctr)
    ref = _numpy_block(seed, ctr)
    assert [int(x) for x in mine] == [int(x) for x in ref]


def test_philox_second_key_word(orc):
    mine = orc.philox(9, (3, 1, 0, 0), key1=77)
    ref = _numpy_block(9, (3, 1, 0, 0), key1=77)
    assert [int(x) for x in mine] == [int(x) for x in ref]


def test_uniform_exact_in_float32_and_open_interval(orc):
    words = [0, 1, 2**41 - 1, 2**41, 2**63, 2**64 - 1, 0x123456789ABCDEF0]
    for w in words:
        u = orc.uniform_from_word(w)
        assert 0.0 < u < 1.0
        assert float(np.float32(u)) == u
    assert orc.uniform_from_word(0) == 2.0**-24
    assert orc.uniform_from_word(2**64 - 1) == 1.0 - 2.0**-24


def test_uniform_is_uniform(orc):
    # 4096 blocks -> 16384 words; mean and a 16-bin histogram
    us = []
    for t in range(64):
        for b in range(64):
            us.extend(orc.uniform_from_word(int(w)) for w in orc.philox(11, (t, b, 0, 0)))
    us = np.array(us)
    assert abs(us.mean() - 0.5) < 4 * np.sqrt(1 / 12 / len(us))
    hist = np.histogram(us, bins=16, range=(0, 1))[0]
    e = len(us) / 16
    chi2 = ((hist - e) ** 2 / e).sum()
    assert chi2 < 50.0  # 15 dof; p ~ 1e-5

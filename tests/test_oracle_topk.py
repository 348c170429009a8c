"""Pins for the oracle's top-K: numpy's stable argsort (a library routine) and
a brute-force repeated-maximum selection."""
import numpy as np
import pytest
import torch

import synth


def _stable_ref(x, k):
    order = np.argsort(-x.astype(np.float64), axis=-1, kind="stable")[..., :k]
    return order.astype(np.int32), np.take_along_axis(x, order, -1).astype(np.float32)


def _brute(x, k):
    x = x.astype(np.float64).copy()
    idx = []
    for _ in range(k):
        m = x.max()
        j = int(np.flatnonzero(x == m)[0])   # lowest index among the maxima
        idx.append(j)
        x[j] = -np.inf
    return np.array(idx, np.int32)


@pytest.mark.parametrize("k", [1, 4, 16])
def test_topk_fp32_matches_stable_argsort(orc, k):
    rng = np.random.default_rng(1)
    x = np.round(rng.normal(size=(6, 777)) * 4).astype(np.float32)   # many ties
    idx, val = orc.topk(x, k)
    ridx, rval = _stable_ref(x, k)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_array_equal(val, rval)


@pytest.mark.parametrize("k", [4, 16])
def test_topk_bf16_matches_stable_argsort(orc, k):
    g = torch.Generator().manual_seed(2)
    x = (3 * torch.randn(5, 3001, generator=g)).to(torch.bfloat16)
    idx, val = orc.topk(x, k)
    xf = x.float().numpy()
    ridx, rval = _stable_ref(xf, k)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_array_equal(val, rval)


def test_topk_bruteforce_v1000(orc):
    rng = np.random.default_rng(3)
    x = np.round(rng.normal(size=(4, 1000)) * 8).astype(np.float32)
    idx, _ = orc.topk(x, 16)
    for r in range(4):
        np.testing.assert_array_equal(idx[r], _brute(x[r], 16))


def test_topk_signed_zero_is_a_tie(orc):
    x = np.array([[-0.0, 0.0, -1.0, 0.0, -0.0]], np.float32)
    idx, _ = orc.topk(x, 5)
    np.testing.assert_array_equal(idx[0], [0, 1, 3, 4, 2])


def test_topk_all_equal_row_takes_lowest_indices(orc):
    x = np.full((2, 100), 1.5, np.float32)
    idx, _ = orc.topk(x, 16)
    np.testing.assert_array_equal(idx, np.tile(np.arange(16, dtype=np.int32), (2, 1)))


def test_topk_tiny_workload_rank_by_counting(orc):
    """The rank of a token is the number of entries that beat it (greater
    value, or equal value at a lower index); the oracle's K-list holds the
    tokens of rank 0..K-1 in that order."""
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, tok, _ = synth.drafter_logits(w)
    idx, val = orc.topk(z, w.K)
    x = z.numpy()
    for t in range(w.T):
        row = x[0, t]
        ar = np.arange(row.size)
        rank = np.array([np.sum(row > row[v]) + np.sum((row == row[v]) & (ar < v)) for v in ar])
        np.testing.assert_array_equal(idx[0, t], np.argsort(rank)[: w.K])
    assert np.all(np.diff(val, axis=-1) <= 0)

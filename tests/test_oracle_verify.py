"""Pins for the oracle's verification.

Greedy: the emitted tokens are the target's own argmax chain (the lossless
greedy claim), the accepted length never exceeds T = block - 1, and full
agreement yields the bonus token.  Rejection sampling: Monte Carlo shows the
emitted tokens follow the target distribution p whatever the proposal q;
q = p always accepts; a near-zero temperature reduces it to greedy."""
import numpy as np
import pytest
import torch

import synth


def test_greedy_output_is_target_argmax_chain(orc):
    g = torch.Generator().manual_seed(0)
    B, T, V = 64, 7, 300
    Z = torch.randn(B, T + 1, V, generator=g)
    y = Z.argmax(-1).numpy()
    path = y[:, :T].copy().astype(np.int32)
    # corrupt a random position (or none) per row
    cut = np.random.default_rng(1).integers(0, T + 1, size=B)
    for b in range(B):
        if cut[b] < T:
            path[b, cut[b]] = (path[b, cut[b]] + 1) % V
    out = orc.verify_greedy(Z, path)
    np.testing.assert_array_equal(out["argmax"], np.argmax(Z.numpy(), -1))
    for b in range(B):
        n = out["accept_len"][b]
        assert n == cut[b] and 0 <= n <= T
        np.testing.assert_array_equal(out["out_tok"][b, : n + 1], y[b, : n + 1])
        assert np.all(out["out_tok"][b, n + 1:] == -1)


def test_greedy_argmax_ties_take_lowest_index(orc):
    Z = np.zeros((1, 2, 10), np.float32)
    Z[0, 0, [3, 7]] = 5.0
    Z[0, 1, [9, 2]] = 1.0
    out = orc.verify_greedy(Z, np.array([[3]], np.int32))
    np.testing.assert_array_equal(out["argmax"][0], [3, 2])
    assert out["accept_len"][0] == 1
    np.testing.assert_array_equal(out["out_tok"][0], [3, 2])


def test_greedy_bf16_tiny_workload(orc):
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, tok, _ = synth.drafter_logits(w)
    Z = synth.target_logits(w, z, tok)
    assert Z.shape == (1, 4, 1000)
    idx, val = orc.topk(z, w.K)
    out = orc.verify_greedy(Z, idx[..., 0])
    assert 0 <= out["accept_len"][0] <= w.T


def _softmax(x, tau):
    x = np.asarray(x, np.float64) / tau
    e = np.exp(x - x.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def _chi2(counts, probs):
    n = counts.sum()
    e = n * probs
    keep = e > 5
    return float((((counts - e) ** 2) / np.maximum(e, 1e-300))[keep].sum())


def test_rejection_sampling_preserves_target_distribution(orc):
    """V = 8, K = 4, T = 2.  Per row b the drafts are drawn from a fixed
    proposal q_t over four candidate tokens (numpy's own generator, not the
    oracle's); the emitted first token must follow p_0, the second (given an
    accepted first draft) p_1 and the bonus (given two accepted drafts) p_2."""
    V, K, T, tau = 8, 4, 2, 1.0
    N = 200_000
    rng = np.random.default_rng(42)
    Zrow = rng.normal(size=(T + 1, V)).astype(np.float32) * 1.5
    p = _softmax(Zrow, tau)
    cands = np.array([[1, 4, 6, 7], [0, 2, 3, 5]], np.int32)
    qrow = np.array([[0.4, 0.3, 0.2, 0.1], [0.1, 0.2, 0.3, 0.4]], np.float32)
    Z = np.broadcast_to(Zrow, (N, T + 1, V)).copy()
    rank = np.stack([rng.choice(K, size=N, p=qrow[t] / qrow[t].sum()) for t in range(T)], 1)
    rank = rank.astype(np.int32)
    tok = np.take_along_axis(np.broadcast_to(cands, (N, T, K)), rank[..., None], -1)[..., 0]
    cand = np.broadcast_to(cands, (N, T, K)).copy()
    q = np.broadcast_to(qrow, (N, T, K)).copy()
    out = orc.verify_reject(Z, tok.astype(np.int32), rank, cand, q, tau, seed=77)
    assert out["fallbacks"] == 0
    n = out["accept_len"]
    o = out["out_tok"]
    assert np.all((0 <= n) & (n <= T))
    assert _chi2(np.bincount(o[:, 0], minlength=V).astype(float), p[0]) < 35.0   # dof <= 7
    sel = n >= 1
    assert _chi2(np.bincount(o[sel, 1], minlength=V).astype(float), p[1]) < 35.0
    sel = n == 2
    assert _chi2(np.bincount(o[sel, 2], minlength=V).astype(float), p[2]) < 35.0
    # acceptance rate of draft 0 is sum_c min(p, q) over the candidates
    qt = np.zeros(V)
    qt[cands[0]] = qrow[0]
    acc0 = np.minimum(p[0], qt).sum()
    got = (n >= 1).mean()
    assert abs(got - acc0) < 5 * np.sqrt(acc0 * (1 - acc0) / N)


def test_rejection_with_q_equal_p_always_accepts(orc):
    V, K, T = 16, 4, 3
    Z = np.full((1, T + 1, V), -1.0e4, np.float32)
    cands = np.array([[[2, 5, 9, 11], [0, 1, 2, 3], [12, 13, 14, 15]]], np.int32)
    for t in range(T):
        Z[0, t, cands[0, t]] = 0.0          # p = 1/4 exactly on the candidates
    Z[0, T, 6] = 0.0
    q = np.full((1, T, K), 0.25, np.float32)
    for seed in range(50):
        rank = np.random.default_rng(seed).integers(0, K, size=(1, T)).astype(np.int32)
        tok = np.take_along_axis(cands, rank[..., None], -1)[..., 0]
        out = orc.verify_reject(Z, tok, rank, cands, q, 1.0, seed=seed)
        assert out["accept_len"][0] == T
        assert out["out_tok"][0, T] == 6


def test_rejection_near_zero_temperature_equals_greedy(orc):
    g = torch.Generator().manual_seed(3)
    B, T, V, K = 32, 5, 200, 16
    Z = 4 * torch.randn(B, T + 1, V, generator=g)
    y = Z.argmax(-1).numpy()
    cand = np.stack([np.argsort(-Z[:, t].numpy(), -1, kind="stable")[:, :K] for t in range(T)], 1)
    cand = cand.astype(np.int32)
    rng = np.random.default_rng(4)
    rank = np.where(rng.random((B, T)) < 0.8, 0, rng.integers(1, K, size=(B, T))).astype(np.int32)
    tok = np.take_along_axis(cand, rank[..., None], -1)[..., 0]
    q = np.zeros((B, T, K), np.float32)
    np.put_along_axis(q, rank[..., None], 1.0, -1)
    rej = orc.verify_reject(Z, tok, rank, cand, q, 1e-4, seed=9)
    gre = orc.verify_greedy(Z, tok)
    np.testing.assert_array_equal(rej["accept_len"], gre["accept_len"])
    np.testing.assert_array_equal(rej["out_tok"], gre["out_tok"])
    assert np.all(gre["out_tok"][np.arange(B), gre["accept_len"]] ==
                  y[np.arange(B), gre["accept_len"]])


def test_reject_requires_positive_temperature(orc):
    Z = np.zeros((1, 2, 8), np.float32)
    with pytest.raises(orc.OracleError):
        orc.verify_reject(Z, np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32),
                          np.zeros((1, 1, 4), np.int32), np.full((1, 1, 4), 0.25, np.float32),
                          0.0, seed=1)


def test_reject_sub_ranges_equal_one_call(orc):
    """The uniforms are keyed by the request's index in the whole batch, so
    verifying a batch as two sub-ranges (with their batch indices) gives
    exactly the result of one call over the batch, and a sub-range called
    with the wrong indices (counted from 0) draws different uniforms."""
    rng = np.random.default_rng(4)
    B, T, V, K = 24, 5, 50, 4
    Z = (rng.normal(size=(B, T + 1, V)) * 2).astype(np.float32)
    idx = np.stack([rng.choice(V, size=(T, K), replace=False) for _ in range(B)]).astype(np.int32)
    rank = rng.integers(0, K, size=(B, T)).astype(np.int32)
    tok = np.take_along_axis(idx, rank[..., None], -1)[..., 0].astype(np.int32)
    q = rng.dirichlet(np.ones(K), size=(B, T)).astype(np.float32)
    full = orc.verify_reject(Z, tok, rank, idx, q, 1.0, 11)
    parts = [orc.verify_reject(Z[a:b], tok[a:b], rank[a:b], idx[a:b], q[a:b], 1.0, 11, b_ids=np.arange(a, b))
             for a, b in ((0, 9), (9, B))]
    np.testing.assert_array_equal(np.concatenate([p["accept_len"] for p in parts]), full["accept_len"])
    np.testing.assert_array_equal(np.concatenate([p["out_tok"] for p in parts]), full["out_tok"])
    wrong = orc.verify_reject(Z[9:], tok[9:], rank[9:], idx[9:], q[9:], 1.0, 11)
    assert not np.array_equal(wrong["out_tok"], full["out_tok"][9:])

"""Pins for the oracle's path search: brute force over every path (with the
tie rule written as an ordering on whole paths), Viterbi >= greedy, the
rank-independent special case, and Monte Carlo for the sampled path."""
import itertools

import numpy as np
import pytest
import torch

import synth


def _path_sum(S, path):
    """float32 running sum along a path, the same additions a chain of
    float adds makes (the score of a path is defined in float)."""
    tot = np.float32(S[0, 0, path[0]])
    for t in range(1, len(path)):
        tot = np.float32(tot + np.float32(S[t, path[t - 1], path[t]]))
    return tot


def _brute(S):
    T, K = S.shape[0], S.shape[1]
    best, best_paths = None, []
    for p in itertools.product(range(K), repeat=T):
        s = _path_sum(S, p)
        if best is None or s > best:
            best, best_paths = s, [p]
        elif s == best:
            best_paths.append(p)
    # tie rule: lowest end rank first, then lowest back-pointers walking back
    chosen = min(best_paths, key=lambda p: tuple(reversed(p)))
    return best, chosen


@pytest.mark.parametrize("B,T,K,ties", [(3, 3, 4, False), (2, 3, 16, False), (2, 7, 4, False),
                                        (4, 4, 4, True), (2, 3, 16, True)])
def test_viterbi_equals_brute_force(orc, B, T, K, ties):
    S = synth.pair_score_lattice(B, T, K, seed=100 + T * K, ties=ties).numpy()
    cand = np.arange(B * T * K, dtype=np.int32).reshape(B, T, K)
    out = orc.path(S, cand, orc.PATH_VITERBI)
    for b in range(B):
        best, chosen = _brute(S[b])
        assert out["score"][b] == best
        assert tuple(out["rank"][b]) == chosen
        np.testing.assert_array_equal(out["tok"][b], cand[b, np.arange(T), out["rank"][b]])


def test_tiny_workload_all_64_paths(orc):
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, _, _ = synth.drafter_logits(w)
    idx, val = orc.topk(z, w.K)
    wa, wb, wh = synth.selector_weights(w)
    S = orc.pair_scores(idx, val, synth.last_tokens(w), synth.embeddings(w),
                        synth.context_hidden(w), wa, wb, wh)
    vit = orc.path(S, idx, orc.PATH_VITERBI)
    gre = orc.path(S, idx, orc.PATH_GREEDY)
    best, chosen = _brute(S[0])
    assert len(list(itertools.product(range(4), repeat=3))) == 64
    assert vit["score"][0] == best and tuple(vit["rank"][0]) == chosen
    assert vit["score"][0] >= gre["score"][0]


def test_viterbi_at_least_greedy(orc):
    S = synth.pair_score_lattice(64, 7, 16, seed=5).numpy()
    cand = np.zeros((64, 7, 16), np.int32)
    v = orc.path(S, cand, orc.PATH_VITERBI)
    g = orc.path(S, cand, orc.PATH_GREEDY)
    assert np.all(v["score"] >= g["score"])
    assert np.any(v["score"] > g["score"])   # the lattices are not all trivial


def test_greedy_follows_best_successor(orc):
    S = synth.pair_score_lattice(8, 5, 16, seed=6).numpy()
    cand = np.zeros((8, 5, 16), np.int32)
    g = orc.path(S, cand, orc.PATH_GREEDY)
    for b in range(8):
        prev = 0
        for t in range(5):
            row = S[b, t, prev]
            assert g["rank"][b, t] == int(np.flatnonzero(row == row.max())[0])
            prev = g["rank"][b, t]
        assert g["score"][b] == _path_sum(S[b], g["rank"][b])


def test_rank_independent_scores_reduce_to_per_position_argmax(orc):
    """S_t(a, b) = U_t(b) for every a (no bigram term): every mode that is
    deterministic picks the per-position argmax of U."""
    g = torch.Generator().manual_seed(8)
    U = 3 * torch.randn(5, 6, 16, generator=g)
    S = U[:, :, None, :].expand(5, 6, 16, 16).clone()
    S[:, 0, 1:, :] = float("-inf")
    cand = np.zeros((5, 6, 16), np.int32)
    am = U.argmax(-1).numpy()
    for mode in (orc.PATH_VITERBI, orc.PATH_GREEDY):
        out = orc.path(S.numpy(), cand, mode)
        np.testing.assert_array_equal(out["rank"], am)


def test_deterministic_modes_store_one_hot_proposals(orc):
    S = synth.pair_score_lattice(3, 4, 16, seed=9).numpy()
    cand = np.zeros((3, 4, 16), np.int32)
    for mode in (orc.PATH_VITERBI, orc.PATH_GREEDY):
        out = orc.path(S, cand, mode)
        np.testing.assert_array_equal(out["q"].argmax(-1), out["rank"])
        np.testing.assert_array_equal(out["q"].sum(-1), 1.0)


def _chi2(counts, probs):
    n = counts.sum()
    e = n * probs
    keep = e > 5
    return float((((counts - e) ** 2) / np.maximum(e, 1e-300))[keep].sum()), int(keep.sum()) - 1


def test_sampled_path_follows_softmax_of_scores(orc):
    """c_0 ~ softmax(S_0(last, .)/tau) and c_1 | c_0 ~ softmax(S_1(c_0, .)/tau).
    Each request row b uses its own Philox counter, so one call with many
    copies of the same lattice is many independent draws."""
    K, T, tau = 4, 2, 0.7
    base = synth.pair_score_lattice(1, T, K, seed=10, spread=1.0).numpy()[0]
    N = 60000
    S = np.broadcast_to(base, (N, T, K, K)).copy()
    cand = np.zeros((N, T, K), np.int32)
    out = orc.path(S, cand, orc.PATH_SAMPLE, temperature=tau, seed=1234)

    def softmax(x):
        e = np.exp((x - x.max()) / tau)
        return e / e.sum()

    p0 = softmax(base[0, 0].astype(np.float64))
    c0 = out["rank"][:, 0]
    chi, dof = _chi2(np.bincount(c0, minlength=K).astype(float), p0)
    assert chi < 25.0, (chi, dof)          # dof 3; p ~ 1e-5
    for a in range(K):
        sel = c0 == a
        if sel.sum() < 2000:
            continue
        p1 = softmax(base[1, a].astype(np.float64))
        chi, dof = _chi2(np.bincount(out["rank"][sel, 1], minlength=K).astype(float), p1)
        assert chi < 25.0, (a, chi, dof)
    # the stored proposal is the distribution the draw used
    np.testing.assert_allclose(out["q"][0, 0], p0.astype(np.float32), rtol=1e-6)
    np.testing.assert_allclose(out["q"].sum(-1), 1.0, rtol=1e-6)


def test_sampled_path_near_zero_temperature_is_greedy(orc):
    S = synth.pair_score_lattice(16, 5, 16, seed=12).numpy()
    cand = np.zeros((16, 5, 16), np.int32)
    g = orc.path(S, cand, orc.PATH_GREEDY)
    s = orc.path(S, cand, orc.PATH_SAMPLE, temperature=1e-5, seed=3)
    np.testing.assert_array_equal(s["rank"], g["rank"])


def test_sampled_path_depends_on_seed_and_is_reproducible(orc):
    S = synth.pair_score_lattice(64, 5, 16, seed=13, spread=0.5).numpy()
    cand = np.zeros((64, 5, 16), np.int32)
    a = orc.path(S, cand, orc.PATH_SAMPLE, temperature=1.0, seed=1)
    b = orc.path(S, cand, orc.PATH_SAMPLE, temperature=1.0, seed=1)
    c = orc.path(S, cand, orc.PATH_SAMPLE, temperature=1.0, seed=2)
    np.testing.assert_array_equal(a["rank"], b["rank"])
    assert np.any(a["rank"] != c["rank"])


def test_sample_requires_positive_temperature(orc):
    S = synth.pair_score_lattice(1, 2, 4, seed=1).numpy()
    with pytest.raises(orc.OracleError):
        orc.path(S, np.zeros((1, 2, 4), np.int32), orc.PATH_SAMPLE, temperature=0.0)


def test_sample_sub_ranges_equal_one_call(orc):
    """Sampled paths draw uniforms keyed by the request's batch index: two
    sub-range calls with their batch indices equal one call."""
    S = synth.pair_score_lattice(20, 6, 16, seed=8, spread=1.0).numpy()
    idx = np.broadcast_to(np.arange(16, dtype=np.int32), (20, 6, 16)).copy()
    full = orc.path(S, idx, orc.PATH_SAMPLE, temperature=1.0, seed=3)
    lo = orc.path(S[:8], idx[:8], orc.PATH_SAMPLE, temperature=1.0, seed=3, b_ids=np.arange(8))
    hi = orc.path(S[8:], idx[8:], orc.PATH_SAMPLE, temperature=1.0, seed=3, b_ids=np.arange(8, 20))
    np.testing.assert_array_equal(np.concatenate([lo["rank"], hi["rank"]]), full["rank"])
    wrong = orc.path(S[8:], idx[8:], orc.PATH_SAMPLE, temperature=1.0, seed=3)
    assert not np.array_equal(wrong["rank"], full["rank"][8:])

"""Pins for the oracle's projections and pair scores.

* projection: a float64 matrix product (numpy, a library routine the C oracle
  does not use);
* pair scores: special cases whose answer is fixed without retyping the
  equation -- H = 0 reduces the score to the drafter's logit (plain DFlash
  top-1 drafting), and one-hot embeddings with identity / permutation maps
  turn the bilinear term into a lookup whose value is known by inspection;
  linearity in W_H; and an einsum written from the equation as a check of
  the index placement.
"""
import numpy as np
import pytest
import torch

import synth


def _bf16(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def _rand_inputs(B=2, T=3, K=4, V=50, d=32, r=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    cand = torch.randint(0, V, (B, T, K), generator=g, dtype=torch.int32)
    U = 3 * torch.randn(B, T, K, generator=g)
    last = torch.randint(0, V, (B,), generator=g, dtype=torch.int32)
    E = (torch.randn(V, d, generator=g) * 0.5).to(torch.bfloat16)
    h = torch.randn(B, T, d, generator=g).to(torch.bfloat16)
    wa = (torch.randn(r, d, generator=g) * 0.3).to(torch.bfloat16)
    wb = (torch.randn(r, d, generator=g) * 0.3).to(torch.bfloat16)
    wh = (torch.randn(r, d, generator=g) * 0.3).to(torch.bfloat16)
    return cand, U, last, E, h, wa, wb, wh


def test_project_matches_float64_matmul(orc):
    g = torch.Generator().manual_seed(1)
    x = torch.randn(37, 96, generator=g).to(torch.bfloat16)
    w = torch.randn(24, 96, generator=g).to(torch.bfloat16)
    out = orc.project(x, w)
    ref = x.double().numpy() @ w.double().numpy().T
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    out_s = orc.project(x, w, gate=orc.GATE_SIGMOID)
    np.testing.assert_allclose(out_s, 1 / (1 + np.exp(-ref)), rtol=1e-12, atol=1e-14)


def test_h_zero_reduces_to_drafter_logits(orc):
    cand, U, last, E, h, wa, wb, wh = _rand_inputs()
    S = orc.pair_scores(cand, U, last, E, h, wa, wb, torch.zeros_like(wh))
    B, T, K, _ = S.shape
    for t in range(T):
        rows = [0] if t == 0 else range(K)
        for i in rows:
            np.testing.assert_array_equal(S[:, t, i, :], U[:, t, :].numpy())
    assert np.all(np.isneginf(S[:, 0, 1:, :]))


def test_one_hot_embeddings_make_the_bigram_a_lookup(orc):
    """E[v] = e_{v mod r}; W_A = I, W_B = P (a permutation), W_H = I, gate
    identity.  Then A(a) = e_{a mod r}, B(b) = e_{pi(b mod r)}, H_t = h_t and
    <A(a) . H_t, B(b)> = h_t[a mod r] if a mod r == pi(b mod r) else 0.
    The predecessor a is a candidate of position t-1 (the last verified
    token at t = 0) and the gate comes from position t."""
    r = d = 8
    B, T, K, V = 2, 4, 3, 40
    rng = np.random.default_rng(5)
    perm = rng.permutation(r)
    P = np.zeros((r, d), np.float32)
    for j in range(r):
        P[perm[j], j] = 1.0        # (P e_j) = e_{perm[j]}
    E = np.zeros((V, d), np.float32)
    E[np.arange(V), np.arange(V) % r] = 1.0
    h = rng.integers(1, 50, size=(B, T, d)).astype(np.float32)   # exact in bf16
    cand = rng.integers(0, V, size=(B, T, K)).astype(np.int32)
    # force some matches: candidate j of position t gets pi(b mod r) == a mod r
    for b in range(B):
        for t in range(1, T):
            a = cand[b, t - 1, 0] % r
            j_of = int(np.flatnonzero(perm == a)[0])
            cand[b, t, 1] = j_of + r * rng.integers(0, V // r)
    last = rng.integers(0, V, size=(B,)).astype(np.int32)
    U = rng.normal(size=(B, T, K)).astype(np.float32)
    S = orc.pair_scores(cand, U, last, _bf16(E), _bf16(h), _bf16(np.eye(r)), _bf16(P),
                        _bf16(np.eye(r)))
    for b in range(B):
        for t in range(T):
            preds = [last[b]] if t == 0 else list(cand[b, t - 1])
            for i, a in enumerate(preds):
                for j in range(K):
                    bb = cand[b, t, j]
                    expect = U[b, t, j] + (h[b, t, a % r] if a % r == perm[bb % r] else 0.0)
                    assert S[b, t, i, j] == np.float32(expect), (b, t, i, j)


def test_bigram_linear_in_gate_weights(orc):
    cand, U, last, E, h, wa, wb, wh = _rand_inputs(seed=3)
    S1 = orc.pair_scores(cand, U, last, E, h, wa, wb, wh).astype(np.float64)
    S2 = orc.pair_scores(cand, U, last, E, h, wa, wb, (wh.float() * 2).to(torch.bfloat16))
    S2 = S2.astype(np.float64)
    Ub = U.numpy()[:, :, None, :].astype(np.float64)
    m = np.isfinite(S1)
    np.testing.assert_allclose((S2 - Ub)[m], 2 * (S1 - Ub)[m], rtol=1e-5, atol=1e-5)
    # negating W_A negates the bigram term
    S3 = orc.pair_scores(cand, U, last, E, h, (-wa.float()).to(torch.bfloat16), wb, wh)
    np.testing.assert_allclose((S3 - Ub)[m], -(S1 - Ub)[m], rtol=1e-5, atol=1e-5)


def test_pair_scores_index_placement_einsum(orc):
    cand, U, last, E, h, wa, wb, wh = _rand_inputs(seed=7)
    S, inter = orc.pair_scores(cand, U, last, E, h, wa, wb, wh, intermediates=True)
    Ed, Wa, Wb, Wh = (t.double().numpy() for t in (E, wa, wb, wh))
    A = Ed @ Wa.T
    Bm = Ed @ Wb.T
    H = h.double().numpy() @ Wh.T
    c = cand.numpy()
    B_, T, K = c.shape
    for b in range(B_):
        for t in range(T):
            pred = A[[last[b]]] if t == 0 else A[c[b, t - 1]]
            bil = np.einsum("ir,r,jr->ij", pred, H[b, t], Bm[c[b, t]])
            ref = U[b, t].double().numpy()[None, :] + bil
            np.testing.assert_allclose(S[b, t, : pred.shape[0]], ref.astype(np.float32), rtol=1e-6,
                                       atol=1e-6)
    np.testing.assert_allclose(inter["a_last"], A[last.numpy()].astype(np.float32), rtol=1e-6)
    np.testing.assert_allclose(inter["h"], H.astype(np.float32), rtol=1e-6, atol=1e-7)


def test_tiny_workload_scores_shape_and_mask(orc):
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, _, _ = synth.drafter_logits(w)
    idx, val = orc.topk(z, w.K)
    E = synth.embeddings(w)
    wa, wb, wh = synth.selector_weights(w)
    S = orc.pair_scores(idx, val, synth.last_tokens(w), E, synth.context_hidden(w), wa, wb, wh)
    assert S.shape == (1, 3, 4, 4)
    assert np.all(np.isneginf(S[:, 0, 1:]))
    assert np.all(np.isfinite(S[:, 0, 0])) and np.all(np.isfinite(S[:, 1:]))

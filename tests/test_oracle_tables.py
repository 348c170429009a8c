"""Pins for the oracle's per-token selector tables and the pair scores read
from them.

* tables: with one-hot embeddings (E = I) the table row of token v is column
  v of W_A next to column v of W_B, exactly -- a transposed operand or
  swapped halves fail;
* pair scores from a table: equal to the C oracle's pair scores from the
  embedding table (an independent implementation, pinned on its own) up to
  the table's rounding to float32; H = 0 reduces them to the drafter's
  logits; a hand-built table with an asymmetric match (A(v) = e_{v mod r},
  B(v) = 2 e_{(v+1) mod r}) and H = 1/2 (sigmoid of a zero projection) makes
  the bigram a lookup known by inspection, which fixes which side is the
  predecessor; ids outside the vocabulary read zero rows.
"""
import numpy as np
import torch


def _bf16(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def _rand_inputs(B=2, T=4, K=5, V=60, d=32, r=8, seed=3):
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


def test_tables_of_one_hot_embeddings_are_the_weight_columns(orc):
    d, r = 24, 8
    g = torch.Generator().manual_seed(11)
    wa = torch.randn(r, d, generator=g).to(torch.bfloat16)
    wb = torch.randn(r, d, generator=g).to(torch.bfloat16)
    E = _bf16(np.eye(d))
    tab = orc.selector_tables(E, wa, wb)
    assert tab.shape == (d, 2 * r)
    np.testing.assert_array_equal(tab[:, :r], wa.double().numpy().T)
    np.testing.assert_array_equal(tab[:, r:], wb.double().numpy().T)
    # a subset of rows is those rows of the whole table
    rows = [5, 0, 23, 5]
    np.testing.assert_array_equal(orc.selector_tables(E, wa, wb, rows=rows), tab[rows])


def test_scores_from_tables_equal_scores_from_embeddings(orc):
    cand, U, last, E, h, wa, wb, wh = _rand_inputs()
    cand[0, 1, 2] = 0
    cand[1, 3, 4] = E.shape[0] - 1
    for gate in (orc.GATE_IDENTITY, orc.GATE_SIGMOID):
        S_emb = orc.pair_scores(cand, U, last, E, h, wa, wb, wh, gate=gate)
        tab = orc.selector_tables(E, wa, wb)
        tab32 = tab.astype(np.float32)
        S_tab = orc.pair_scores_tab(cand, U, last, tab32, h, wh, gate=gate)
        fin = np.isfinite(S_emb)
        assert np.array_equal(fin, np.isfinite(S_tab))
        assert np.all(np.isneginf(S_tab[:, 0, 1:, :]))
        # the table rounded to float32 moves each product by at most 2 u of
        # its size; both results are then rounded to float32 once
        r = wa.shape[0]
        Hm = np.abs(orc.project(h.reshape(-1, h.shape[-1]), wh, gate)).reshape(h.shape[0], h.shape[1], r)
        absA, absB = np.abs(tab[..., :r]), np.abs(tab[..., r:])
        B, T, K = cand.shape
        ci, lt = cand.numpy(), last.numpy()
        for b in range(B):
            for t in range(T):
                preds = absA[[lt[b]]] if t == 0 else absA[ci[b, t - 1]]
                mag = (preds * Hm[b, t]) @ absB[ci[b, t]].T
                got, ref = S_tab[b, t, :len(preds)], S_emb[b, t, :len(preds)]
                bound = 3 * 2.0 ** -24 * mag + 2 * 2.0 ** -24 * np.abs(ref)
                assert np.all(np.abs(got.astype(np.float64) - ref) <= bound + 1e-30)


def test_scores_from_tables_with_zero_gate_are_the_drafter_logits(orc):
    cand, U, last, E, h, wa, wb, wh = _rand_inputs()
    tab = orc.selector_tables(E, wa, wb).astype(np.float32)
    S = orc.pair_scores_tab(cand, U, last, tab, h, torch.zeros_like(wh))
    B, T, K, _ = S.shape
    for t in range(T):
        for i in ([0] if t == 0 else range(K)):
            np.testing.assert_array_equal(S[:, t, i, :], U[:, t, :].numpy())
    assert np.all(np.isneginf(S[:, 0, 1:, :]))


def test_hand_built_table_makes_the_bigram_a_lookup(orc):
    """A(v) = e_{v mod r}, B(v) = 2 e_{(v+1) mod r}; W_H = 0 with the sigmoid
    gate gives H = 1/2.  Then <A(a) . H, B(b)> = 1 exactly when
    a mod r == (b + 1) mod r, else 0: predecessor a and candidate b enter
    asymmetrically."""
    r, V, d = 6, 30, 16
    B, T, K = 2, 4, 5
    tab = np.zeros((V, 2 * r), np.float32)
    tab[np.arange(V), np.arange(V) % r] = 1.0
    tab[np.arange(V), r + (np.arange(V) + 1) % r] = 2.0
    rng = np.random.default_rng(9)
    cand = rng.integers(0, V, size=(B, T, K)).astype(np.int32)
    last = rng.integers(0, V, size=(B,)).astype(np.int32)
    for b in range(B):      # plant a match after the last token and after every first candidate
        cand[b, 0, 2] = (last[b] - 1) % r + r * rng.integers(0, V // r)
        for t in range(1, T):
            cand[b, t, 3] = (cand[b, t - 1, 0] - 1) % r + r * rng.integers(0, V // r)
    U = rng.normal(size=(B, T, K)).astype(np.float32)
    h = torch.randn(B, T, d).to(torch.bfloat16)
    wh = torch.zeros(r, d, dtype=torch.bfloat16)
    S = orc.pair_scores_tab(cand, U, last, tab, h, wh, gate=orc.GATE_SIGMOID)
    hits = 0
    for b in range(B):
        for t in range(T):
            preds = [last[b]] if t == 0 else list(cand[b, t - 1])
            for i, a in enumerate(preds):
                for j in range(K):
                    want = U[b, t, j] + (1.0 if a % r == (cand[b, t, j] + 1) % r else 0.0)
                    hits += a % r == (cand[b, t, j] + 1) % r
                    assert S[b, t, i, j] == np.float32(want)
    assert hits >= B * T


def test_ids_outside_the_vocabulary_read_zero_rows(orc):
    cand, U, last, E, h, wa, wb, wh = _rand_inputs()
    tab = orc.selector_tables(E, wa, wb).astype(np.float32)
    cand[0, 2, 1] = 10_000
    cand[1, 1, 3] = -1
    last[1] = -7
    S = orc.pair_scores_tab(cand, U, last, tab, h, wh)
    np.testing.assert_array_equal(S[0, 2, :, 1], np.full(S.shape[2], U[0, 2, 1].item(), np.float32))
    np.testing.assert_array_equal(S[0, 3, 1, :], U[0, 3, :].numpy())        # as predecessor
    np.testing.assert_array_equal(S[1, 1, :, 3], np.full(S.shape[2], U[1, 1, 3].item(), np.float32))
    np.testing.assert_array_equal(S[1, 0, 0, :], U[1, 0, :].numpy())        # last token

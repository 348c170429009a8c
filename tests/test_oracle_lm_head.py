"""Pins for the oracle's drafter LM head + top-K (oracle.lm_head_topk).

The drafter reuses the target's embedding and LM head ("大模型推理，加速王者：
DFlash", paragraph before the three-step pipeline); the selector takes its
top-k candidates from that dense head ("DFlash 2 讓 Qwen3.8-27B 快了兩倍",
"坑 2"-"坑 4").  The logits z[r, v] = <h_r, E_v> are checked against cases
whose answer is known without the oracle's own arithmetic:
  * one-hot embedding rows E_v = c_v e_{p(v)}: every logit is one entry of h
    times c_v (an exact product), with the best tokens pointing at the LAST
    coordinate so that a dropped final term shows;
  * a permutation of E's rows permutes the selected indices;
  * scaling h by a power of two scales the logits exactly;
  * small-integer inputs, whose logits are exact in float: the same result
    as the pinned oracle.topk on those logits."""
import numpy as np
import torch

import oracle


def _bf16(a):
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16)


def test_one_hot_rows_give_entries_of_h():
    rng = np.random.default_rng(0)
    rows, d, V, k = 3, 96, 700, 16
    hn = np.clip(rng.normal(size=(rows, d)), -1.5, 1.5)
    hn[:, d - 1] = 8.0       # the last coordinate: c_v * 8 >= 4 beats every other logit (<= 3)
    h = _bf16(hn)
    hf = h.float().numpy().astype(np.float64)
    p = rng.integers(0, d - 1, size=V)
    p[::7] = d - 1                                   # many tokens read the last coordinate
    c = np.round(rng.uniform(0.5, 2.0, size=V) * 8) / 8     # exact in bf16
    E = np.zeros((V, d), np.float32)
    E[np.arange(V), p] = c
    idx, val = oracle.lm_head_topk(h, _bf16(E), k)
    for r in range(rows):
        z = c * hf[r, p]                            # exact products
        order = sorted(range(V), key=lambda v: (-z[v], v))[:k]
        assert idx[r].tolist() == order
        assert np.array_equal(val[r], z[order])
    # the selected tokens read coordinate d - 1: a dropped last term changes them
    assert all(p[idx[r, 0]] == d - 1 for r in range(rows))


def test_row_permutation_permutes_indices():
    rng = np.random.default_rng(1)
    rows, d, V, k = 4, 64, 500, 16
    h = _bf16(rng.normal(size=(rows, d)))
    E = _bf16(rng.normal(size=(V, d)) * 0.05)
    idx, val = oracle.lm_head_topk(h, E, k)
    perm = rng.permutation(V)                        # new row j holds old row perm[j]
    inv = np.argsort(perm)
    idx2, val2 = oracle.lm_head_topk(h, E[torch.from_numpy(perm)], k)
    assert np.array_equal(perm[idx2], idx)           # continuous values: no ties
    assert np.array_equal(val2, val)
    assert np.array_equal(idx2, inv[idx])


def test_scaling_h_by_two_scales_logits():
    rng = np.random.default_rng(2)
    h = _bf16(rng.normal(size=(2, 128)))
    E = _bf16(rng.normal(size=(300, 128)) * 0.05)
    idx, val = oracle.lm_head_topk(h, E, 8)
    idx2, val2 = oracle.lm_head_topk(_bf16(2 * h.float().numpy()), E, 8)
    assert np.array_equal(idx2, idx)
    assert np.array_equal(val2, 2 * val)


def test_integer_logits_agree_with_topk():
    """Entries in {-3..3}: every logit is an integer below 2^24, exact in
    float, so the LM head's selection is oracle.topk's on those logits
    (ties, which are frequent, included)."""
    rng = np.random.default_rng(3)
    rows, d, V = 5, 40, 900
    h = rng.integers(-3, 4, size=(rows, d)).astype(np.float32)
    E = rng.integers(-3, 4, size=(V, d)).astype(np.float32)
    idx, val = oracle.lm_head_topk(_bf16(h), _bf16(E), 16)
    z = (h.astype(np.int64) @ E.astype(np.int64).T).astype(np.float32)
    ti, tv = oracle.topk(z, 16)
    assert np.array_equal(idx, ti)
    assert np.array_equal(val, tv.astype(np.float64))


# ------------------------------------------------ greedy verification from the head
def test_verify_greedy_head_equals_verify_greedy_on_exact_logits():
    """Integer inputs: the target logits are exact, so verifying from the
    hidden states equals oracle.verify_greedy on the logits themselves
    (argmax ties, frequent here, to the lower id)."""
    rng = np.random.default_rng(6)
    B, T, V, d = 6, 5, 400, 24
    h = rng.integers(-3, 4, size=(B, T + 1, d)).astype(np.float32)
    E = rng.integers(-3, 4, size=(V, d)).astype(np.float32)
    Z = (h.astype(np.int64) @ E.astype(np.int64).T).astype(np.float32)
    y = np.argmax(Z, -1)
    path = y[:, :T].copy().astype(np.int32)
    path[1, 2] = (path[1, 2] + 1) % V
    path[3, 0] = (path[3, 0] + 7) % V
    o = oracle.verify_greedy_head(_bf16(h), _bf16(E), path)
    g = oracle.verify_greedy(Z, path)
    assert np.array_equal(o["argmax"], g["argmax"])
    assert np.array_equal(o["accept_len"], g["accept_len"])
    assert np.array_equal(o["out_tok"], g["out_tok"])
    assert o["accept_len"].tolist() == [T, 2, T, 0, T, T]


def test_verify_greedy_head_one_hot_head():
    """E_v = e_{v mod d} scaled by 1 + v / V: the logit of v is h[v mod d]
    (1 + v / V), so each row's argmax is known by inspection; the emitted
    tokens are that argmax chain."""
    B, T, d = 2, 3, 32
    V = 4 * d
    E = np.zeros((V, d), np.float32)
    scale = 1 + np.round(np.arange(V) / V * 64) / 64     # exact in bf16
    E[np.arange(V), np.arange(V) % d] = scale
    rng = np.random.default_rng(7)
    h = np.round(rng.normal(size=(B, T + 1, d)) * 16) / 16
    want = np.zeros((B, T + 1), np.int64)
    for b in range(B):
        for t in range(T + 1):
            z = h[b, t, np.arange(V) % d] * scale
            want[b, t] = min(range(V), key=lambda v: (-z[v], v))
    path = want[:, :T].astype(np.int32)
    o = oracle.verify_greedy_head(_bf16(h), _bf16(E), path)
    assert np.array_equal(o["argmax"], want)
    assert o["accept_len"].tolist() == [T, T]
    assert np.array_equal(o["out_tok"], want)


def test_verify_reject_head_equals_verify_reject_on_exact_logits():
    """Integer inputs: the target logits are exact in float, so rejection
    verification from the hidden states draws the same uniforms and decides
    exactly as oracle.verify_reject on the logits (sampled proposals, mixed
    accepted lengths, resampled and bonus tokens)."""
    rng = np.random.default_rng(11)
    B, T, K, V, d = 40, 4, 4, 60, 16
    h = rng.integers(-2, 3, size=(B, T + 1, d)).astype(np.float32)
    E = rng.integers(-1, 2, size=(V, d)).astype(np.float32)
    Z = (h.astype(np.int64) @ E.astype(np.int64).T).astype(np.float32)
    # candidates: each position's K best target tokens (so drafts are often accepted)
    cand = np.argsort(-Z[:, :T, :], axis=-1, kind="stable")[..., :K].astype(np.int32)
    q = rng.dirichlet(np.ones(K), size=(B, T)).astype(np.float32)
    rank = np.array([[rng.choice(K, p=q[b, t] / q[b, t].sum()) for t in range(T)] for b in range(B)],
                    np.int32)
    tok = np.take_along_axis(cand, rank[..., None], -1)[..., 0].astype(np.int32)
    for tau in (1.0, 0.5):
        o = oracle.verify_reject_head(_bf16(h), _bf16(E), tok, rank, cand, q, tau, 21, b_ids=np.arange(B) + 3)
        g = oracle.verify_reject(Z, tok, rank, cand, q, tau, 21, b_ids=np.arange(B) + 3)
        assert np.array_equal(o["accept_len"], g["accept_len"])
        assert np.array_equal(o["out_tok"], g["out_tok"])
        assert len(set(o["accept_len"].tolist())) >= 3

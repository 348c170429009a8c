"""GPU parity of dflash2_lm_head_topk (drafter logits through the shared LM
head, fused with the top-K) against the oracle (oracle.lm_head_topk: float64
logits, then the K best by value desc, index asc).

The GPU sums bf16 products in fp32, the oracle in float64, so the two can
order a pair of tokens differently only when their logits are closer than
the fp32 rounding error.  Rule (for every row and rank i):
  * value: |val_g[i] - z64[idx_g[i]]| <= eps[idx_g[i]], with
    eps[v] = 8 sqrt(d) u sum_k |h_k E_vk| (u = 2^-24): the probabilistic
    bound of an fp32 sum of d terms (Higham and Mary, "A new approach to
    probabilistic rounding error analysis", 2019; lambda = 8, failure
    probability below 1e-13 per logit);
  * index: idx_g[i] == idx_o[i], or the two tokens' float64 logits differ by
    at most eps_g + eps_o (the i-th largest of two sequences within eps of
    each other are within eps of each other); such near-ties are counted and
    must stay rare.
Small-integer inputs make every logit exact in fp32 and float64: there the
result must be bit-identical, ties (frequent) included.

dflash2_verify_greedy_head (greedy verification with the target's LM head
fused in) is compared with oracle.verify_greedy_head the same way: accepted
lengths and emitted tokens exact, except for a request whose deciding
argmax had a top-2 gap within twice the fp32 bound."""
import numpy as np
import pytest
import torch

import draft_selection_bf16_amd as df2
import oracle
import synth
from gpu_util import DEV, report, ws

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

U32 = 2.0 ** -24


def _gpu(h, E, k):
    rows, d = h.shape
    idx = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    val = torch.empty((rows, k), dtype=torch.float32, device=DEV)
    w = ws(df2.dflash2_lm_head_topk_workspace_bytes(rows, E.shape[0], d, k))
    df2.dflash2_lm_head_topk(h.to(DEV), E.to(DEV), k, idx, val, w)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def _check(h, E, k, rows, gi, gv, label):
    """Compare GPU rows `rows` (gi, gv: all rows) with the oracle on those rows."""
    hs = h[torch.as_tensor(rows)]
    oi, ov = oracle.lm_head_topk(hs, E, k)
    d = h.shape[1]
    hf = hs.float().numpy().astype(np.float64)
    near, n = 0, 0
    for j, r in enumerate(rows):
        toks = np.union1d(gi[r], oi[j])
        Et = E[torch.from_numpy(toks.astype(np.int64))].float().numpy().astype(np.float64)
        z = dict(zip(toks.tolist(), (Et @ hf[j]).tolist()))
        eps = dict(zip(toks.tolist(), (8 * np.sqrt(d) * U32 * (np.abs(Et) @ np.abs(hf[j]))).tolist()))
        for i in range(k):
            g, o = int(gi[r, i]), int(oi[j, i])
            assert abs(float(gv[r, i]) - z[g]) <= eps[g], (label, r, i, float(gv[r, i]), z[g], eps[g])
            n += 1
            if g != o:
                assert abs(z[g] - z[o]) <= eps[g] + eps[o], (label, r, i, g, o, z[g], z[o])
                near += 1
        assert np.isclose(ov[j, 0], z[int(oi[j, 0])])
    assert near <= max(2, n // 50), (label, near, n)
    report(f"lm_head_topk {label}", rows=len(rows), near_tie_swaps=near)


def _inputs(rows, V, d, seed, scale_h=1.0):
    g = torch.Generator().manual_seed(seed)
    h = (scale_h * torch.randn(rows, d, generator=g)).to(torch.bfloat16)
    E = (0.02 * torch.randn(V, d, generator=g)).to(torch.bfloat16)
    return h, E


@pytest.mark.parametrize("rows,V,d,k", [(133, 5003, 640, 16), (1, 131, 64, 16), (7, 20011, 256, 16),
                                        (300, 2500, 128, 5), (64, 17, 192, 16), (260, 1000, 64, 1),
                                        (1100, 3001, 128, 16)])
def test_lm_head_topk_small_shapes(rows, V, d, k):
    """Every row-tile height: 64 rows (1, 7, 64), 128 (260, 300), 256 (133:
    one ragged block; 1,100: five blocks, the last ragged, 48 token ranges);
    a ragged last token block, fewer tokens than one block (17, 131), k < 16,
    d from 64 to 640; every row checked."""
    print(f"[case] lm_head_topk rows={rows} V={V} d={d} k={k}", flush=True)
    h, E = _inputs(rows, V, d, rows + V)
    gi, gv = _gpu(h, E, k)
    _check(h, E, k, list(range(rows)), gi, gv, f"{rows}x{V}x{d}")


def test_lm_head_topk_integer_inputs_bit_exact():
    """Entries in {-3..3}: every logit is an integer, exact in fp32 and in
    float64, with many ties; indices and values must be identical, ties
    going to the lower token id."""
    rng = np.random.default_rng(5)
    rows, V, d = 150, 3001, 256
    h = torch.from_numpy(rng.integers(-3, 4, size=(rows, d)).astype(np.float32)).to(torch.bfloat16)
    E = torch.from_numpy(rng.integers(-3, 4, size=(V, d)).astype(np.float32)).to(torch.bfloat16)
    gi, gv = _gpu(h, E, 16)
    oi, ov = oracle.lm_head_topk(h, E, 16)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.astype(np.float64), ov)


def test_lm_head_topk_b32_blk16_launch_shape():
    """480 rows (32 requests x 15 draft positions), vocabulary 151,936,
    hidden 5120: the launch configuration the benchmark times.  The oracle
    recomputes sampled rows one by one: the first and last of each 128-row
    block and two more."""
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    rows, V, d = w.B * w.T, w.V, w.d
    print(f"[case] lm_head_topk rows={rows} V={V} d={d}", flush=True)
    E = synth.embeddings(w, device=DEV)
    h = synth.context_hidden(w, device=DEV).reshape(rows, d)
    gi, gv = _gpu(h, E, 16)
    assert np.all(np.diff(gv, axis=1) <= 0)
    sample = [0, 127, 128, 255, 256, 383, 384, 479, 77, 301]
    _check(h.cpu(), E.cpu(), 16, sample, gi, gv, "480x151936x5120")


def test_lm_head_topk_b1_blk8_launch_shape():
    """7 rows (one request, block 8), vocabulary 151,936: a skinny product
    that streams the whole LM head; every row checked."""
    w = synth.WORKLOADS["b1_blk8_v151936"]
    rows, V, d = w.T, w.V, w.d
    E = synth.embeddings(w, device=DEV)
    h = synth.context_hidden(w, device=DEV).reshape(rows, d)
    gi, gv = _gpu(h, E, 16)
    _check(h.cpu(), E.cpu(), 16, list(range(rows)), gi, gv, "7x151936x5120")


# ------------------------------------------------ greedy verification from the head
def _verify_head_gpu(h, E, path):
    B, T1, d = h.shape
    acc = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, T1), dtype=torch.int32, device=DEV)
    w = ws(df2.dflash2_verify_greedy_head_workspace_bytes(B, T1 - 1, E.shape[0], d))
    df2.dflash2_verify_greedy_head(h.to(DEV), E.to(DEV), path.to(DEV), acc, out, w)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def _paths_from_chain(y, T, seed):
    """Drafts equal to the target's argmax chain up to a planted mismatch at
    a random position (or none), so every accepted length occurs."""
    rng = np.random.default_rng(seed)
    B = y.shape[0]
    path = y[:, :T].astype(np.int32).copy()
    cut = rng.integers(0, T + 1, size=B)
    for b in range(B):
        if cut[b] < T:
            path[b, cut[b]] = (path[b, cut[b]] + 1 + rng.integers(0, 1000)) % 151936
    return torch.from_numpy(path), cut


def _check_verify_head(h, E, path, ga, go, reqs, label):
    """reqs: request indices to recompute with the oracle.  Exact unless a
    row's argmax had a near-tie (top-2 gap within twice the fp32 bound)."""
    hs = h[torch.as_tensor(reqs)]
    o = oracle.verify_greedy_head(hs, E, path[torch.as_tensor(reqs)])
    d = h.shape[-1]
    emax = float(E.float().abs().max())
    near = 0
    for j, b in enumerate(reqs):
        if ga[b] == o["accept_len"][j] and np.array_equal(go[b], o["out_tok"][j]):
            continue
        hb = hs[j].float().numpy().astype(np.float64)
        eps = 8 * np.sqrt(d) * U32 * np.abs(hb).sum(-1) * emax      # per row, an upper bound of the fp32 bound
        n = min(int(ga[b]), int(o["accept_len"][j]))
        assert o["margin"][j, n] <= 2 * eps[n], (label, b, int(ga[b]), int(o["accept_len"][j]))
        near += 1
    report(f"verify_greedy_head {label}", requests=len(reqs), near_tie_rows=near,
           mean_accept=float(np.mean(ga[reqs])))
    assert near <= max(1, len(reqs) // 8)


@pytest.mark.parametrize("B,T,V,d", [(3, 7, 5003, 640), (5, 15, 2049, 128), (2, 1, 300, 64), (25, 7, 3001, 128)])
def test_verify_greedy_head_small(B, T, V, d):
    """Rows B (T + 1) = 24 and 4 (64-row tiles), 80 (128), 200 (one ragged
    256-row block)."""
    g = torch.Generator().manual_seed(B * 100 + T)
    h = torch.randn(B, T + 1, d, generator=g).to(torch.bfloat16)
    E = (0.02 * torch.randn(V, d, generator=g)).to(torch.bfloat16)
    y = oracle.verify_greedy_head(h, E, torch.zeros(B, T, dtype=torch.int32))["argmax"]
    path, _ = _paths_from_chain(y, T, B)
    path = path % V
    ga, go = _verify_head_gpu(h, E, path)
    _check_verify_head(h, E, path, ga, go, list(range(B)), f"B{B}T{T}V{V}d{d}")


def test_verify_greedy_head_integer_inputs_bit_exact():
    """Exact logits with frequent argmax ties (lowest id wins on both sides)."""
    rng = np.random.default_rng(8)
    B, T, V, d = 4, 7, 2000, 128
    h = torch.from_numpy(rng.integers(-2, 3, size=(B, T + 1, d)).astype(np.float32)).to(torch.bfloat16)
    E = torch.from_numpy(rng.integers(-2, 3, size=(V, d)).astype(np.float32)).to(torch.bfloat16)
    y = oracle.verify_greedy_head(h, E, torch.zeros(B, T, dtype=torch.int32))["argmax"]
    path, _ = _paths_from_chain(y, T, 9)
    path = path % V
    ga, go = _verify_head_gpu(h, E, path)
    o = oracle.verify_greedy_head(h, E, path)
    assert np.array_equal(ga, o["accept_len"]) and np.array_equal(go, o["out_tok"])


def test_verify_greedy_head_b32_blk16_launch_shape():
    """32 requests x 16 verified rows, vocabulary 151,936, hidden 5120 (the
    launch shape of the batch-32, block-16 cycle); requests 0 and 31
    recomputed by the oracle, with drafts built from its argmax chain."""
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    B, T, V, d = w.B, w.T, w.V, w.d
    print(f"[case] verify_greedy_head B={B} T={T} V={V} d={d}", flush=True)
    E = synth.embeddings(w, device=DEV)
    g = torch.Generator().manual_seed(31)
    h = torch.randn(B, T + 1, d, generator=g).to(torch.bfloat16)
    reqs = [0, 31]
    Ec = E.cpu()
    y = np.zeros((B, T + 1), np.int64)
    y[reqs] = oracle.verify_greedy_head(h[reqs], Ec, torch.zeros(2, T, dtype=torch.int32))["argmax"]
    path, _ = _paths_from_chain(y, T, 10)
    ga, go = _verify_head_gpu(h, E, path)
    _check_verify_head(h, Ec, path, ga, go, reqs, "B32T15V151936")


def test_verify_greedy_head_b1_blk8_launch_shape():
    w = synth.WORKLOADS["b1_blk8_v151936"]
    B, T, V, d = w.B, w.T, w.V, w.d
    E = synth.embeddings(w, device=DEV)
    g = torch.Generator().manual_seed(32)
    h = torch.randn(B, T + 1, d, generator=g).to(torch.bfloat16)
    Ec = E.cpu()
    y = oracle.verify_greedy_head(h, Ec, torch.zeros(B, T, dtype=torch.int32))["argmax"]
    path = torch.from_numpy(y[:, :T].astype(np.int32))          # all drafts accepted: the bonus row counts
    ga, go = _verify_head_gpu(h, E, path)
    _check_verify_head(h, Ec, path, ga, go, [0], "B1T7V151936")
    assert ga[0] == T

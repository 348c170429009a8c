"""GPU parity of dflash2_verify_reject_head (rejection verification with the
target's LM head fused in) against the oracle (oracle.verify_reject_head:
float64 logits h E^T, float64 probabilities, the same Philox uniforms).

The GPU's logits are fp32 sums of bf16 products; each is within
eps = 8 sqrt(d) u max_v sum_k |h_k E_vk| of the float64 logit (u = 2^-24;
the probabilistic bound of Higham and Mary, "A new approach to
probabilistic rounding error analysis", 2019, with lambda = 8, taken at the
row's largest term sum).  A probability p = exp((z - lse) / tau) then moves
by a factor within exp(+-2 eps / tau), plus fp32 rounding (~1e-6), so:
  * an accept decision (u1 < p / q) may come out differently only where the
    oracle's |u1 - p/q| is at most 2.5 eps / tau * max(1, p/q) + 1e-6;
  * a residual or bonus draw only where the oracle's distance of u2 * mass
    to the nearest token boundary (relative to the mass) is at most
    6 eps / tau + 1e-6 (partial and total masses both move, and the block
    search and the in-block walk see logits from two summation orders).
Only the first decision where the two runs part is excused (the rest follows
from it); every other request must match exactly.  Small-integer inputs make
the logits exact on both sides: there only fp32 probability rounding
(NEAR_TIE = 1e-6) may excuse a difference."""
import numpy as np
import pytest
import torch

import draft_selection_bf16_amd as df2
import oracle
import synth
from gpu_util import DEV, NEAR_TIE, report, ws

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

U32 = 2.0 ** -24


def _gpu(h, E, tok, rank, cand, q, tau, seed, b0=0):
    B, T1, d = h.shape
    K = cand.shape[-1]
    acc = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, T1), dtype=torch.int32, device=DEV)
    w = ws(df2.dflash2_verify_reject_head_workspace_bytes(B, T1 - 1, E.shape[0], d, K))
    sd = torch.tensor([seed], dtype=torch.int64, device=DEV)
    t = lambda a: torch.as_tensor(np.ascontiguousarray(a)).to(DEV)
    df2.dflash2_verify_reject_head(h.to(DEV), E.to(DEV), t(tok), t(rank), t(cand), t(q), tau, sd, acc, out, w,
                                   b0=b0)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def _chunks(E, step=8192):
    """E [V, d] bf16 in float64 row chunks (never the whole table at once)."""
    for v0 in range(0, E.shape[0], step):
        yield v0, E[v0:v0 + step].float().numpy().astype(np.float64)


def _logits64(hrows, E):
    """float64 logits [R, V] of hidden rows [R, d]."""
    H = hrows.float().numpy().astype(np.float64)
    return np.concatenate([H @ Ec.T for _, Ec in _chunks(E)], axis=1)


def _drafts(h, E, reqs, K, tau, seed, V):
    """Candidates, proposal and drafted path per request.  For the requests
    in `reqs` the candidates are the target's own top-K (float64 logits) and
    q a perturbed softmax over them, so that acceptance varies from none to
    all; the other requests get random candidates."""
    B, T1, d = h.shape
    T = T1 - 1
    rng = np.random.default_rng(seed)
    cand = np.zeros((B, T, K), np.int32)
    for b in range(B):
        for t in range(T):
            cand[b, t] = rng.choice(V, size=K, replace=False)
    logit = rng.normal(size=(B, T, K))
    for b in reqs:
        z = _logits64(h[b, :T], E)                                  # [T, V]
        top = np.argsort(-z, axis=1, kind="stable")[:, :K]
        cand[b] = top
        logit[b] = np.take_along_axis(z, top, 1) / tau + 0.3 * rng.normal(size=(T, K))
    q = np.exp(logit - logit.max(-1, keepdims=True))
    q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
    rank = np.zeros((B, T), np.int32)
    for b in range(B):
        for t in range(T):
            pr = q[b, t].astype(np.float64)
            rank[b, t] = rng.choice(K, p=pr / pr.sum())
    tok = np.take_along_axis(cand, rank[..., None], -1)[..., 0].astype(np.int32)
    return tok, rank, cand, q


def _row_eps(h, E):
    """eps per row of h [R, d]: the fp32 bound at the row's largest term sum."""
    d = h.shape[-1]
    Ha = np.abs(h.float().numpy().astype(np.float64)).reshape(-1, d)
    S = np.zeros(Ha.shape[0])
    for _, Ec in _chunks(E):
        S = np.maximum(S, (np.abs(Ec) @ Ha.T).max(0))
    return 8 * np.sqrt(d) * U32 * S


def _check(h, E, tok, rank, cand, q, tau, seed, ga, go, reqs, label, exact_logits=False):
    """Compare GPU requests `reqs` (ga, go: all requests) with the oracle run
    on those requests with their batch indices as counters."""
    r = np.asarray(reqs)
    hs = h[torch.as_tensor(r)]
    o = oracle.verify_reject_head(hs, E, tok[r], rank[r], cand[r], q[r], tau, seed, b_ids=r.astype(np.int32))
    T = tok.shape[1]
    eps = np.zeros((len(r), T + 1)) if exact_logits else _row_eps(hs, E).reshape(len(r), T + 1)
    near = 0
    for j, b in enumerate(r):
        na, no = int(ga[b]), int(o["accept_len"][j])
        if na == no and np.array_equal(go[b], o["out_tok"][j]):
            continue
        if na != no:   # an accept decision at min(na, no)
            t = min(na, no)
            ma = float(o["margin_accept"][j, t])
            tol = 2.5 * eps[j, t] / tau * (1.0 + ma) + NEAR_TIE     # p/q < u1 + ma < 1 + ma
            assert ma <= tol, (label, int(b), "accept", t, na, no, ma, tol)
        else:          # the draw at row n
            ms = float(o["margin_sample"][j])
            tol = 6 * eps[j, na] / tau + NEAR_TIE
            assert ms <= tol, (label, int(b), "draw", na, int(go[b, na]), int(o["out_tok"][j, na]), ms, tol)
        near += 1
    report(f"verify_reject_head {label}", requests=len(r), near_tie=near,
           mean_accept=float(np.mean(o["accept_len"])), fallbacks=o["fallbacks"])
    assert near <= max(1, len(r) // 8), (label, near)
    return o


def _hidden(B, T, E, seed):
    """Target hidden states N(0, 1) plus a planted direction a E_y / |E_y|^2
    towards one random token y per row, a uniform in [2, 16]: the logit of y
    stands a above the rest's spread, so rows range from flat to a single
    dominant token and acceptance from none to all."""
    V, d = E.shape
    g = torch.Generator().manual_seed(seed)
    y = torch.randint(0, V, (B * (T + 1),), generator=g)
    a = 2.0 + 14.0 * torch.rand(B * (T + 1), 1, generator=g)
    Ey = E[y.to(E.device)].float().cpu()
    dirn = Ey / (Ey * Ey).sum(-1, keepdim=True).clamp_min(1e-12)
    h = torch.randn(B * (T + 1), d, generator=g) + a * dirn
    return h.reshape(B, T + 1, d).to(torch.bfloat16)


@pytest.mark.parametrize("B,T,V,d,K,tau", [(4, 7, 5003, 640, 16, 1.0), (5, 15, 2049, 128, 16, 0.7),
                                           (2, 1, 300, 64, 5, 1.3), (3, 3, 129, 64, 16, 1.0),
                                           (6, 7, 20011, 256, 8, 0.5), (25, 7, 3001, 128, 16, 0.8)])
def test_verify_reject_head_small(B, T, V, d, K, tau):
    """Rows B (T + 1) up to 64 (64-row tiles), 80 (128), 200 (one ragged
    256-row block)."""
    g = torch.Generator().manual_seed(B * 100 + T)
    E = (0.02 * torch.randn(V, d, generator=g)).to(torch.bfloat16)
    h = _hidden(B, T, E, B * 7 + T)
    seed = 11 + B
    tok, rank, cand, q = _drafts(h, E, range(B), K, tau, seed, V)
    ga, go = _gpu(h, E, tok, rank, cand, q, tau, seed)
    o = _check(h, E, tok, rank, cand, q, tau, seed, ga, go, list(range(B)), f"B{B}T{T}V{V}d{d}K{K}")
    # emitted tokens are valid ids, -1 after the draw
    for b in range(B):
        n = int(ga[b])
        assert 0 <= n <= T and (go[b, : n + 1] >= 0).all() and (go[b, : n + 1] < V).all()
        assert (go[b, n + 1:] == -1).all() and np.array_equal(go[b, :n], tok[b, :n])


def test_verify_reject_head_integer_inputs():
    """Exact logits (small integers): only probability rounding may excuse."""
    rng = np.random.default_rng(21)
    B, T, V, d, K, tau = 6, 7, 1000, 128, 16, 2.0
    h = torch.from_numpy(rng.integers(-1, 2, size=(B, T + 1, d)).astype(np.float32)).to(torch.bfloat16)
    E = torch.from_numpy(rng.integers(-1, 2, size=(V, d)).astype(np.float32)).to(torch.bfloat16)
    tok, rank, cand, q = _drafts(h, E, range(B), K, tau, 4, V)
    ga, go = _gpu(h, E, tok, rank, cand, q, tau, 4)
    _check(h, E, tok, rank, cand, q, tau, 4, ga, go, list(range(B)), "integer", exact_logits=True)


def test_verify_reject_head_sub_ranges_draw_the_batch_counters():
    """Two calls over requests 0-2 (b0 = 0) and 3-7 (b0 = 3) give what one
    call over the batch gives."""
    B, T, V, d, K, tau, seed = 8, 7, 3001, 128, 16, 1.0, 9
    g = torch.Generator().manual_seed(5)
    E = (0.02 * torch.randn(V, d, generator=g)).to(torch.bfloat16)
    h = _hidden(B, T, E, 6)
    tok, rank, cand, q = _drafts(h, E, range(B), K, tau, seed, V)
    full = _gpu(h, E, tok, rank, cand, q, tau, seed)
    lo = _gpu(h[:3].contiguous(), E, tok[:3], rank[:3], cand[:3], q[:3], tau, seed, b0=0)
    hi = _gpu(h[3:].contiguous(), E, tok[3:], rank[3:], cand[3:], q[3:], tau, seed, b0=3)
    assert np.array_equal(np.concatenate([lo[0], hi[0]]), full[0])
    assert np.array_equal(np.concatenate([lo[1], hi[1]]), full[1])


def test_verify_reject_head_distribution():
    """Many copies of one request: the first emitted token follows p_0 (drafts
    drawn from q over 4 candidates; acceptance plus residual restore p)."""
    N, T, V, d, K, tau = 16384, 2, 200, 64, 4, 1.0
    g = torch.Generator().manual_seed(3)
    E = (0.25 * torch.randn(V, d, generator=g)).to(torch.bfloat16)
    h1 = (0.6 * torch.randn(1, T + 1, d, generator=g)).to(torch.bfloat16)
    z0 = _logits64(h1[0, :1], E)[0]
    p0 = np.exp((z0 - z0.max()) / tau)
    p0 /= p0.sum()
    rng = np.random.default_rng(3)
    cands = np.stack([np.argsort(-z0)[:K], rng.choice(V, K, replace=False)]).astype(np.int32)
    qrow = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]], np.float32)
    rank = np.stack([rng.choice(K, size=N, p=qrow[t] / qrow[t].sum()) for t in range(T)], 1).astype(np.int32)
    tok = np.take_along_axis(np.broadcast_to(cands, (N, T, K)), rank[..., None], -1)[..., 0].astype(np.int32)
    h = h1.expand(N, T + 1, d).contiguous()
    ga, go = _gpu(h, E, tok, rank, np.broadcast_to(cands, (N, T, K)), np.broadcast_to(qrow, (N, T, K)), tau, 17)
    counts = np.bincount(go[:, 0], minlength=V).astype(float)
    e = N * p0
    keep = e > 5
    chi2 = float((((counts - e) ** 2) / e)[keep].sum() + ((counts[~keep].sum() - e[~keep].sum()) ** 2)
                 / max(e[~keep].sum(), 1e-9))
    report("verify_reject_head MC", chi2=round(chi2, 1), dof=int(keep.sum()))
    assert chi2 < int(keep.sum()) + 1 + 8 * np.sqrt(2 * (keep.sum() + 1))


def test_verify_reject_head_b32_blk16_launch_shape():
    """32 requests x 16 verified rows, vocabulary 151,936, hidden 5120 (the
    launch shape of the batch-32, block-16 cycle); requests 0, 17 and 31
    recomputed by the oracle with their batch counters."""
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    B, T, V, d, K, tau = w.B, w.T, w.V, w.d, 16, 1.0
    print(f"[case] verify_reject_head B={B} T={T} V={V} d={d}", flush=True)
    E = synth.embeddings(w, device=DEV)
    Ec = E.cpu()
    h = _hidden(B, T, E, 41)
    reqs = [0, 17, 31]
    tok, rank, cand, q = _drafts(h, Ec, reqs, K, tau, 12, V)
    ga, go = _gpu(h, E, tok, rank, cand, q, tau, 12)
    _check(h, Ec, tok, rank, cand, q, tau, 12, ga, go, reqs, "B32T15V151936")


def test_verify_reject_head_b1_blk8_launch_shape():
    w = synth.WORKLOADS["b1_blk8_v151936"]
    B, T, V, d, K, tau = w.B, w.T, w.V, w.d, 16, 0.8
    E = synth.embeddings(w, device=DEV)
    Ec = E.cpu()
    h = _hidden(B, T, E, 42)
    tok, rank, cand, q = _drafts(h, Ec, [0], K, tau, 13, V)
    ga, go = _gpu(h, E, tok, rank, cand, q, tau, 13)
    _check(h, Ec, tok, rank, cand, q, tau, 13, ga, go, [0], "B1T7V151936")

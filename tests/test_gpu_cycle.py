"""GPU parity of whole cycles at the workloads' real sizes, and of the cycle
captured as a HIP graph.

Stages are chained on both sides (GPU: conv -> top-K -> pair scores -> path
-> verify; oracle: the same from the same inputs).  The oracle recomputes a
sample of requests one by one.  Top-K and greedy verification are compared
exactly, conv outputs within 1e-3 of their terms' magnitudes; the path is
compared exactly except where the decision that flipped is one the score
parity cannot decide (tests/path_compare.py: its oracle margin is under
1e-6 plus the allowance the score difference gives for that decision);
such flips are counted, bounded and reported, and the verification of
those requests is checked against the oracle run on the GPU's path."""
import numpy as np
import pytest
import torch

import oracle
import synth
from draft_selection_bf16_amd.cycle import ConvSite, Cycle
from gpu_util import (DEV, NEAR_TIE, bf16_ulp_close, close, conv_close, conv_error_bound, conv_rel_close,
                      conv_rel_close_bf16, conv_term_scale, report)
from path_compare import compare_path

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def build(w, with_conv=None, y_dtype=torch.bfloat16, tables=False):
    """Inputs for workload w on the GPU, and the Cycle that runs them."""
    z, tok, rank = synth.drafter_logits(w, device=DEV)
    Z = synth.target_logits(w, z, tok, device=DEV)
    E = synth.embeddings(w, device=DEV)
    wa, wb, wh = synth.selector_weights(w, device=DEV)
    h = synth.context_hidden(w, device=DEV)
    last = synth.last_tokens(w, device=DEV)
    nsites = w.conv_sites if with_conv is None else with_conv
    sites = []
    for s in range(nsites):
        x, xp, wt, bs = synth.conv_site(w, s, device=DEV)
        sites.append(ConvSite(x, xp, wt, bs, torch.empty(x.shape, dtype=y_dtype, device=DEV)))
    path_mode = "viterbi" if w.path_mode == "both" else w.path_mode
    cyc = Cycle(logits=z, target=Z, emb=E, h=h, w_a=wa, w_b=wb, w_h=wh, last_tok=last, K=w.K,
                path_mode=path_mode, verify=w.verify, tau=w.tau if w.tau > 0 else 1.0,
                conv_sites=sites, seed=w.seed, tables=tables)
    return cyc, dict(tok=tok, rank=rank)


def emb_rows(E, toks):
    uniq, inv = np.unique(np.asarray(toks).ravel(), return_inverse=True)
    sub = E[torch.from_numpy(uniq).to(E.device).long()].cpu()
    return sub, inv.reshape(np.asarray(toks).shape).astype(np.int32)


def oracle_cycle(cyc, rows, w, seed):
    """The oracle's own cycle for the requests in `rows`."""
    z = cyc.logits[rows].cpu()
    idx, val = oracle.topk(z, w.K)
    last = cyc.last_tok[rows].cpu().numpy()
    sub, remap = emb_rows(cyc.emb, np.concatenate([idx.ravel(), last]))
    ridx = remap[: idx.size].reshape(idx.shape)
    rlast = remap[idx.size:]
    S = oracle.pair_scores(ridx, val, rlast, sub, cyc.h[rows].cpu(), cyc.w_a.cpu(), cyc.w_b.cpu(),
                           cyc.w_h.cpu(), gate=cyc.gate)
    return dict(idx=idx, val=val, S=S)


def check_cycle(cyc, w, rows, label, check_conv_sites=(0,)):
    torch.cuda.synchronize()
    o = oracle_cycle(cyc, rows, w, w.seed)
    gi = cyc.cand_idx[rows].cpu().numpy()
    gv = cyc.cand_val[rows].cpu().numpy()
    assert np.array_equal(gi, o["idx"]), "top-K indices"
    assert np.array_equal(gv, o["val"]), "top-K values"
    Sg = cyc.scores[rows].cpu().numpy()
    worst = close(Sg, o["S"])
    mode = {0: oracle.PATH_VITERBI, 1: oracle.PATH_GREEDY, 2: oracle.PATH_SAMPLE}[cyc.path_mode]
    seed = int(cyc.seed.item())
    g_rows = np.array(rows)
    op = oracle.path(o["S"], o["idx"], mode, temperature=cyc.tau, seed=seed, b_ids=g_rows)
    g_rank = cyc.path_rank[rows].cpu().numpy()
    cmp = compare_path(g_rank, op, Sg, o["S"], mode, cyc.tau, w.T)
    assert cmp["bad"] == 0, cmp
    # a flip is rare: at most one checked request in eight may take one
    assert cmp["undecided_flips"] <= max(1, len(rows) // 8), cmp
    # verification: rows whose path equals the oracle's are compared with the
    # oracle's own chain; rows with an excused flip with the oracle's
    # verification run on the GPU's path (and the GPU's proposal q)
    same = np.array([np.array_equal(g_rank[i], op["rank"][i]) for i in range(len(rows))])
    g_tok = cyc.path_tok[rows].cpu().numpy()
    g_q = cyc.q[rows].cpu().numpy()
    v_tok = np.where(same[:, None], op["tok"], g_tok)
    v_rank = np.where(same[:, None], op["rank"], g_rank)
    v_q = np.where(same[:, None, None], op["q"], g_q)
    Z = cyc.target[rows].cpu()
    ga = cyc.accept_len[rows].cpu().numpy()
    go = cyc.out_tok[rows].cpu().numpy()
    greedy = np.ones(len(rows), bool)
    if cyc.verify == "reject":
        greedy[:] = False
    elif cyc.verify == "mixed":
        greedy = g_rows < cyc.greedy_rows
    near_v = 0
    if greedy.any():
        ov = oracle.verify_greedy(Z[greedy], v_tok[greedy])
        assert np.array_equal(ga[greedy], ov["accept_len"])
        assert np.array_equal(go[greedy], ov["out_tok"])
    if (~greedy).any():
        sel = ~greedy
        # Philox counters are keyed by the request's index in the whole batch
        ov = oracle.verify_reject(Z[sel], v_tok[sel], v_rank[sel], o["idx"][sel], v_q[sel],
                                  cyc.tau, seed, b_ids=g_rows[sel])
        for i in range(int(sel.sum())):
            if ga[sel][i] == ov["accept_len"][i] and np.array_equal(go[sel][i], ov["out_tok"][i]):
                continue
            ma = ov["margin_accept"][i]
            assert (np.nanmin(ma[: ov["accept_len"][i] + 1]) < NEAR_TIE or
                    ov["margin_sample"][i] < NEAR_TIE), ("reject mismatch", i)
            near_v += 1
    worst_conv = 0.0
    for s in check_conv_sites:
        if s >= len(cyc.conv_sites):
            continue
        site = cyc.conv_sites[s]
        args = (site.x[rows].cpu(), site.x_prev[rows].cpu(), site.w.cpu(),
                None if site.base is None else site.base.cpu())
        yo = oracle.dynconv2(*args)
        if site.y.dtype == torch.bfloat16:
            conv_rel_close_bf16(site.y[rows], yo, conv_term_scale(*args))
            bf16_ulp_close(site.y[rows], yo, conv_error_bound(*args))
        else:
            yg = site.y[rows].cpu().numpy()
            worst_conv = max(worst_conv, conv_rel_close(yg, yo, conv_term_scale(*args)))
            conv_close(yg, yo, conv_error_bound(*args))
    cmp.pop("excused_rows")
    report(label, rows=len(rows), S_worst=round(worst, 4), mean_accept=float(ga.mean()),
           reject_near_ties=near_v, **cmp)


def test_cycle_tiny_all_modes():
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    for mode in ("viterbi", "greedy"):
        cyc, _ = build(synth.scaled(w, path_mode=mode))
        cyc.run()
        check_cycle(cyc, synth.scaled(w, path_mode=mode), [0], f"tiny {mode}")


def test_cycle_b1_blk8_full_size():
    w = synth.WORKLOADS["b1_blk8_v151936"]
    cyc, _ = build(w)
    cyc.run()
    check_cycle(cyc, w, [0], w.name)


def test_cycle_b8_blk8_sampled_full_size():
    w = synth.WORKLOADS["b8_blk8_v151936_sampled"]
    cyc, _ = build(w)
    cyc.run()
    check_cycle(cyc, w, list(range(8)), w.name)


def test_cycle_b32_blk16_conv_full_size():
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    cyc, _ = build(w)
    cyc.run()
    check_cycle(cyc, w, [0, 13, 31], w.name, check_conv_sites=(0, 7, 19))


def test_cycle_b32_blk16_tables_graph():
    """The batch-32 / block-16 cycle with pair scores read from per-token
    tables (built once), captured as a graph and replayed: the same checks
    against the oracle's own cycle, which projects the embedding rows."""
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    print(f"[case] {w.name} tables graph", flush=True)
    cyc, _ = build(w, with_conv=0, tables=True)
    cyc.capture(conv=False)
    for _ in range(3):
        cyc.replay()
    check_cycle(cyc, w, [0, 13, 31], w.name + " tables")


def test_stress_shape_tables_graph():
    """64 requests, block 16, vocabulary 262,144 (a 537 MB table), greedy
    verification for requests 0-31 and rejection sampling for 32-63, pair
    scores from per-token tables, captured and replayed."""
    w = synth.WORKLOADS["b64_blk16_v262144_stress"]
    print(f"[case] {w.name} tables graph", flush=True)
    cyc, _ = build(w, with_conv=0, tables=True)
    cyc.set_seed(4_000_000)
    cyc.capture(conv=False)
    for _ in range(3):
        cyc.replay()
    check_cycle(cyc, w, [0, 31, 32, 63], w.name + " tables")


def test_cycle_b8_blk8_sampled_tables():
    w = synth.WORKLOADS["b8_blk8_v151936_sampled"]
    cyc, _ = build(w, tables=True)
    cyc.run()
    check_cycle(cyc, w, list(range(8)), w.name + " tables")


def test_graph_replay_equals_eager_and_is_deterministic():
    w = synth.scaled(synth.WORKLOADS["b8_blk8_v151936_sampled"], V=32768, d=1024)
    cyc, _ = build(w, with_conv=2)
    cyc.run()
    torch.cuda.synchronize()
    eager = {k: getattr(cyc, k).clone() for k in ("cand_idx", "scores", "path_rank", "q", "out_tok",
                                                  "accept_len")}
    y_eager = cyc.conv_sites[1].y.clone()
    cyc.capture()
    for rep in range(4):
        for k in eager:
            getattr(cyc, k).fill_(-7)
        cyc.conv_sites[1].y.zero_()
        cyc.replay()
        torch.cuda.synchronize()
        for k, v in eager.items():
            assert torch.equal(getattr(cyc, k), v), (rep, k)
        assert torch.equal(cyc.conv_sites[1].y, y_eager)
        _ = torch.randn(1000, device=DEV).sum().item()    # eager work between replays
    # a new seed changes the sampled path; the old seed reproduces it
    cyc.set_seed(w.seed + 1)
    cyc.replay()
    torch.cuda.synchronize()
    changed = not torch.equal(cyc.path_rank, eager["path_rank"])
    cyc.set_seed(w.seed)
    cyc.replay()
    torch.cuda.synchronize()
    assert torch.equal(cyc.path_rank, eager["path_rank"])
    assert changed


def test_stress_b64_blk16_v262144_graph_1000_replays():
    """Full stress cycle captured once and replayed 1,000 times with a fresh
    seed per replay (seed = 4,000,000 + cycle); the oracle checks cycles
    0, 99, ..., 999 on sampled requests of both verify halves."""
    w = synth.WORKLOADS["b64_blk16_v262144_stress"]
    cyc, _ = build(w)
    cyc.set_seed(4_000_000)
    cyc.capture()
    rows = [0, 17, 32, 47, 63]
    checks = set(range(0, 1000, 99)) | {999}
    results = {}
    for c in range(1000):
        cyc.set_seed(4_000_000 + c)
        cyc.replay()
        if c in checks:
            torch.cuda.synchronize()
            results[c] = (cyc.accept_len.clone(), cyc.out_tok.clone())
    torch.cuda.synchronize()
    # seed-independent stages once
    cyc.set_seed(4_000_000)
    cyc.replay()
    check_cycle(cyc, w, rows, w.name + " cycle 0", check_conv_sites=(0, 19))
    half = list(range(32, 64))
    o = oracle_cycle(cyc, half, w, 0)
    op = oracle.path(o["S"], o["idx"], oracle.PATH_VITERBI)
    g_rank = cyc.path_rank[32:].cpu().numpy()
    cmp = compare_path(g_rank, op, cyc.scores[32:].cpu().numpy(), o["S"], oracle.PATH_VITERBI, cyc.tau, w.T)
    assert cmp["bad"] == 0 and cmp["undecided_flips"] <= 4, cmp
    # requests whose path flipped on an undecided decision are verified
    # against the oracle run on the GPU's own path
    same = np.array([np.array_equal(g_rank[i], op["rank"][i]) for i in range(32)])
    v_tok = np.where(same[:, None], op["tok"], cyc.path_tok[32:].cpu().numpy())
    v_rank = np.where(same[:, None], op["rank"], g_rank)
    v_q = np.where(same[:, None, None], op["q"], cyc.q[32:].cpu().numpy())
    Z = cyc.target[32:].cpu()
    near = 0
    for c in sorted(checks):
        acc, out = results[c]
        # the reject half's Philox counters carry the requests' batch indices
        ov = oracle.verify_reject(Z, v_tok, v_rank, o["idx"], v_q, cyc.tau, 4_000_000 + c, b_ids=np.array(half))
        ga, go = acc[32:].cpu().numpy(), out[32:].cpu().numpy()
        for i in range(32):
            if ga[i] == ov["accept_len"][i] and np.array_equal(go[i], ov["out_tok"][i]):
                continue
            ma = ov["margin_accept"][i]
            assert np.nanmin(ma[: ov["accept_len"][i] + 1]) < NEAR_TIE or \
                ov["margin_sample"][i] < NEAR_TIE, (c, i)
            near += 1
        # the greedy half does not depend on the seed
        assert torch.equal(acc[:32], results[0][0][:32])
    report("stress 1000 replays", checked_cycles=len(checks), reject_near_ties=near,
           undecided_flips=cmp["undecided_flips"])

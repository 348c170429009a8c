"""GPU parity of the per-token selector tables (dflash2_selector_tables) and
of the pair scores read from them (dflash2_pair_scores_tab), against the
CPU oracle: the tables against oracle.selector_tables (all rows at small
sizes, sampled rows at the full vocabulary), the scores against
oracle.pair_scores_tab on an oracle-built table, and end to end (GPU tables,
then GPU scores) against the oracle's pair scores from the embeddings.
Scores within 1e-3 relative (rms floor), as for the projection path; table
rows within 1e-3 relative, each magnitude floored at 1 % of the rms entry
(an entry is a sum of d products and may cancel), and within the forward
error bound of an fp32 sum of exact bf16 products (gpu_util.gemm_error_bound)
as well."""
import numpy as np
import pytest
import torch

import draft_selection_bf16_amd as df2
import oracle
import synth
from gpu_util import DEV, close, conv_close, dev, gemm_error_bound, report, ws

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _table_bound(E, wa, wb):
    return np.concatenate([gemm_error_bound(E, wa), gemm_error_bound(E, wb)], axis=1)


def _tables_gpu(E, wa, wb):
    tab = torch.empty((E.shape[0], 2 * wa.shape[0]), dtype=torch.float32, device=DEV)
    df2.dflash2_selector_tables(dev(E), dev(wa), dev(wb), tab)
    return tab


def _scores_tab_gpu(cand, val, last, tab, h, wh, gate=0):
    B, T, K = cand.shape
    d, r = h.shape[-1], wh.shape[0]
    S = torch.empty((B, T, K, K), dtype=torch.float32, device=DEV)
    w = ws(df2.dflash2_pair_scores_tab_workspace_bytes(B, T, d, r))
    df2.dflash2_pair_scores_tab(dev(cand), dev(val), dev(last), dev(tab), dev(h), dev(wh), S, w, gate=gate)
    torch.cuda.synchronize()
    return S.cpu().numpy()


def _inputs(w):
    z, _, _ = synth.drafter_logits(w)
    idx, val = oracle.topk(z, w.K)
    E = synth.embeddings(w)
    wa, wb, wh = synth.selector_weights(w)
    return torch.from_numpy(idx), torch.from_numpy(val), synth.last_tokens(w), E, synth.context_hidden(w), \
        wa, wb, wh


@pytest.mark.parametrize("r", [256, 64])
def test_selector_tables_all_rows(r):
    """V = 3000 (23 full 128-row tiles and a ragged tail of 56), d = 384;
    rank 64 projects W_A and W_B as two problems."""
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], V=3000, d=384, r=r)
    E = synth.embeddings(w)
    wa, wb, _ = synth.selector_weights(w)
    tab = _tables_gpu(E, wa, wb)
    torch.cuda.synchronize()
    tg, to = tab.cpu().numpy(), oracle.selector_tables(E, wa, wb)
    worst = close(tg, to, floor=1e-2)
    worst_b = conv_close(tg, to, _table_bound(E, wa, wb))
    report("selector_tables", V=w.V, d=w.d, r=r, worst_err_over_1e3=round(worst, 4),
           worst_err_over_sum_bound=round(worst_b, 4))


@pytest.mark.parametrize("gate", [0, 1])
def test_pair_scores_tab_mid(gate):
    """B=3, T=7, K=16, V=4096, d=512, r=256; the H projection split over d."""
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=3, V=4096, d=512)
    idx, val, last, E, h, wa, wb, wh = _inputs(w)
    tab_o = oracle.selector_tables(E, wa, wb).astype(np.float32)
    Sg = _scores_tab_gpu(idx, val, last, torch.from_numpy(tab_o), h, wh, gate)
    worst = close(Sg, oracle.pair_scores_tab(idx, val, last, tab_o, h, wh, gate=gate))
    # end to end: tables and scores on the GPU against the scores from the embeddings
    Sg2 = _scores_tab_gpu(idx, val, last, _tables_gpu(E, wa, wb), h, wh, gate)
    worst2 = close(Sg2, oracle.pair_scores(idx, val, last, E, h, wa, wb, wh, gate=gate))
    report("pair_scores_tab mid", gate=gate, worst_err_over_bound=round(max(worst, worst2), 4))


@pytest.mark.parametrize("B,block,r,K", [(2, 8, 64, 7), (1, 8, 256, 16), (5, 4, 128, 16), (3, 2, 256, 1),
                                         (2, 3, 16, 2)])
def test_pair_scores_tab_shapes(B, block, r, K):
    """Ragged K x K lattices (K = 7), one request, short blocks, ranks 64 and
    128; one draft position with one candidate; rank 16 with two."""
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=B, block=block, V=3000, d=384, r=r, K=K)
    idx, val, last, E, h, wa, wb, wh = _inputs(w)
    Sg = _scores_tab_gpu(idx, val, last, _tables_gpu(E, wa, wb), h, wh)
    worst = close(Sg, oracle.pair_scores(idx, val, last, E, h, wa, wb, wh))
    report("pair_scores_tab shapes", B=B, T=w.T, r=r, K=K, worst_err_over_bound=round(worst, 4))


def test_pair_scores_tab_in_two_halves_on_two_streams():
    """dflash2_h_projection on a side stream, joined by an event, then
    dflash2_pair_scores_tab_from_h: the same kernels as the one call, so the
    same bits, and the oracle's scores."""
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=4, V=4096, d=512)
    idx, val, last, E, h, wa, wb, wh = _inputs(w)
    tab = _tables_gpu(E, wa, wb)
    one = _scores_tab_gpu(idx, val, last, tab, h, wh, gate=1)
    B, T, K = idx.shape
    hd, whd = dev(h), dev(wh)
    wsp = ws(df2.dflash2_pair_scores_tab_workspace_bytes(B, T, w.d, w.r))
    S = torch.empty((B, T, K, K), dtype=torch.float32, device=DEV)
    args = [dev(idx), dev(val), dev(last)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        df2.dflash2_h_projection(hd, whd, wsp)
    torch.cuda.current_stream().wait_stream(side)
    df2.dflash2_pair_scores_tab_from_h(*args, tab, w.d, S, wsp, gate=1)
    torch.cuda.synchronize()
    two = S.cpu().numpy()
    assert np.array_equal(one, two)
    worst = close(two, oracle.pair_scores(idx, val, last, E, h, wa, wb, wh, gate=1))
    report("pair_scores_tab two halves", worst_err_over_bound=round(worst, 4))


def test_pair_scores_tab_out_of_range_ids_read_zero_rows():
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=2, V=600, d=128, r=32, K=4)
    idx, val, last, E, h, wa, wb, wh = _inputs(w)
    idx[0, 3, 2] = 10_000_000
    idx[1, 1, 0] = -3
    last[1] = w.V
    tab_o = oracle.selector_tables(E, wa, wb).astype(np.float32)
    Sg = _scores_tab_gpu(idx, val, last, torch.from_numpy(tab_o), h, wh)
    So = oracle.pair_scores_tab(idx, val, last, tab_o, h, wh)
    close(Sg, So)
    assert np.all(Sg[0, 3, :, 2] == val[0, 3, 2].item())
    assert np.all(Sg[1, 0, 0, :] == val[1, 0, :].numpy())


def test_pair_scores_tab_full_size():
    """32 requests, block 16 (T = 15), K = 16, V = 151,936, d = 5120, r = 256:
    the launch shapes the cycle uses.  Candidate ids uniform over the
    vocabulary with the first and last token planted; every score against
    the oracle's pair scores from the embeddings, and 64 table rows (the
    first and last tile among them) against the oracle's tables."""
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    print(f"[case] pair_scores_tab full size B={w.B} T={w.T} K={w.K} V={w.V} d={w.d}", flush=True)
    E = synth.embeddings(w, device=DEV)
    wa, wb, wh = synth.selector_weights(w, device=DEV)
    h, last = synth.context_hidden(w, device=DEV), synth.last_tokens(w, device=DEV)
    g = torch.Generator().manual_seed(77)
    cand = torch.randint(0, w.V, (w.B, w.T, w.K), generator=g, dtype=torch.int32)
    cand[0, 0, 0], cand[-1, -1, -1] = 0, w.V - 1
    U = 3 * torch.randn(w.B, w.T, w.K, generator=g)
    tab = _tables_gpu(E, wa, wb)
    Sg = _scores_tab_gpu(cand, U, last, tab, h, wh)
    Ec, wac, wbc, whc, hc, lc = E.cpu(), wa.cpu(), wb.cpu(), wh.cpu(), h.cpu(), last.cpu()
    worst = close(Sg, oracle.pair_scores(cand, U, lc, Ec, hc, wac, wbc, whc))
    rng = np.random.default_rng(78)
    rows = np.r_[0, 1, 127, 128, w.V - 128, w.V - 1, rng.integers(0, w.V, 58)]
    Er = Ec[torch.from_numpy(rows)]
    tg = tab[torch.from_numpy(rows).to(DEV)].cpu().numpy()
    to = oracle.selector_tables(Ec, wac, wbc, rows=rows)
    worst_t = close(tg, to, floor=1e-2)
    conv_close(tg, to, _table_bound(Er, wac, wbc))
    report("pair_scores_tab full", worst_err_over_bound=round(worst, 4), table_rows=round(worst_t, 4))

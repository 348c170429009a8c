"""GPU parity, stage by stage: each C-ABI entry point against the CPU oracle
on the same seeded inputs.  Index, path and decision outputs must be
bit-exact (sampling decisions at an oracle margin below 1e-6 are reported,
not failed); scores within 1e-3 relative (rms floor); fp32 conv outputs
within 1e-3 relative to the magnitudes of the two terms of eq. Conv_k
(gpu_util.conv_term_scale; taps floored at 1 % of the rms tap), bf16 conv
outputs within one bf16 step more; the worst-case summation bound
(gpu_util.conv_error_bound) is checked as well."""
import numpy as np
import pytest
import torch

import draft_selection_bf16_amd as df2
import oracle
import synth
from gpu_util import (DEV, NEAR_TIE, bf16_ulp_close, close, conv_close, conv_error_bound, conv_rel_close,
                      conv_rel_close_bf16, conv_term_scale, dev, report, ws)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------- Philox
def test_philox_words_match_oracle():
    n = 300
    rng = np.random.default_rng(0)
    b = rng.integers(0, 1 << 20, n).astype(np.int32)
    t = rng.integers(0, 64, n).astype(np.int32)
    for seed in (0, 2, 4_000_123, 2**63 - 5):
        sd = torch.tensor([seed], dtype=torch.int64, device=DEV)
        out = torch.empty(4 * n, dtype=torch.int64, device=DEV)
        df2.dflash2_philox4x64(sd, dev(torch.from_numpy(b)), dev(torch.from_numpy(t)), out)
        _sync()
        got = out.cpu().numpy().view(np.uint64).reshape(n, 4)
        for i in range(0, n, 7):
            ref = oracle.philox(seed, (int(t[i]), int(b[i]), 0, 0))
            assert np.array_equal(got[i], ref), (seed, i)


# ----------------------------------------------------------------- top-K
def _topk_gpu(x, k):
    V = x.shape[-1]
    rows = x.numel() // V
    idx = torch.empty(x.shape[:-1] + (k,), dtype=torch.int32, device=DEV)
    val = torch.empty(x.shape[:-1] + (k,), dtype=torch.float32, device=DEV)
    w = ws(df2.dflash2_topk_workspace_bytes(rows, V, k))
    df2.dflash2_topk(x, k, idx, val, w)
    _sync()
    return idx.cpu().numpy(), val.cpu().numpy()


def _check_topk(x_cpu, k):
    gi, gv = _topk_gpu(dev(x_cpu), k)
    oi, ov = oracle.topk(x_cpu, k)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv, ov)


@pytest.mark.parametrize("k", [1, 4, 16])
def test_topk_tiny_fp32(k):
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, _, _ = synth.drafter_logits(w)
    _check_topk(z, k)


@pytest.mark.parametrize("V", [1001, 4099, 16384, 151936, 151939])
def test_topk_bf16_ragged_vocab(V):
    """Row lengths that are not multiples of 8 start rows off 16-byte
    alignment: the head/tail path runs."""
    g = torch.Generator().manual_seed(V)
    z = (3 * torch.randn(5, V, generator=g)).to(torch.bfloat16)
    _check_topk(z, 16)


def test_topk_ties_and_signed_zero():
    g = torch.Generator().manual_seed(1)
    z = torch.round(torch.randn(9, 50000, generator=g) * 2) / 2     # heavy ties
    z[0] = 0.0
    z[0, ::2] = -0.0
    z[1] = 1.0
    z[2, :100] = 7.0
    _check_topk(z.to(torch.bfloat16), 16)
    _check_topk(z, 16)


def test_topk_merge_many_survivors_falls_back_exactly():
    """Few rows, so every row is split into 15 chunks and the per-chunk
    lists are merged.  Five chunks each hold 16 distinct large values,
    interleaved across the five (chunk c gets 10 + (5 i + c) / 16): every
    chunk's 16th best is small, the first three keys of all 15 lists hold
    only 15 large ones, so both lower bounds of the merge stay low and 76
    keys pass them, more than the 64 of the ranked path: the exact fallback
    has to pick the 16 best."""
    V = 15 * 8192
    g = torch.Generator().manual_seed(21)
    z = torch.randn(2, V, generator=g)
    for row in range(2):
        for c in range(5):
            hot = (3 * c + row) % 15
            pos = hot * 8192 + torch.randperm(8192, generator=g)[:16]
            z[row, pos] = 10.0 + 0.0625 * (5 * torch.arange(16, dtype=torch.float32) + c)   # exact in bf16
    z = z.to(torch.bfloat16)
    gi, gv = _topk_gpu(dev(z), 16)
    oi, ov = oracle.topk(z.float(), 16)
    assert np.array_equal(gi, oi) and np.array_equal(gv, ov)


def test_topk_fp16():
    g = torch.Generator().manual_seed(2)
    z = (3 * torch.randn(4, 32771, generator=g)).to(torch.float16)
    _check_topk(z, 16)


def test_topk_adversarial_ascending_rows():
    """Ascending rows make every entry a new maximum: the threshold filter
    hits its slow path on every load."""
    V = 70000
    z = torch.arange(V, dtype=torch.float32).repeat(3, 1) * 1e-3
    z[1] = z[1].flip(0)
    _check_topk(z.to(torch.bfloat16), 16)


def test_topk_launch_shape_of_the_b32_blk16_workload():
    """480 rows of 151,936 bf16 logits, the launch configuration the
    benchmark times; all rows compared."""
    w = synth.WORKLOADS["b32_blk16_v151936_conv"]
    z, tok, rank = synth.drafter_logits(w, device=DEV)
    gi, gv = _topk_gpu(z, 16)
    oi, ov = oracle.topk(z.cpu(), 16)
    assert np.array_equal(gi, oi) and np.array_equal(gv, ov)
    tok = tok.cpu().numpy()
    r16 = (gi == tok[..., None]).any(-1).mean()
    report("topk b32_blk16", recall16=round(float(r16), 4))


@pytest.mark.parametrize("name", ["b1_blk16_v151936", "b8_blk8_v151936_sampled", "b8_blk16_v151936",
                                  "b32_blk8_v151936"])
def test_topk_small_batch_launch_shapes(name):
    """The drafter logits of the other batch x block points (15, 56, 120 and
    224 rows of 151,936: 19 short chunks per row for 15 and 56 rows, 2 and 1
    streamed chunks for 120 and 224, then the merge where there is more than
    one), all rows compared."""
    w = synth.WORKLOADS[name]
    z, _, _ = synth.drafter_logits(w, device=DEV)
    gi, gv = _topk_gpu(z, 16)
    oi, ov = oracle.topk(z.cpu(), 16)
    assert np.array_equal(gi, oi) and np.array_equal(gv, ov)


def test_topk_gumbel_v262144_rows():
    w = synth.scaled(synth.WORKLOADS["b64_blk16_v262144_stress"], B=2)
    z, _, _ = synth.drafter_logits(w, device=DEV)
    gi, gv = _topk_gpu(z, 16)
    oi, ov = oracle.topk(z.cpu(), 16)
    assert np.array_equal(gi, oi) and np.array_equal(gv, ov)


def _mixed_rows(n_rows, V, seed):
    """Rows of many kinds: random, heavy ties, all negative, ascending,
    constant, signed zeros, NaN-sprinkled, with infinities."""
    g = torch.Generator().manual_seed(seed)
    z = 3 * torch.randn(n_rows, V, generator=g)
    kinds = 8
    for r in range(n_rows):
        kind = r % kinds
        if kind == 1:
            z[r] = torch.round(z[r] * 0.6) / 2
        elif kind == 2:
            z[r] = -z[r].abs() - 1
        elif kind == 3:
            z[r] = torch.arange(V, dtype=torch.float32) * 1e-3
        elif kind == 4:
            z[r] = 1.0
        elif kind == 5:
            z[r] = 0.0
            z[r, r % 3::3] = -0.0
        elif kind == 6:
            z[r, torch.randint(0, V, (V // 10,), generator=g)] = float("nan")
        elif kind == 7:
            z[r, torch.randint(0, V, (8,), generator=g)] = float("inf")
            z[r, torch.randint(0, V, (V // 50,), generator=g)] = float("-inf")
    return z


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 151939), (torch.float16, 50001),
                                     (torch.float32, 50003)])
def test_topk_one_chunk_per_row(dtype, V):
    """Enough rows that each row is one work-group (no merge kernel): the
    pooled final selection, its many-ties fallback, the threshold test for
    negative rows and the NaN-padded head/tail groups all run.  NaN is never
    selected, so the oracle sees NaN as -inf (every row keeps >= 16 other
    entries)."""
    z = _mixed_rows(456, V, seed=V).to(dtype)
    gi, gv = _topk_gpu(dev(z), 16)
    zo = torch.where(torch.isnan(z), torch.full_like(z, float("-inf")), z)
    oi, ov = oracle.topk(zo, 16)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv, ov)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 151939), (torch.float16, 50001),
                                     (torch.float32, 50003), (torch.bfloat16, 7000)])
def test_topk_short_chunks_mixed_rows(dtype, V):
    """Few rows, so rows are cut into chunks of at most 8,192 entries on the
    short-chunk kernel (one round of loads per work-group): the same kinds of
    rows as above -- constant and signed-zero rows take its exact fallback
    for massive ties -- plus a row that is NaN except for 20 entries, so most
    chunks hold fewer than 16 numbers; V = 7,000 is one chunk per row (no
    merge)."""
    z = _mixed_rows(17, V, seed=V + 1)
    g = torch.Generator().manual_seed(V)
    keep = torch.randperm(V, generator=g)[:20]
    row = torch.full((V,), float("nan"))
    row[keep] = torch.randn(20, generator=g)
    z[16] = row
    z = z.to(dtype)
    gi, gv = _topk_gpu(dev(z), 16)
    zo = torch.where(torch.isnan(z), torch.full_like(z, float("-inf")), z)
    oi, ov = oracle.topk(zo, 16)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv, ov)


def test_topk_random_shapes():
    """Seeded random shapes around the plan's boundaries (one chunk per row,
    short chunks, streamed chunks; vocabularies from 17 to ~200k, ragged and
    unaligned; k from 1 to 16; all three dtypes; NaN densities up to a
    half; some constant rows): every row against the oracle (NaN as -inf;
    rows keep >= 16 numbers)."""
    rng = np.random.default_rng(2026)
    dts = [torch.float32, torch.bfloat16, torch.float16]
    for case in range(24):
        rows = int(rng.integers(1, 41))
        V = int(rng.choice([17, 31, 64, 1000, 4096, 8191, 8192, 8193, 16384, 50021, 151936, 151939, 200003]))
        k = int(rng.integers(1, min(16, V) + 1))
        dt = dts[case % 3]
        nan_frac = float(rng.choice([0.0, 0.0, 0.01, 0.5]))
        g = torch.Generator().manual_seed(1000 + case)
        z = 3 * torch.randn(rows, V, generator=g)
        if rows > 2:
            z[1] = 0.5                                   # constant row: ties everywhere
        if nan_frac > 0 and V >= 64:
            m = torch.rand(rows, V, generator=g) < nan_frac
            z[m] = float("nan")
            z[torch.isnan(z).sum(1) > V - 16] = 1.0      # keep >= 16 numbers per row
        z = z.to(dt)
        print(f"[case] topk random {case}: rows={rows} V={V} k={k} dt={dt} nan={nan_frac}", flush=True)
        gi, gv = _topk_gpu(dev(z), k)
        zo = torch.where(torch.isnan(z), torch.full_like(z, float("-inf")), z)
        oi, ov = oracle.topk(zo, k)
        assert np.array_equal(gi, oi), case
        assert np.array_equal(gv, ov), case


# ----------------------------------------------------------------- pair scores
def _pair_gpu(cand_idx, cand_val, last, E, h, wa, wb, wh, gate=0):
    B, T, K = cand_idx.shape
    d, r = E.shape[1], wa.shape[0]
    S = torch.empty((B, T, K, K), dtype=torch.float32, device=DEV)
    nb = df2.dflash2_pair_scores_workspace_bytes(B, T, K, d, r)
    w = ws(nb)
    df2.dflash2_pair_scores(dev(cand_idx), dev(cand_val), dev(last), dev(E), dev(h), dev(wa), dev(wb),
                            dev(wh), S, w, gate=gate)
    _sync()
    return S.cpu().numpy(), w


def _ws_views(w, B, T, K, r, gate=0):
    """The projection's results in the pair-scores workspace: [A|B] of the
    candidates, A of the last tokens and H, each stored as S slices of
    partial products over the hidden size (S found from the workspace size);
    with S > 1 the library has summed the slices into slice 0 (in place)
    before the epilogue.  H is stored before its gate."""
    def a256(n):
        return (n + 255) // 256 * 256
    n_ab, n_al, n_h = B * T * K * 2 * r, B * r, B * T * r
    nbytes = w.numel()
    S = next(s for s in range(1, 33) if a256(s * n_ab * 4) + a256(s * n_al * 4) + a256(s * n_h * 4) == nbytes)
    f = w.view(torch.float32)
    off_al = a256(S * n_ab * 4) // 4
    off_h = off_al + a256(S * n_al * 4) // 4

    def summed(off, n):
        return f[off:off + n].cpu().numpy()
    ab = summed(0, n_ab).reshape(B, T, K, 2 * r)
    al = summed(off_al, n_al).reshape(B, r)
    hg = summed(off_h, n_h).reshape(B, T, r)
    if gate == 1:
        hg = 1.0 / (1.0 + np.exp(-hg))
    return ab, al, hg


@pytest.mark.parametrize("gate", [0, 1])
def test_pair_scores_tiny(gate):
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, _, _ = synth.drafter_logits(w)
    idx, val = oracle.topk(z, w.K)
    E = synth.embeddings(w)
    wa, wb, wh = synth.selector_weights(w)
    h, last = synth.context_hidden(w), synth.last_tokens(w)
    Sg, _ = _pair_gpu(torch.from_numpy(idx), torch.from_numpy(val), last, E, h, wa, wb, wh, gate)
    So = oracle.pair_scores(idx, val, last, E, h, wa, wb, wh, gate=gate)
    close(Sg, So)


@pytest.mark.parametrize("gate", [0, 1])
def test_pair_scores_mid_with_intermediates(gate):
    """B=3, T=7, K=16, V=4096, d=512, r=256: several GEMM tiles, a ragged
    M tail (3*7*16 = 336 rows), gathered rows, the projection split over d
    into slices (few tiles), the gate applied after the slices are added."""
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=3, V=4096, d=512)
    z, _, _ = synth.drafter_logits(w)
    idx, val = oracle.topk(z, 16)
    E = synth.embeddings(w)
    wa, wb, wh = synth.selector_weights(w)
    h, last = synth.context_hidden(w), synth.last_tokens(w)
    Sg, wsp = _pair_gpu(torch.from_numpy(idx), torch.from_numpy(val), last, E, h, wa, wb, wh, gate)
    So, inter = oracle.pair_scores(idx, val, last, E, h, wa, wb, wh, gate=gate, intermediates=True)
    worst = close(Sg, So)
    ab, al, hg = _ws_views(wsp, 3, 7, 16, 256, gate)
    # A of the last block position is never a predecessor and is not computed
    close(ab[:, :-1, :, :256], inter["a_cand"][:, :-1])
    close(ab[..., 256:], inter["b_cand"])
    close(al, inter["a_last"])
    close(hg, inter["h"])
    report("pair_scores mid", worst_err_over_bound=round(worst, 4))


@pytest.mark.parametrize("r,K", [(128, 16), (64, 7)])
def test_pair_scores_other_ranks(r, K):
    """Rank 128 (one W tile per half of [W_A; W_B]) and rank 64 with K = 7
    (W_A and W_B projected as separate problems; ragged K x K lattices)."""
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=2, V=3000, d=384, r=r, K=K)
    z, _, _ = synth.drafter_logits(w)
    idx, val = oracle.topk(z, K)
    E = synth.embeddings(w)
    wa, wb, wh = synth.selector_weights(w)
    h, last = synth.context_hidden(w), synth.last_tokens(w)
    Sg, _ = _pair_gpu(torch.from_numpy(idx), torch.from_numpy(val), last, E, h, wa, wb, wh)
    So = oracle.pair_scores(idx, val, last, E, h, wa, wb, wh)
    worst = close(Sg, So)
    report("pair_scores other ranks", r=r, K=K, worst_err_over_bound=round(worst, 4))


@pytest.mark.parametrize("B,block,V", [(32, 16, 151936), (32, 8, 151936), (64, 16, 262144)])
def test_pair_scores_full_size_every_request(B, block, V):
    """K = 16, d = 5120, r = 256 through the per-cycle projection: the
    benchmark's launch (32 requests, block 16: 7,680 gathered rows on
    128 x 128 tiles, no K split), block 8 (3,584 rows, two slices summed by
    the reduce pass) and the stress shape (64 requests, V = 262,144: a
    2.7 GB embedding table, whose byte offsets exceed 31 bits); every score
    of every request against the oracle.  Candidate ids uniform over the
    vocabulary, the first and last token planted."""
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=B, block=block, V=V)
    print(f"[case] pair_scores full size B={w.B} T={w.T} K={w.K} V={w.V} d={w.d}", flush=True)
    E = synth.embeddings(w, device=DEV)
    wa, wb, wh = synth.selector_weights(w, device=DEV)
    h, last = synth.context_hidden(w, device=DEV), synth.last_tokens(w, device=DEV)
    g = torch.Generator().manual_seed(79 + block + B)
    cand = torch.randint(0, w.V, (w.B, w.T, w.K), generator=g, dtype=torch.int32)
    cand[0, 0, 0], cand[-1, -1, -1] = 0, w.V - 1
    U = 3 * torch.randn(w.B, w.T, w.K, generator=g)
    Sg, _ = _pair_gpu(cand, U, last, E, h, wa, wb, wh)
    So = oracle.pair_scores(cand, U, last.cpu(), E.cpu(), h.cpu(), wa.cpu(), wb.cpu(), wh.cpu())
    del E
    worst = close(Sg, So)
    report("pair_scores full", T=w.T, worst_err_over_bound=round(worst, 4))


def test_pair_scores_out_of_range_tokens_read_zero_rows():
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=1, V=512, d=128, r=32)
    E = synth.embeddings(w)
    wa, wb, wh = synth.selector_weights(w)
    h = synth.context_hidden(w)
    cand = torch.randint(0, 512, (1, 7, 4), dtype=torch.int32)
    cand[0, 3, 2] = 10_000_000      # out of range -> zero embedding -> bigram 0
    val = torch.randn(1, 7, 4)
    last = torch.tensor([-5], dtype=torch.int32)
    Sg, _ = _pair_gpu(cand, val, last, E, h, wa, wb, wh)
    assert np.all(Sg[0, 3, :, 2] == val[0, 3, 2].item())
    assert np.all(Sg[0, 0, 0, :] == val[0, 0].numpy())   # last token -> zero A


# ----------------------------------------------------------------- path
def _path_gpu(S, cand, mode, tau=0.0, seed=0, b0=0):
    B, T, K, _ = S.shape
    pr = torch.empty((B, T), dtype=torch.int32, device=DEV)
    pt = torch.empty((B, T), dtype=torch.int32, device=DEV)
    q = torch.empty((B, T, K), dtype=torch.float32, device=DEV)
    ps = torch.empty((B,), dtype=torch.float32, device=DEV)
    sd = torch.tensor([seed], dtype=torch.int64, device=DEV)
    df2.dflash2_path_viterbi(dev(S), dev(cand), mode, pr, pt, q, ps, temperature=tau, seed_dev=sd, b0=b0)
    _sync()
    return dict(rank=pr.cpu().numpy(), tok=pt.cpu().numpy(), q=q.cpu().numpy(), score=ps.cpu().numpy())


@pytest.mark.parametrize("B,T,K,ties", [(1, 3, 4, False), (32, 15, 16, False), (64, 15, 16, True),
                                        (8, 7, 16, True), (5, 1, 16, False), (3, 63, 16, False),
                                        (7, 9, 5, True), (3, 5, 1, False), (4, 6, 2, True)])
@pytest.mark.parametrize("mode", [0, 1])
def test_path_deterministic_modes_bit_exact(B, T, K, ties, mode):
    S = synth.pair_score_lattice(B, T, K, seed=B * 100 + T, ties=ties)
    cand = torch.randint(0, 151936, (B, T, K), dtype=torch.int32,
                         generator=torch.Generator().manual_seed(T))
    g = _path_gpu(S, cand, mode)
    o = oracle.path(S.numpy(), cand.numpy(), mode)
    for key in ("rank", "tok", "q", "score"):
        assert np.array_equal(g[key], o[key]), key


def test_path_random_shapes():
    """Seeded random lattices (batch up to 300, block positions 1 to 63,
    1 to 16 candidates, scores on a quarter grid in half the cases so that
    equal sums occur): both deterministic modes bit-exact against the
    oracle."""
    rng = np.random.default_rng(7171)
    for case in range(16):
        B = int(rng.integers(1, 301))
        T = int(rng.integers(1, 64))
        K = int(rng.integers(1, 17))
        ties = bool(case % 2)
        S = synth.pair_score_lattice(B, T, K, seed=9000 + case, ties=ties)
        cand = torch.randint(0, 151936, (B, T, K), dtype=torch.int32,
                             generator=torch.Generator().manual_seed(case))
        for mode in (0, 1):
            print(f"[case] path random {case}: B={B} T={T} K={K} ties={ties} mode={mode}", flush=True)
            g = _path_gpu(S, cand, mode)
            o = oracle.path(S.numpy(), cand.numpy(), mode)
            for key in ("rank", "tok", "q", "score"):
                assert np.array_equal(g[key], o[key]), (case, mode, key)


@pytest.mark.parametrize("B,T,K,tau", [(64, 15, 16, 1.0), (8, 7, 16, 0.5), (200, 3, 4, 2.0)])
def test_path_sampled(B, T, K, tau):
    S = synth.pair_score_lattice(B, T, K, seed=7 + T, spread=1.0)
    cand = torch.randint(0, 151936, (B, T, K), dtype=torch.int32,
                         generator=torch.Generator().manual_seed(5))
    seed = 2
    g = _path_gpu(S, cand, 2, tau, seed)
    o = oracle.path(S.numpy(), cand.numpy(), 2, temperature=tau, seed=seed)
    near, bad = 0, 0
    for b in range(B):
        if np.array_equal(g["rank"][b], o["rank"][b]):
            close(g["q"][b], o["q"][b], rel=1e-5)
            assert g["score"][b] == o["score"][b]
            continue
        t = int(np.flatnonzero(g["rank"][b] != o["rank"][b])[0])
        if o["margin"][b, t] < NEAR_TIE:
            near += 1
        else:
            bad += 1
    report("path sample", B=B, T=T, near_tie_mismatches=near)
    assert bad == 0
    near_ties = int((o["margin"] < NEAR_TIE).sum())
    report("path sample", decisions=B * T, near_ties=near_ties)


def test_path_sample_sub_ranges_draw_the_batch_counters():
    """A batch sampled in two calls (requests 0-4 with b0 = 0, 5-11 with
    b0 = 5) draws the same uniforms, so the same paths, as one call; the
    oracle with the requests' batch indices agrees."""
    B, T, K, tau, seed = 12, 7, 16, 1.0, 9
    S = synth.pair_score_lattice(B, T, K, seed=3, spread=1.0)
    cand = torch.randint(0, 151936, (B, T, K), dtype=torch.int32, generator=torch.Generator().manual_seed(4))
    full = _path_gpu(S, cand, 2, tau, seed)
    lo = _path_gpu(S[:5].contiguous(), cand[:5].contiguous(), 2, tau, seed, b0=0)
    hi = _path_gpu(S[5:].contiguous(), cand[5:].contiguous(), 2, tau, seed, b0=5)
    for key in ("rank", "tok", "q", "score"):
        assert np.array_equal(np.concatenate([lo[key], hi[key]]), full[key]), key
    o = oracle.path(S[5:].numpy(), cand[5:].numpy(), 2, temperature=tau, seed=seed, b_ids=np.arange(5, B))
    o_full = oracle.path(S.numpy(), cand.numpy(), 2, temperature=tau, seed=seed)
    assert np.array_equal(o["rank"], o_full["rank"][5:])
    ok = o["margin"].min(axis=1) >= NEAR_TIE
    assert np.array_equal(hi["rank"][ok], o["rank"][ok])


# ----------------------------------------------------------------- verify
def _verify_greedy_gpu(Z, path_tok):
    B, T1, V = Z.shape
    acc = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, T1), dtype=torch.int32, device=DEV)
    w = ws(df2.dflash2_verify_workspace_bytes(B, T1 - 1, V))
    df2.dflash2_verify_greedy(dev(Z), dev(path_tok), acc, out, w)
    _sync()
    return acc.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("name,B,T,V,dtype", [("tiny", 1, 3, 1000, torch.float32),
                                               ("ragged", 5, 7, 10007, torch.bfloat16),
                                               ("b32_blk16", 32, 15, 151936, torch.bfloat16),
                                               ("fp16", 3, 5, 5003, torch.float16),
                                               ("t63", 2, 63, 3001, torch.bfloat16),
                                               ("b1_blk8", 1, 7, 151936, torch.bfloat16)])
def test_verify_greedy_exact(name, B, T, V, dtype):
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=B, block=T + 1, V=V)
    d_dev = DEV if V > 100000 else "cpu"
    z, tok, _ = synth.drafter_logits(w, device=d_dev)
    Z = synth.target_logits(w, z, tok, device=d_dev).to(dtype)
    # drafts: mostly the true token, so prefixes of every length occur
    path = tok.to(torch.int32).clone()
    g = torch.Generator(device=d_dev).manual_seed(B)
    flip = torch.rand(path.shape, generator=g, device=d_dev) < 0.15
    path = torch.where(flip, (path + 1) % V, path).to(torch.int32)
    ga, go = _verify_greedy_gpu(Z, path)
    o = oracle.verify_greedy(Z.cpu(), path.cpu())
    assert np.array_equal(ga, o["accept_len"])
    assert np.array_equal(go, o["out_tok"])
    report(f"verify greedy {name}", mean_accept=float(ga.mean()))


def test_verify_greedy_random_shapes():
    """Seeded random shapes around the verification plan's boundaries (one
    chunk per row; one-pass chunks of at most 16,384 entries; the smaller
    chunks of very few rows; ragged vocabularies), all three dtypes, rows
    rounded to integers in some cases so that the argmax ties: acceptance
    lengths and emitted tokens bit-exact against the oracle."""
    rng = np.random.default_rng(4242)
    dts = [torch.bfloat16, torch.float16, torch.float32]
    for case in range(20):
        B = int(rng.integers(1, 49))
        T = int(rng.integers(1, 24))
        V = int(rng.choice([16, 100, 4096, 16383, 16384, 16385, 40000, 151936, 151939, 200003]))
        while B > 1 and B * (T + 1) * V > 24_000_000:
            B //= 2
        dt = dts[case % 3]
        g = torch.Generator().manual_seed(3000 + case)
        Z = 3 * torch.randn(B, T + 1, V, generator=g)
        if case % 4 == 1:
            Z = torch.round(Z)                           # ties at the argmax
        Z = Z.to(dt)
        am = Z.float().argmax(-1).to(torch.int32)
        flip = torch.rand(B, T, generator=g) < 0.2
        path = torch.where(flip, (am[:, :T] + 1) % V, am[:, :T]).to(torch.int32).contiguous()
        print(f"[case] verify greedy random {case}: B={B} T={T} V={V} dt={dt}", flush=True)
        ga, go = _verify_greedy_gpu(Z, path)
        o = oracle.verify_greedy(Z, path)
        assert np.array_equal(ga, o["accept_len"]), case
        assert np.array_equal(go, o["out_tok"]), case


def test_verify_greedy_ties_take_lowest_index():
    Z = torch.zeros((2, 3, 40000), dtype=torch.bfloat16)
    Z[:, :, 777] = 5.0
    Z[:, :, 30001] = 5.0
    Z[1, 1, 5] = 5.0
    path = torch.tensor([[777, 777], [777, 5]], dtype=torch.int32)
    ga, go = _verify_greedy_gpu(Z, path)
    o = oracle.verify_greedy(Z, path)
    assert np.array_equal(ga, o["accept_len"]) and np.array_equal(go, o["out_tok"])
    assert list(go[0]) == [777, 777, 777] and list(go[1]) == [777, 5, 777]


def _verify_reject_gpu(Z, path_tok, path_rank, cand, q, tau, seed, b0=0):
    B, T1, V = Z.shape
    acc = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, T1), dtype=torch.int32, device=DEV)
    w = ws(df2.dflash2_verify_workspace_bytes(B, T1 - 1, V))
    sd = torch.tensor([seed], dtype=torch.int64, device=DEV)
    df2.dflash2_verify_reject(dev(Z), dev(path_tok), dev(path_rank), dev(cand), dev(q), tau, sd, acc,
                              out, w, b0=b0)
    _sync()
    return acc.cpu().numpy(), out.cpu().numpy()


def _reject_case(B, T, V, tau, seed, sampled=True, dtype=torch.bfloat16):
    w = synth.scaled(synth.WORKLOADS["b8_blk8_v151936_sampled"], B=B, block=T + 1, V=V, tau=tau)
    d_dev = DEV if V > 100000 else "cpu"
    z, tok, _ = synth.drafter_logits(w, device=d_dev)
    Z = synth.target_logits(w, z, tok, device=d_dev).to(dtype)
    idx, val = oracle.topk(z.cpu(), 16)
    S = synth.pair_score_lattice(B, T, 16, seed=seed, spread=1.0).numpy()
    S = S + val[:, :, None, :]
    mode = oracle.PATH_SAMPLE if sampled else oracle.PATH_VITERBI
    pth = oracle.path(S, idx, mode, temperature=tau, seed=seed)
    return Z, pth, idx


@pytest.mark.parametrize("B,T,V,tau,sampled", [(8, 7, 151936, 1.0, True), (16, 15, 20000, 0.7, True),
                                               (16, 15, 20000, 1.0, False), (4, 3, 1000, 1.5, True),
                                               (1, 7, 151936, 1.0, True), (2, 63, 3001, 1.0, True),
                                               (3, 5, 20011, 0.8, True), (8, 7, 163840, 1.0, True),
                                               (32, 15, 151936, 1.0, True)])
def test_verify_reject_matches_oracle(B, T, V, tau, sampled):
    """Residual draws in one work-group per request (streaming chunks of at
    most 16,384 entries: every case but the last, which takes the two-pass
    search; V = 163,840 at 8 requests gives chunks of exactly 16,384), 63
    drafted positions, an odd vocabulary (rows not 16-byte aligned)."""
    seed = 2
    Z, pth, idx = _reject_case(B, T, V, tau, seed, sampled)
    ga, go = _verify_reject_gpu(Z, torch.from_numpy(pth["tok"]), torch.from_numpy(pth["rank"]),
                                torch.from_numpy(idx), torch.from_numpy(pth["q"]), tau, seed)
    o = oracle.verify_reject(Z.cpu(), pth["tok"], pth["rank"], idx, pth["q"], tau, seed)
    near, bad = 0, 0
    for b in range(B):
        if ga[b] == o["accept_len"][b] and np.array_equal(go[b], o["out_tok"][b]):
            continue
        ma = o["margin_accept"][b]
        if np.nanmin(ma[: o["accept_len"][b] + 1]) < NEAR_TIE or o["margin_sample"][b] < NEAR_TIE:
            near += 1
        else:
            bad += 1
    report("verify reject", B=B, T=T, V=V, near_tie_mismatches=near,
           mean_accept=float(np.mean(o["accept_len"])), fallbacks=o["fallbacks"])
    assert bad == 0


def test_verify_reject_random_shapes():
    """Seeded random shapes for rejection verification (batch, block,
    vocabulary across the chunk and residual-chunk boundaries, temperature,
    sampled or Viterbi drafts, all three dtypes): every request against the
    oracle, mismatches only at counted near-ties."""
    rng = np.random.default_rng(5151)
    dts = [torch.bfloat16, torch.float16, torch.float32]
    near = 0
    for case in range(12):
        B = int(rng.integers(1, 33))
        T = int(rng.integers(1, 16))
        V = int(rng.choice([64, 1000, 4096, 4097, 8193, 20000, 65536, 151936]))
        while B > 1 and B * (T + 1) * V > 12_000_000:
            B //= 2
        tau = float(rng.choice([0.5, 1.0, 1.7]))
        sampled = bool(case % 2 == 0)
        seed = 100 + case
        print(f"[case] verify reject random {case}: B={B} T={T} V={V} tau={tau} sampled={sampled}",
              flush=True)
        Z, pth, idx = _reject_case(B, T, V, tau, seed, sampled, dtype=dts[case % 3])
        ga, go = _verify_reject_gpu(Z, torch.from_numpy(pth["tok"]), torch.from_numpy(pth["rank"]),
                                    torch.from_numpy(idx), torch.from_numpy(pth["q"]), tau, seed)
        o = oracle.verify_reject(Z.cpu(), pth["tok"], pth["rank"], idx, pth["q"], tau, seed)
        for b in range(B):
            if ga[b] == o["accept_len"][b] and np.array_equal(go[b], o["out_tok"][b]):
                continue
            ma = o["margin_accept"][b]
            assert np.nanmin(ma[: o["accept_len"][b] + 1]) < NEAR_TIE or o["margin_sample"][b] < NEAR_TIE, \
                (case, b)
            near += 1
    report("verify reject random", near_tie_mismatches=near)


def test_verify_reject_sub_ranges_draw_the_batch_counters():
    """Rejection verification of a batch in two calls (requests 0-6 with
    b0 = 0, 7-15 with b0 = 7) gives what one call over the batch gives, and
    the upper call matches the oracle run with the batch indices 7..15."""
    B, T, V, tau, seed = 16, 7, 20000, 1.0, 5
    Z, pth, idx = _reject_case(B, T, V, tau, seed, True)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    full = _verify_reject_gpu(Z, t(pth["tok"]), t(pth["rank"]), t(idx), t(pth["q"]), tau, seed)
    lo = _verify_reject_gpu(Z[:7].contiguous(), t(pth["tok"][:7]), t(pth["rank"][:7]), t(idx[:7]),
                            t(pth["q"][:7]), tau, seed, b0=0)
    hi = _verify_reject_gpu(Z[7:].contiguous(), t(pth["tok"][7:]), t(pth["rank"][7:]), t(idx[7:]),
                            t(pth["q"][7:]), tau, seed, b0=7)
    assert np.array_equal(np.concatenate([lo[0], hi[0]]), full[0])
    assert np.array_equal(np.concatenate([lo[1], hi[1]]), full[1])
    o = oracle.verify_reject(Z[7:].cpu(), pth["tok"][7:], pth["rank"][7:], idx[7:], pth["q"][7:], tau, seed,
                             b_ids=np.arange(7, B))
    for b in range(B - 7):
        if hi[0][b] == o["accept_len"][b] and np.array_equal(hi[1][b], o["out_tok"][b]):
            continue
        ma = o["margin_accept"][b]
        assert np.nanmin(ma[: o["accept_len"][b] + 1]) < NEAR_TIE or o["margin_sample"][b] < NEAR_TIE


def test_verify_reject_distribution_on_gpu():
    """Many copies of one request: the first emitted token must follow p_0
    (the drafts are drawn from q, so acceptance + residual restore p)."""
    V, K, T, tau, N = 64, 4, 2, 1.0, 100_000
    rng = np.random.default_rng(3)
    Zrow = (rng.normal(size=(T + 1, V)) * 1.5).astype(np.float32)
    p0 = np.exp(Zrow[0] - Zrow[0].max())
    p0 /= p0.sum()
    cands = np.array([[3, 9, 27, 40], [1, 2, 5, 63]], np.int32)
    qrow = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]], np.float32)
    rank = np.stack([rng.choice(K, size=N, p=qrow[t] / qrow[t].sum()) for t in range(T)], 1)
    rank = rank.astype(np.int32)
    tok = np.take_along_axis(np.broadcast_to(cands, (N, T, K)), rank[..., None], -1)[..., 0]
    Z = torch.from_numpy(np.broadcast_to(Zrow, (N, T + 1, V)).copy())
    ga, go = _verify_reject_gpu(Z, torch.from_numpy(tok.astype(np.int32)), torch.from_numpy(rank),
                                torch.from_numpy(np.broadcast_to(cands, (N, T, K)).copy()),
                                torch.from_numpy(np.broadcast_to(qrow, (N, T, K)).copy()), tau, 11)
    counts = np.bincount(go[:, 0], minlength=V).astype(float)
    e = N * p0
    keep = e > 5
    chi2 = float((((counts - e) ** 2) / e)[keep].sum())
    report("verify reject MC", chi2=round(chi2, 1), dof=int(keep.sum()) - 1)
    assert chi2 < int(keep.sum()) + 8 * np.sqrt(2 * keep.sum())


# ----------------------------------------------------------------- dynconv2
def _conv_gpu(x, xp, wt, base, y_dtype):
    B, L, d = x.shape
    y = torch.empty((B, L, d), dtype=y_dtype, device=DEV)
    w = ws(df2.dflash2_dynconv2_workspace_bytes(B, L, d))
    df2.dflash2_dynconv2(dev(x), None if xp is None else dev(xp), dev(wt),
                         None if base is None else dev(base), y, w)
    _sync()
    return y


@pytest.mark.parametrize("B,L,d,base,prev", [(1, 4, 64, True, True), (2, 16, 256, False, True),
                                             (3, 5, 320, True, False), (32, 16, 5120, False, True),
                                             (65, 16, 1024, True, True), (2, 4, 8192, True, True),
                                             (1, 3, 16384, False, True)])
def test_dynconv2_matches_oracle(B, L, d, base, prev):
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=B, block=L, d=d, conv_base=base)
    x, xp, wt, bs = synth.conv_site(w, 0)
    if not prev:
        xp = None
    yo = oracle.dynconv2(x, xp, wt, bs)
    scale = conv_term_scale(x, xp, wt, bs)
    bound = conv_error_bound(x, xp, wt, bs)
    y32 = _conv_gpu(x, xp, wt, bs, torch.float32).cpu().numpy()
    worst = conv_rel_close(y32, yo, scale)
    worst_b = conv_close(y32, yo, bound)
    y16 = _conv_gpu(x, xp, wt, bs, torch.bfloat16)
    ulp = conv_rel_close_bf16(y16, yo, scale)
    bf16_ulp_close(y16, yo, bound)
    report("dynconv2", B=B, L=L, d=d, worst_err_over_1e3_terms=round(worst, 4),
           worst_err_over_sum_bound=round(worst_b, 4), bf16_steps=round(ulp, 3))


def test_dynconv2_random_shapes():
    """Seeded random shapes for the conv: batch and block lengths whose
    B L rows cross the GEMM's tile-height switch at 1,024 rows and its K
    split sizes; hidden sizes of any multiple of 64 up to 16,384; base and
    previous token present or not; fp32 and bf16 outputs against the oracle
    under the same rules as above."""
    rng = np.random.default_rng(6161)
    for case in range(12):
        d = 64 * int(rng.integers(1, 1 + (4, 16, 64, 256)[case % 4]))
        B = int(rng.integers(1, 81))
        L = int(rng.integers(1, 21))
        if case % 3 == 2:                                # 1,024 rows or more
            B, L, d = int(rng.integers(64, 81)), 16, 64 * int(rng.integers(1, 33))
        while B > 1 and B * L * d * d > 8_000_000_000:  # keeps the fp64 oracle at seconds
            B //= 2
        base, prev = bool(rng.integers(2)), bool(rng.integers(2))
        print(f"[case] dynconv2 random {case}: B={B} L={L} d={d} base={base} prev={prev}", flush=True)
        w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=B, block=L, d=d, conv_base=base,
                         seed=70 + case)
        x, xp, wt, bs = synth.conv_site(w, case)
        if not prev:
            xp = None
        yo = oracle.dynconv2(x, xp, wt, bs)
        scale = conv_term_scale(x, xp, wt, bs)
        bound = conv_error_bound(x, xp, wt, bs)
        y32 = _conv_gpu(x, xp, wt, bs, torch.float32).cpu().numpy()
        conv_rel_close(y32, yo, scale)
        conv_close(y32, yo, bound)
        y16 = _conv_gpu(x, xp, wt, bs, torch.bfloat16)
        conv_rel_close_bf16(y16, yo, scale)
        bf16_ulp_close(y16, yo, bound)


def test_dynconv2_identity_and_shift_exact():
    B, L, d = 2, 16, 5120
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=B, d=d)
    x, xp, _, _ = synth.conv_site(w, 1)
    zero = torch.zeros((2 * d // 16, d), dtype=torch.bfloat16)
    ident = torch.stack([torch.ones(d), torch.zeros(d)])
    shift = torch.stack([torch.zeros(d), torch.ones(d)])
    y = _conv_gpu(x, xp, zero, ident, torch.bfloat16).cpu()
    assert torch.equal(y, x)
    y = _conv_gpu(x, xp, zero, shift, torch.bfloat16).cpu()
    assert torch.equal(y[:, 0], xp) and torch.equal(y[:, 1:], x[:, :-1])

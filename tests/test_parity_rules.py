"""The GPU parity rules themselves, checked on the CPU.

The conv outputs are held to 1e-3 relative against the magnitudes of the two
terms of eq. Conv_k ("DFlash 2: Keep Drafting Parallel", section "A
lightweight local convolution").  These tests show that the rule accepts what
a correct fp32 evaluation produces and rejects a plausible precision bug: a
split-K tap GEMM that rounds each slice's partial sum to bf16 before adding
the slices.  The older worst-case rule (gamma_d * sum |w_i x_i|, Higham) lets
that bug through; it stays in the GPU tests only as an extra check.

The same rule is checked for the path comparison of the chained cycle tests:
a flip is excused only when the decision that flipped had an oracle margin
under the allowance the score error gives, and nowhere else."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import conv_close, conv_error_bound, conv_rel_close, conv_rel_close_bf16, conv_term_scale
from path_compare import compare_path


def _bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 -> float32, round to nearest even."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _conv_split_k(x, xp, w, slices: int, round_partials: bool) -> np.ndarray:
    """fp32 evaluation of the conv with the tap product split over d into
    `slices` slices: each slice's partial sum in fp32 (optionally rounded to
    bf16), the slices added in fp32 in slice order, then the fp32 epilogue."""
    xf = x.float().numpy()
    wf = w.float().numpy()
    B, L, d = xf.shape
    G = d // 16
    # slice edges on 64-wide K-tiles, as a split-K kernel cuts them
    edge = [64 * ((s * (d // 64)) // slices) for s in range(slices)] + [d]
    taps = np.zeros((B, L, 2 * G), np.float32)
    for s in range(slices):
        lo, hi = edge[s], edge[s + 1]
        part = (xf[..., lo:hi] @ wf[:, lo:hi].T).astype(np.float32)
        taps = (taps + (_bf16_round(part) if round_partials else part)).astype(np.float32)
    ch = np.arange(d) // 16
    xm1 = np.concatenate([xp.float().numpy()[:, None, :], xf[:, :-1, :]], axis=1)
    return (taps[..., ch] * xf + taps[..., G + ch] * xm1).astype(np.float32)


@pytest.fixture(scope="module")
def site():
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=4)
    x, xp, wt, bs = synth.conv_site(w, 0)
    assert bs is None
    yo = oracle.dynconv2(x, xp, wt, None)
    return x, xp, wt, yo, conv_term_scale(x, xp, wt), conv_error_bound(x, xp, wt)


def test_correct_fp32_split_k_passes(site):
    x, xp, wt, yo, scale, bound = site
    y = _conv_split_k(x, xp, wt, 6, round_partials=False)
    worst = conv_rel_close(y, yo, scale)
    assert worst < 0.1           # a correct fp32 sum is far inside the rule (measured 0.04)
    conv_close(y, yo, bound)
    conv_rel_close_bf16(_bf16_round(y), yo, scale)


def test_bf16_rounded_partials_fail(site):
    x, xp, wt, yo, scale, bound = site
    y = _conv_split_k(x, xp, wt, 6, round_partials=True)
    with pytest.raises(AssertionError):
        conv_rel_close(y, yo, scale)
    with pytest.raises(AssertionError):
        conv_rel_close_bf16(_bf16_round(y), yo, scale)
    # the worst-case summation bound alone does not see this bug
    assert conv_close(y, yo, bound) <= 1.0


def test_wrong_group_map_fails(site):
    """A channel-to-group map off by one group moves most outputs by ~|y|."""
    x, xp, wt, yo, scale, _ = site
    y = np.roll(yo, 16, axis=-1)
    with pytest.raises(AssertionError):
        conv_rel_close(y, yo, scale)


def test_cancelling_taps_have_a_floor():
    """A site whose current-position tap is zero for one group (the weight
    rows of that group are zero): the floor keeps the allowance finite and
    the exact answer passes."""
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=2, block=4, d=256)
    x, xp, wt, _ = synth.conv_site(w, 0)
    wt = wt.clone()
    wt[3] = 0
    scale = conv_term_scale(x, xp, wt)
    assert np.all(scale > 0)
    yo = oracle.dynconv2(x, xp, wt, None)
    assert conv_rel_close(yo, yo, scale) == 0.0


# ------------------------------------------------------------------ path flips
def _lattice(B, T, K, seed):
    S = synth.pair_score_lattice(B, T, K, seed).numpy()
    idx = np.broadcast_to(np.arange(K, dtype=np.int32), (B, T, K)).copy()
    return S, idx


@pytest.mark.parametrize("mode", [oracle.PATH_VITERBI, oracle.PATH_GREEDY])
def test_compare_path_accepts_identical(mode):
    S, idx = _lattice(8, 7, 16, 5)
    op = oracle.path(S, idx, mode)
    r = compare_path(op["rank"].copy(), op, S, S, mode, 1.0, S.shape[1])
    assert r["bad"] == 0 and r["undecided_flips"] == 0


@pytest.mark.parametrize("mode", [oracle.PATH_VITERBI, oracle.PATH_GREEDY])
def test_compare_path_flags_a_flip_at_a_clear_decision(mode):
    """Change one decision of row 0 whose oracle margin is large: the row is
    bad although other rows' decisions may be close."""
    S, idx = _lattice(4, 7, 16, 6)
    op = oracle.path(S, idx, mode)
    g = op["rank"].copy()
    t = int(np.argmax(op["margin"][0]))
    g[0, t] = (g[0, t] + 1) % 16
    r = compare_path(g, op, S, S + 1e-7, mode, 1.0, S.shape[1])
    assert r["bad"] == 1


def _two_step_lattice(second_score: float):
    """B = 1, T = 2, K = 4: delta_0 = [1, 0, 0, 0]; at t = 1 only the edges
    0 -> 0 (score 5) and 0 -> 1 (score `second_score`) stand out, so the end
    decision compares 6 with 1 + second_score."""
    S = np.zeros((1, 2, 4, 4), np.float32)
    S[0, 0, 0] = [1, 0, 0, 0]
    S[0, 0, 1:] = -np.inf
    S[0, 1, 0, 0] = 5
    S[0, 1, 0, 1] = second_score
    return S, np.arange(4, dtype=np.int32).reshape(1, 1, 4).repeat(2, 1)


def test_compare_path_excuses_only_the_undecided_decision():
    """An exact tie in the end decision: the oracle takes end 0 (lowest
    rank); a path ending in 1 is excused.  With the runner-up 1.0 behind, the
    same path is a real mismatch."""
    S, idx = _two_step_lattice(5.0)
    op = oracle.path(S, idx, oracle.PATH_VITERBI)
    assert op["rank"].tolist() == [[0, 0]] and op["margin"][0, 1] == 0.0
    g = np.array([[0, 1]], np.int32)
    r = compare_path(g, op, S + np.float32(1e-6), S, oracle.PATH_VITERBI, 1.0, 2)
    assert r["bad"] == 0 and r["undecided_flips"] == 1 and r["excused_rows"] == [0]
    S, idx = _two_step_lattice(4.0)
    op = oracle.path(S, idx, oracle.PATH_VITERBI)
    assert op["rank"].tolist() == [[0, 0]]
    r = compare_path(g, op, S + np.float32(1e-6), S, oracle.PATH_VITERBI, 1.0, 2)
    assert r["bad"] == 1 and r["undecided_flips"] == 0

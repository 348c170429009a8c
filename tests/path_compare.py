"""Comparison of a GPU path with the oracle's path when the two ran on
slightly different pair scores (the chained cycle tests: each side computes
its own scores, equal within the 1e-3 score tolerance).

Only the decision that actually flipped is looked at, with the allowance
that the score difference gives for that decision:
  * VITERBI ("DFlash 2 讓 Qwen3.8-27B 快了兩倍", section "DFlash 2 的三個改進",
    item 2): the backtrack runs from the last position, so the flipped
    decision sits at the LAST position where the paths differ (later
    positions agree).  It compares two sums of n scores (n = T at the end
    argmax, t + 2 for the back-pointer that fixed c_t), each score off by at
    most max|dS|, so the allowance is 2 n max|dS| / max(1, |best|) in the
    oracle's relative margin units, plus the float rounding of the sums.
  * GREEDY and SAMPLE ("DFlash 2: Keep Drafting Parallel", section "A
    lightweight path selector"): the path runs forward, so the flipped
    decision is at the FIRST differing position.  Greedy compares two
    scores: 2 max|dS| / max(1, |best|).  Sampling compares u with a
    cumulative softmax, which moves by at most 2 max|dS| / tau.
A flip is excused only when the oracle margin of that one decision is under
NEAR_TIE plus this allowance; any other difference is a mismatch."""
import numpy as np

NEAR_TIE = 1e-6
U32 = 2.0 ** -24
PATH_VITERBI, PATH_GREEDY, PATH_SAMPLE = 0, 1, 2


def _path_values(S_row, rank_row):
    """Score of each step along a path: S[t, c_{t-1}, c_t] (t = 0: row 0)."""
    T = S_row.shape[0]
    prev = np.r_[0, rank_row[:-1]]
    return S_row[np.arange(T), prev, rank_row].astype(np.float64)


def compare_path(g_rank, o_path, S_g, S_o, mode, tau, T):
    fin = np.isfinite(S_o)
    dS = float(np.max(np.abs(np.asarray(S_g, np.float64)[fin] - np.asarray(S_o, np.float64)[fin]))) \
        if fin.any() else 0.0
    o_rank = o_path["rank"]
    undecided, bad, excused = 0, 0, []
    for b in range(g_rank.shape[0]):
        diff = np.flatnonzero(g_rank[b] != o_rank[b])
        if diff.size == 0:
            continue
        steps = _path_values(S_o[b], o_rank[b])
        if mode == PATH_VITERBI:
            t = int(diff[-1])
            n = T if t == T - 1 else t + 2
            best = abs(float(np.sum(steps[: min(t + 2, T)])))
            allow = 2 * n * dS / max(1.0, best) + 2 * n * U32
        elif mode == PATH_GREEDY:
            t = int(diff[0])
            allow = 2 * dS / max(1.0, abs(float(steps[t]))) + 2 * U32
        else:
            t = int(diff[0])
            allow = 2 * dS / float(tau)
        if float(o_path["margin"][b, t]) < NEAR_TIE + allow:
            undecided += 1
            excused.append(b)
        else:
            bad += 1
    near = int((o_path["margin"] < NEAR_TIE).sum())
    return dict(max_dS=dS, undecided_flips=undecided, bad=bad, near_ties=near, excused_rows=excused)

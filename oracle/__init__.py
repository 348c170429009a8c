"""ctypes wrapper around the CPU oracle (oracle/dflash2_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product path.  Inputs are
host numpy arrays (or CPU torch tensors); bf16 tensors are passed as their
raw 16-bit patterns.  Every function returns fresh numpy outputs.

Parity status per function (details in the C source):
  topk, project, pair_scores, path, verify_greedy, verify_reject, dynconv2,
  lm_head_topk, verify_greedy_head, verify_reject_head, philox -- all pinned by the CPU tests in
  tests/test_oracle_*.py;
  selector_tables, pair_scores_tab (numpy, below) -- pinned by
  tests/test_oracle_tables.py.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DFLASH2_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

FP32, BF16, FP16 = 0, 1, 2
PATH_VITERBI, PATH_GREEDY, PATH_SAMPLE = 0, 1, 2
GATE_IDENTITY, GATE_SIGMOID = 0, 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = C.c_void_p
I32, I64, U64, F64 = C.c_int32, C.c_int64, C.c_uint64, C.c_double


def _declare(L):
    L.oracle_set_num_threads.argtypes = [C.c_int]
    L.oracle_get_num_threads.restype = C.c_int
    L.oracle_philox4x64_10.argtypes = [U64, U64, P, P]
    L.oracle_uniform_from_word.argtypes = [U64]
    L.oracle_uniform_from_word.restype = F64
    L.oracle_topk.argtypes = [P, C.c_int, I64, I64, C.c_int, P, P]
    L.oracle_project.argtypes = [P, C.c_int, I64, C.c_int, P, C.c_int, C.c_int, P]
    L.oracle_pair_scores.argtypes = [P, P, P, P, C.c_int, I64, P, P, P, P, C.c_int, C.c_int,
                                     C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P, P]
    L.oracle_path.argtypes = [P, P, C.c_int, C.c_int, C.c_int, C.c_int, F64, U64, P, P, P, P, P, P]
    L.oracle_verify_greedy.argtypes = [P, C.c_int, I64, P, C.c_int, C.c_int, P, P, P]
    L.oracle_verify_reject.argtypes = [P, C.c_int, I64, P, P, P, P, C.c_int, C.c_int, C.c_int,
                                       F64, U64, P, P, P, P, P, P]
    L.oracle_dynconv2.argtypes = [P, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, P]
    L.oracle_lm_head_topk.argtypes = [P, P, I64, I64, C.c_int, C.c_int, P, P]
    L.oracle_verify_greedy_head.argtypes = [P, P, I64, C.c_int, P, C.c_int, C.c_int, P, P, P, P]
    L.oracle_verify_reject_head.argtypes = [P, P, I64, C.c_int, P, P, P, P, C.c_int, C.c_int, C.c_int, F64,
                                            U64, P, P, P, P, P, P]
    for f in ("oracle_topk", "oracle_project", "oracle_pair_scores", "oracle_path",
              "oracle_verify_greedy", "oracle_verify_reject", "oracle_dynconv2",
              "oracle_lm_head_topk", "oracle_verify_greedy_head", "oracle_verify_reject_head"):
        getattr(L, f).restype = C.c_int


class OracleError(RuntimeError):
    pass


def _check(rc, name):
    if rc != 0:
        raise OracleError(f"{name} returned {rc}")


def host(x, dtype=None):
    """Contiguous host numpy array from a numpy array or a torch tensor.
    bf16 / fp16 torch tensors become uint16 bit patterns plus a dtype code."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), BF16
        if x.dtype == torch.float16:
            return x.view(torch.int16).numpy().view(np.uint16), FP16
        x = x.numpy()
    x = np.ascontiguousarray(x if dtype is None else x.astype(dtype))
    code = {np.dtype(np.float32): FP32}.get(x.dtype, None)
    return x, code


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def set_num_threads(n: int):
    lib().oracle_set_num_threads(int(n))


def num_threads() -> int:
    return int(lib().oracle_get_num_threads())


def philox(seed: int, counter, key1: int = 0) -> np.ndarray:
    ctr = np.ascontiguousarray(np.array(counter, dtype=np.uint64).reshape(4))
    out = np.zeros(4, dtype=np.uint64)
    lib().oracle_philox4x64_10(int(seed) & (2**64 - 1), int(key1), _ptr(ctr), _ptr(out))
    return out


def uniform_from_word(w: int) -> float:
    return float(lib().oracle_uniform_from_word(int(w)))


def topk(logits, k: int):
    """logits [..., V] (fp32/bf16/fp16) -> (idx int32 [..., k], val fp32 [..., k])."""
    a, dt = host(logits)
    if dt is None:
        a, dt = host(a, np.float32)
    V = a.shape[-1]
    rows = int(np.prod(a.shape[:-1]))
    idx = np.zeros(a.shape[:-1] + (k,), dtype=np.int32)
    val = np.zeros(a.shape[:-1] + (k,), dtype=np.float32)
    _check(lib().oracle_topk(_ptr(a), dt, rows, V, k, _ptr(idx), _ptr(val)), "oracle_topk")
    return idx, val


def lm_head_topk(h, emb, k: int):
    """Drafter logits z = h E^T (float64) through the shared LM head, then
    the k best per row.  h [rows, d] bf16, emb [V, d] bf16 ->
    (idx int32 [rows, k], val float64 [rows, k])."""
    ha, hdt = host(h)
    ea, edt = host(emb)
    assert hdt == BF16 and edt == BF16
    rows, d = ha.shape
    V = ea.shape[0]
    idx = np.zeros((rows, k), np.int32)
    val = np.zeros((rows, k), np.float64)
    _check(lib().oracle_lm_head_topk(_ptr(ha), _ptr(ea), rows, V, d, k, _ptr(idx), _ptr(val)),
           "oracle_lm_head_topk")
    return idx, val


def project(x, w, gate: int = GATE_IDENTITY) -> np.ndarray:
    """x [n, d] (bf16 or fp32), w [r, d] bf16 -> gate(x @ w.T) in float64."""
    xa, xdt = host(x)
    if xdt is None:
        xa, xdt = host(xa, np.float32)
    wa, wdt = host(w)
    assert wdt == BF16
    n, d = xa.shape
    r = wa.shape[0]
    out = np.zeros((n, r), dtype=np.float64)
    _check(lib().oracle_project(_ptr(xa), xdt, n, d, _ptr(wa), r, gate, _ptr(out)), "oracle_project")
    return out


def pair_scores(cand_idx, cand_val, last_tok, emb, h, w_a, w_b, w_h, gate: int = GATE_IDENTITY,
                intermediates: bool = False):
    ci = np.ascontiguousarray(np.asarray(host(cand_idx)[0], dtype=np.int32))
    cv = np.ascontiguousarray(np.asarray(host(cand_val)[0], dtype=np.float32))
    lt = np.ascontiguousarray(np.asarray(host(last_tok)[0], dtype=np.int32))
    ea, edt = host(emb)
    if edt is None:
        ea, edt = host(ea, np.float32)
    ha, hdt = host(h)
    wa, _ = host(w_a)
    wb, _ = host(w_b)
    wh, _ = host(w_h)
    assert hdt == BF16
    B, T, K = ci.shape
    V, d = ea.shape
    r = wa.shape[0]
    S = np.zeros((B, T, K, K), dtype=np.float32)
    outs = [None] * 4
    if intermediates:
        outs = [np.zeros((B, r), np.float32), np.zeros((B, T, K, r), np.float32),
                np.zeros((B, T, K, r), np.float32), np.zeros((B, T, r), np.float32)]
    _check(lib().oracle_pair_scores(_ptr(ci), _ptr(cv), _ptr(lt), _ptr(ea), edt, V, _ptr(ha),
                                    _ptr(wa), _ptr(wb), _ptr(wh), B, T, K, d, r, gate, _ptr(S),
                                    *[_ptr(o) for o in outs]), "oracle_pair_scores")
    if intermediates:
        return S, dict(a_last=outs[0], a_cand=outs[1], b_cand=outs[2], h=outs[3])
    return S


def selector_tables(emb, w_a, w_b, rows=None) -> np.ndarray:
    """Per-token rows of the selector: "DFlash 2: Keep Drafting Parallel",
    section "A lightweight path selector" gives every token its own compact
    rank-r vectors A(tok) and B(tok), read as A(v) = W_A E[v] and
    B(v) = W_B E[v].  Returns [A(v) | B(v)] in float64 for the token ids
    `rows` (default: every token), one row per id.  emb: torch bf16 [V, d];
    w_a, w_b: bf16 [r, d]."""
    import torch
    V = emb.shape[0]
    ids = torch.arange(V) if rows is None else torch.as_tensor(np.asarray(rows, np.int64))
    sub = emb[ids]
    return np.concatenate([project(sub, w_a), project(sub, w_b)], axis=1)


def pair_scores_tab(cand_idx, cand_val, last_tok, tab, h, w_h, gate: int = GATE_IDENTITY) -> np.ndarray:
    """Pair scores with A and B read from a per-token table: same section,
    equation S_t(a,b) = U_t(b) + <A(a) (.) H(h_t), B(b)>, where row v of
    tab [V, 2r] is [A(v) | B(v)] and ids outside [0, V) read zero rows.  At
    t = 0 the only predecessor is the last verified token (row a = 0, rows
    a >= 1 are -inf); for t >= 1 a ranges over the candidates of t - 1.
    H = gate(W_H h_t) by project().  Sums in float64, rounded once to
    float32."""
    ci = np.asarray(host(cand_idx)[0], np.int64)
    U = np.asarray(host(cand_val)[0], np.float64)
    lt = np.asarray(host(last_tok)[0], np.int64)
    tb = np.asarray(host(tab)[0], np.float64)
    V, r2 = tb.shape
    r = r2 // 2
    B, T, K = ci.shape
    d = h.shape[-1]
    H = project(h.reshape(B * T, d), w_h, gate).reshape(B, T, r)

    def rows(ids):
        out = np.zeros(ids.shape + (r2,))
        ok = (ids >= 0) & (ids < V)
        out[ok] = tb[ids[ok]]
        return out
    cand_rows = rows(ci)
    A_c, B_c = cand_rows[..., :r], cand_rows[..., r:]
    A_last = rows(lt)[:, :r]
    S = np.full((B, T, K, K), -np.inf)
    for b in range(B):
        for t in range(T):
            pred = A_last[b][None, :] if t == 0 else A_c[b, t - 1]     # [P, r]
            bigram = (pred * H[b, t][None, :]) @ B_c[b, t].T          # [P, K]
            S[b, t, :pred.shape[0], :] = U[b, t][None, :] + bigram
    return S.astype(np.float32)


def _bids(b_ids, B):
    if b_ids is None:
        return None
    a = np.ascontiguousarray(np.asarray(b_ids, dtype=np.int32).reshape(B))
    return a


def path(scores, cand_idx, mode: int, temperature: float = 0.0, seed: int = 0, b_ids=None):
    """-> dict(rank, tok, q, score, margin).  b_ids: request index per row
    for the Philox counter (default: the row number)."""
    S = np.ascontiguousarray(np.asarray(host(scores)[0], dtype=np.float32))
    ci = np.ascontiguousarray(np.asarray(host(cand_idx)[0], dtype=np.int32))
    B, T, K, _ = S.shape
    rank = np.zeros((B, T), np.int32)
    tok = np.zeros((B, T), np.int32)
    q = np.zeros((B, T, K), np.float32)
    score = np.zeros((B,), np.float32)
    margin = np.zeros((B, T), np.float64)
    bi = _bids(b_ids, B)
    _check(lib().oracle_path(_ptr(S), _ptr(ci), B, T, K, mode, float(temperature),
                             int(seed) & (2**64 - 1), _ptr(bi), _ptr(rank), _ptr(tok), _ptr(q),
                             _ptr(score), _ptr(margin)), "oracle_path")
    return dict(rank=rank, tok=tok, q=q, score=score, margin=margin)


def verify_greedy(target, path_tok):
    za, zdt = host(target)
    if zdt is None:
        za, zdt = host(za, np.float32)
    pt = np.ascontiguousarray(np.asarray(host(path_tok)[0], dtype=np.int32))
    B, T = pt.shape
    V = za.shape[-1]
    assert za.shape[:2] == (B, T + 1)
    acc = np.zeros((B,), np.int32)
    out = np.zeros((B, T + 1), np.int32)
    am = np.zeros((B, T + 1), np.int32)
    _check(lib().oracle_verify_greedy(_ptr(za), zdt, V, _ptr(pt), B, T, _ptr(acc), _ptr(out),
                                      _ptr(am)), "oracle_verify_greedy")
    return dict(accept_len=acc, out_tok=out, argmax=am)


def verify_greedy_head(h, emb, path_tok):
    """Greedy verification with the target logits computed from its final
    hidden states h [B, T+1, d] (bf16) through its LM head emb [V, d] (bf16),
    in float64.  -> dict(accept_len, out_tok, argmax, margin) (margin: the
    argmax logit minus the runner-up, per row)."""
    ha, hdt = host(h)
    ea, edt = host(emb)
    assert hdt == BF16 and edt == BF16
    pt = np.ascontiguousarray(np.asarray(host(path_tok)[0], dtype=np.int32))
    B, T = pt.shape
    V, d = ea.shape
    assert ha.shape == (B, T + 1, d)
    acc = np.zeros((B,), np.int32)
    out = np.zeros((B, T + 1), np.int32)
    am = np.zeros((B, T + 1), np.int32)
    mg = np.zeros((B, T + 1), np.float64)
    _check(lib().oracle_verify_greedy_head(_ptr(ha), _ptr(ea), V, d, _ptr(pt), B, T, _ptr(acc), _ptr(out),
                                           _ptr(am), _ptr(mg)), "oracle_verify_greedy_head")
    return dict(accept_len=acc, out_tok=out, argmax=am, margin=mg)


def verify_reject(target, path_tok, path_rank, cand_idx, q, temperature: float, seed: int,
                  b_ids=None):
    za, zdt = host(target)
    if zdt is None:
        za, zdt = host(za, np.float32)
    pt = np.ascontiguousarray(np.asarray(host(path_tok)[0], dtype=np.int32))
    pr = np.ascontiguousarray(np.asarray(host(path_rank)[0], dtype=np.int32))
    ci = np.ascontiguousarray(np.asarray(host(cand_idx)[0], dtype=np.int32))
    qa = np.ascontiguousarray(np.asarray(host(q)[0], dtype=np.float32))
    B, T = pt.shape
    K = ci.shape[-1]
    V = za.shape[-1]
    assert za.shape[:2] == (B, T + 1)
    acc = np.zeros((B,), np.int32)
    out = np.zeros((B, T + 1), np.int32)
    ma = np.zeros((B, T), np.float64)
    ms = np.zeros((B,), np.float64)
    fb = np.zeros((1,), np.int32)
    bi = _bids(b_ids, B)
    _check(lib().oracle_verify_reject(_ptr(za), zdt, V, _ptr(pt), _ptr(pr), _ptr(ci), _ptr(qa), B, T,
                                      K, float(temperature), int(seed) & (2**64 - 1), _ptr(bi),
                                      _ptr(acc),
                                      _ptr(out), _ptr(ma), _ptr(ms), _ptr(fb)),
           "oracle_verify_reject")
    return dict(accept_len=acc, out_tok=out, margin_accept=ma, margin_sample=ms,
                fallbacks=int(fb[0]))


def verify_reject_head(h, emb, path_tok, path_rank, cand_idx, q, temperature: float, seed: int, b_ids=None):
    """Rejection-sampling verification with the target logits computed in
    float64 from its hidden states h [B, T+1, d] through its LM head emb
    [V, d] (both bf16); outputs as verify_reject."""
    ha, hdt = host(h)
    ea, edt = host(emb)
    assert hdt == BF16 and edt == BF16
    pt = np.ascontiguousarray(np.asarray(host(path_tok)[0], dtype=np.int32))
    pr = np.ascontiguousarray(np.asarray(host(path_rank)[0], dtype=np.int32))
    ci = np.ascontiguousarray(np.asarray(host(cand_idx)[0], dtype=np.int32))
    qa = np.ascontiguousarray(np.asarray(host(q)[0], dtype=np.float32))
    B, T = pt.shape
    K = ci.shape[-1]
    V, d = ea.shape
    assert ha.shape == (B, T + 1, d)
    acc = np.zeros((B,), np.int32)
    out = np.zeros((B, T + 1), np.int32)
    ma = np.zeros((B, T), np.float64)
    ms = np.zeros((B,), np.float64)
    fb = np.zeros((1,), np.int32)
    bi = _bids(b_ids, B)
    _check(lib().oracle_verify_reject_head(_ptr(ha), _ptr(ea), V, d, _ptr(pt), _ptr(pr), _ptr(ci), _ptr(qa), B, T,
                                           K, float(temperature), int(seed) & (2**64 - 1), _ptr(bi), _ptr(acc),
                                           _ptr(out), _ptr(ma), _ptr(ms), _ptr(fb)), "oracle_verify_reject_head")
    return dict(accept_len=acc, out_tok=out, margin_accept=ma, margin_sample=ms, fallbacks=int(fb[0]))


def dynconv2(x, x_prev, w, base=None, group: int = 16) -> np.ndarray:
    """x [B, L, d] bf16, x_prev [B, d] bf16 or None, w [2G, d] bf16,
    base [2, d] fp32 or None -> y [B, L, d] fp32."""
    xa, xdt = host(x)
    wa, wdt = host(w)
    assert xdt == BF16 and wdt == BF16
    xp = None
    if x_prev is not None:
        xp, pdt = host(x_prev)
        assert pdt == BF16
    bs = None
    if base is not None:
        bs = np.ascontiguousarray(np.asarray(host(base)[0], dtype=np.float32))
    B, L, d = xa.shape
    y = np.zeros((B, L, d), np.float32)
    _check(lib().oracle_dynconv2(_ptr(xa), _ptr(xp), _ptr(wa), _ptr(bs), B, L, d, group, _ptr(y)),
           "oracle_dynconv2")
    return y

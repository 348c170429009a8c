"""Python binding of libdflash2.so, the MI355X (gfx950) DFlash 2 draft-block
library.

The functions below carry the names of the C ABI (include/dflash2.h) and do
argument marshalling only: they read sizes from tensor shapes, pass device
pointers and the current HIP stream, and raise DFlash2Error on a non-zero
status.  Every step of the path runs in the library's HIP kernels; PyTorch
supplies device memory and streams.  There is no fallback: if the library is
missing, importing a function raises.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdflash2.so")

DF2_OK, DF2_ERR_NULL, DF2_ERR_DTYPE, DF2_ERR_SHAPE, DF2_ERR_WORKSPACE, DF2_ERR_UNSUPPORTED, \
    DF2_ERR_HIP = range(7)
DF2_FP32, DF2_BF16, DF2_FP16 = 0, 1, 2
DF2_PATH_VITERBI, DF2_PATH_GREEDY, DF2_PATH_SAMPLE = 0, 1, 2
DF2_GATE_IDENTITY, DF2_GATE_SIGMOID = 0, 1

EXPORTS = [
    "dflash2_abi_version", "dflash2_status_string", "dflash2_last_error", "dflash2_init",
    "dflash2_topk_workspace_bytes", "dflash2_topk",
    "dflash2_lm_head_topk_workspace_bytes", "dflash2_lm_head_topk",
    "dflash2_pair_scores_workspace_bytes", "dflash2_pair_scores",
    "dflash2_selector_tables", "dflash2_pair_scores_tab_workspace_bytes", "dflash2_pair_scores_tab",
    "dflash2_h_projection", "dflash2_pair_scores_tab_from_h",
    "dflash2_path_viterbi",
    "dflash2_dynconv2_workspace_bytes", "dflash2_dynconv2",
    "dflash2_verify_workspace_bytes", "dflash2_verify_greedy", "dflash2_verify_reject",
    "dflash2_verify_greedy_noalloc", "dflash2_verify_greedy_noalloc_max_bytes",
    "dflash2_verify_greedy_head_workspace_bytes", "dflash2_verify_greedy_head",
    "dflash2_verify_reject_head_workspace_bytes", "dflash2_verify_reject_head",
    "dflash2_cycle_fused_workspace_bytes", "dflash2_cycle_fused_init", "dflash2_cycle_fused",
    "dflash2_philox4x64", "dflash2_profile_start", "dflash2_profile_stop",
]


class DFlash2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


_lib = None
P, I, I64, SZ, F = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_float


def lib():
    """Load libdflash2.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        L.dflash2_abi_version.restype = I
        L.dflash2_status_string.argtypes = [I]
        L.dflash2_status_string.restype = C.c_char_p
        L.dflash2_last_error.restype = C.c_char_p
        L.dflash2_init.restype = I
        L.dflash2_topk_workspace_bytes.argtypes = [I64, I64, I]
        L.dflash2_topk_workspace_bytes.restype = SZ
        L.dflash2_topk.argtypes = [P, I, I64, I64, I, P, P, P, SZ, P]
        L.dflash2_lm_head_topk_workspace_bytes.argtypes = [I, I64, I, I]
        L.dflash2_lm_head_topk_workspace_bytes.restype = SZ
        L.dflash2_lm_head_topk.argtypes = [P, P, I, I64, I, I, I, P, P, P, SZ, P]
        L.dflash2_pair_scores_workspace_bytes.argtypes = [I, I, I, I, I]
        L.dflash2_pair_scores_workspace_bytes.restype = SZ
        L.dflash2_pair_scores.argtypes = [P, P, P, P, I, I64, P, P, P, P, I, I, I, I, I, I, P, P, SZ, P]
        L.dflash2_selector_tables.argtypes = [P, I, I64, I, P, P, I, P, P]
        L.dflash2_pair_scores_tab_workspace_bytes.argtypes = [I, I, I, I]
        L.dflash2_pair_scores_tab_workspace_bytes.restype = SZ
        L.dflash2_pair_scores_tab.argtypes = [P, P, P, P, I64, P, P, I, I, I, I, I, I, P, P, SZ, P]
        L.dflash2_h_projection.argtypes = [P, P, I, I, I, I, P, SZ, P]
        L.dflash2_pair_scores_tab_from_h.argtypes = [P, P, P, P, I64, I, I, I, I, I, I, P, P, SZ, P]
        L.dflash2_path_viterbi.argtypes = [P, P, I, I, I, I, F, P, I, P, P, P, P, P]
        L.dflash2_dynconv2_workspace_bytes.argtypes = [I, I, I, I]
        L.dflash2_dynconv2_workspace_bytes.restype = SZ
        L.dflash2_dynconv2.argtypes = [P, P, P, P, I, I, I, I, P, I, P, SZ, P]
        L.dflash2_verify_workspace_bytes.argtypes = [I, I, I64]
        L.dflash2_verify_workspace_bytes.restype = SZ
        L.dflash2_verify_greedy.argtypes = [P, I, I64, P, I, I, P, P, P, SZ, P]
        L.dflash2_verify_reject.argtypes = [P, I, I64, P, P, P, P, I, I, I, F, P, I, P, P, P, SZ, P]
        L.dflash2_verify_greedy_noalloc.argtypes = [P, I, I64, P, I, I, P, P, P]
        L.dflash2_verify_greedy_head_workspace_bytes.argtypes = [I, I, I64, I]
        L.dflash2_verify_greedy_head_workspace_bytes.restype = SZ
        L.dflash2_verify_greedy_head.argtypes = [P, P, I, I64, I, P, I, I, P, P, P, SZ, P]
        L.dflash2_verify_reject_head_workspace_bytes.argtypes = [I, I, I64, I, I]
        L.dflash2_verify_reject_head_workspace_bytes.restype = SZ
        L.dflash2_verify_reject_head.argtypes = [P, P, I, I64, I, P, P, P, P, I, I, I, F, P, I, P, P, P, SZ, P]
        L.dflash2_cycle_fused_workspace_bytes.argtypes = [I, I, I, I64, I, I]
        L.dflash2_cycle_fused_workspace_bytes.restype = SZ
        L.dflash2_cycle_fused_init.argtypes = [I, I, I, I64, I, I, P, SZ, P]
        L.dflash2_cycle_fused.argtypes = [P, I, P, I, I64, P, I, P, P, P, P, P, I, I, I, I, I, I, I,
                                          P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.dflash2_verify_greedy_noalloc_max_bytes.restype = SZ
        L.dflash2_philox4x64.argtypes = [P, P, P, I, P, P]
        L.dflash2_profile_start.argtypes = [C.c_char_p, I]
        L.dflash2_profile_start.restype = I
        L.dflash2_profile_stop.argtypes = [P, I, P]
        L.dflash2_profile_stop.restype = I
        for name in ("dflash2_topk", "dflash2_lm_head_topk", "dflash2_pair_scores", "dflash2_selector_tables",
                     "dflash2_pair_scores_tab", "dflash2_h_projection", "dflash2_pair_scores_tab_from_h",
                     "dflash2_path_viterbi",
                     "dflash2_dynconv2", "dflash2_verify_greedy", "dflash2_verify_reject",
                     "dflash2_verify_greedy_noalloc", "dflash2_verify_greedy_head", "dflash2_verify_reject_head",
                     "dflash2_cycle_fused_init", "dflash2_cycle_fused",
                     "dflash2_philox4x64"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dt(t: torch.Tensor) -> int:
    return {torch.float32: DF2_FP32, torch.bfloat16: DF2_BF16, torch.float16: DF2_FP16}.get(t.dtype, 99)


def _check(status: int, name: str):
    if status != DF2_OK:
        msg = lib().dflash2_last_error().decode(errors="replace")
        raise DFlash2Error(status, f"{name}: {msg}")


def _bytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


def dflash2_abi_version() -> int:
    return int(lib().dflash2_abi_version())


def dflash2_status_string(status: int) -> str:
    return lib().dflash2_status_string(int(status)).decode()


def dflash2_init():
    _check(lib().dflash2_init(), "dflash2_init")


def dflash2_topk_workspace_bytes(rows: int, vocab: int, k: int) -> int:
    return int(lib().dflash2_topk_workspace_bytes(rows, vocab, k))


def dflash2_topk(logits, k, out_idx, out_val, ws=None, stream=None):
    """logits [..., V] -> out_idx int32 [..., k], out_val fp32 [..., k]."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    _check(lib().dflash2_topk(_ptr(logits), _dt(logits), rows, V, int(k), _ptr(out_idx), _ptr(out_val),
                              _ptr(ws), _bytes(ws), _stream(stream)), "dflash2_topk")


def dflash2_lm_head_topk_workspace_bytes(rows: int, vocab: int, d: int, k: int) -> int:
    return int(lib().dflash2_lm_head_topk_workspace_bytes(rows, vocab, d, k))


def dflash2_lm_head_topk(h, emb, k, out_idx, out_val, ws, stream=None):
    """h [..., d] bf16, emb [V, d] bf16 -> the k best tokens of h E^T per row
    (out_idx int32 [..., k], out_val fp32 [..., k])."""
    d = h.shape[-1]
    rows = h.numel() // d if d else 0
    V = emb.shape[0]
    _check(lib().dflash2_lm_head_topk(_ptr(h), _ptr(emb), _dt(emb), V, rows, d, int(k), _ptr(out_idx),
                                      _ptr(out_val), _ptr(ws), _bytes(ws), _stream(stream)),
           "dflash2_lm_head_topk")


def dflash2_pair_scores_workspace_bytes(B, T, K, d, r) -> int:
    return int(lib().dflash2_pair_scores_workspace_bytes(B, T, K, d, r))


def dflash2_pair_scores(cand_idx, cand_val, last_tok, emb, h, w_a, w_b, w_h, scores, ws,
                        gate=DF2_GATE_IDENTITY, stream=None):
    B, T, K = cand_idx.shape
    V, d = emb.shape
    r = w_a.shape[0]
    _check(lib().dflash2_pair_scores(_ptr(cand_idx), _ptr(cand_val), _ptr(last_tok), _ptr(emb), _dt(emb),
                                     V, _ptr(h), _ptr(w_a), _ptr(w_b), _ptr(w_h), B, T, K, d, r,
                                     int(gate), _ptr(scores), _ptr(ws), _bytes(ws), _stream(stream)),
           "dflash2_pair_scores")


def dflash2_selector_tables(emb, w_a, w_b, tab, stream=None):
    """tab [V, 2r] fp32 <- [E W_A^T | E W_B^T] for every token."""
    V, d = emb.shape
    r = w_a.shape[0]
    _check(lib().dflash2_selector_tables(_ptr(emb), _dt(emb), V, d, _ptr(w_a), _ptr(w_b), r, _ptr(tab),
                                         _stream(stream)), "dflash2_selector_tables")


def dflash2_pair_scores_tab_workspace_bytes(B, T, d, r) -> int:
    return int(lib().dflash2_pair_scores_tab_workspace_bytes(B, T, d, r))


def dflash2_pair_scores_tab(cand_idx, cand_val, last_tok, tab, h, w_h, scores, ws,
                            gate=DF2_GATE_IDENTITY, stream=None):
    B, T, K = cand_idx.shape
    V, r2 = tab.shape
    d = h.shape[-1]
    _check(lib().dflash2_pair_scores_tab(_ptr(cand_idx), _ptr(cand_val), _ptr(last_tok), _ptr(tab), V,
                                         _ptr(h), _ptr(w_h), B, T, K, d, r2 // 2, int(gate), _ptr(scores),
                                         _ptr(ws), _bytes(ws), _stream(stream)), "dflash2_pair_scores_tab")


def dflash2_h_projection(h, w_h, ws, stream=None):
    """H's partial products for dflash2_pair_scores_tab_from_h (h [B, T, d])."""
    B, T, d = h.shape
    _check(lib().dflash2_h_projection(_ptr(h), _ptr(w_h), B, T, d, w_h.shape[0], _ptr(ws), _bytes(ws),
                                      _stream(stream)), "dflash2_h_projection")


def dflash2_pair_scores_tab_from_h(cand_idx, cand_val, last_tok, tab, d, scores, ws,
                                   gate=DF2_GATE_IDENTITY, stream=None):
    B, T, K = cand_idx.shape
    V, r2 = tab.shape
    _check(lib().dflash2_pair_scores_tab_from_h(_ptr(cand_idx), _ptr(cand_val), _ptr(last_tok), _ptr(tab), V,
                                                B, T, K, int(d), r2 // 2, int(gate), _ptr(scores), _ptr(ws),
                                                _bytes(ws), _stream(stream)), "dflash2_pair_scores_tab_from_h")


def dflash2_path_viterbi(scores, cand_idx, mode, path_rank, path_tok, q, path_score=None,
                         temperature=0.0, seed_dev=None, b0=0, stream=None):
    """b0: index of scores[0]'s request in the batch the seed covers."""
    B, T, K, _ = scores.shape
    _check(lib().dflash2_path_viterbi(_ptr(scores), _ptr(cand_idx), B, T, K, int(mode),
                                      float(temperature), _ptr(seed_dev), int(b0), _ptr(path_rank),
                                      _ptr(path_tok), _ptr(q), _ptr(path_score), _stream(stream)),
           "dflash2_path_viterbi")


def dflash2_dynconv2_workspace_bytes(B, L, d, group=16) -> int:
    return int(lib().dflash2_dynconv2_workspace_bytes(B, L, d, group))


def dflash2_dynconv2(x, x_prev, w, base, y, ws, group=16, stream=None):
    B, L, d = x.shape
    _check(lib().dflash2_dynconv2(_ptr(x), _ptr(x_prev), _ptr(w), _ptr(base), B, L, d, int(group),
                                  _ptr(y), _dt(y), _ptr(ws), _bytes(ws), _stream(stream)),
           "dflash2_dynconv2")


def dflash2_verify_workspace_bytes(B, T, vocab) -> int:
    return int(lib().dflash2_verify_workspace_bytes(B, T, vocab))


def dflash2_verify_greedy(target, path_tok, accept_len, out_tok, ws, stream=None):
    B, T1, V = target.shape
    _check(lib().dflash2_verify_greedy(_ptr(target), _dt(target), V, _ptr(path_tok), B, T1 - 1,
                                       _ptr(accept_len), _ptr(out_tok), _ptr(ws), _bytes(ws),
                                       _stream(stream)), "dflash2_verify_greedy")


def dflash2_verify_greedy_head_workspace_bytes(B: int, T: int, vocab: int, d: int) -> int:
    return int(lib().dflash2_verify_greedy_head_workspace_bytes(B, T, vocab, d))


def dflash2_verify_greedy_head(h, emb, path_tok, accept_len, out_tok, ws, stream=None):
    """Greedy verification with the target logits computed from its hidden
    states h [B, T+1, d] through its LM head emb [V, d] (both bf16)."""
    B, T1, d = h.shape
    V = emb.shape[0]
    _check(lib().dflash2_verify_greedy_head(_ptr(h), _ptr(emb), _dt(emb), V, d, _ptr(path_tok), B, T1 - 1,
                                            _ptr(accept_len), _ptr(out_tok), _ptr(ws), _bytes(ws),
                                            _stream(stream)), "dflash2_verify_greedy_head")


def dflash2_verify_reject_head_workspace_bytes(B: int, T: int, vocab: int, d: int, K: int) -> int:
    return int(lib().dflash2_verify_reject_head_workspace_bytes(B, T, vocab, d, K))


def dflash2_verify_reject_head(h, emb, path_tok, path_rank, cand_idx, q, temperature, seed_dev,
                               accept_len, out_tok, ws, b0=0, stream=None):
    """Rejection verification with the target logits computed from its
    hidden states h [B, T+1, d] through its LM head emb [V, d] (both bf16).
    b0: index of h[0]'s request in the batch the seed covers."""
    B, T1, d = h.shape
    V = emb.shape[0]
    K = cand_idx.shape[-1]
    _check(lib().dflash2_verify_reject_head(_ptr(h), _ptr(emb), _dt(emb), V, d, _ptr(path_tok), _ptr(path_rank),
                                            _ptr(cand_idx), _ptr(q), B, T1 - 1, K, float(temperature),
                                            _ptr(seed_dev), int(b0), _ptr(accept_len), _ptr(out_tok), _ptr(ws),
                                            _bytes(ws), _stream(stream)), "dflash2_verify_reject_head")


def dflash2_cycle_fused_workspace_bytes(B: int, T: int, K: int, vocab: int, d: int, r: int) -> int:
    return int(lib().dflash2_cycle_fused_workspace_bytes(B, T, K, vocab, d, r))


def dflash2_cycle_fused_init(B: int, T: int, K: int, vocab: int, d: int, r: int, ws, stream=None):
    """Zero the control words of a fresh dflash2_cycle_fused workspace."""
    _check(lib().dflash2_cycle_fused_init(B, T, K, vocab, d, r, _ptr(ws), _bytes(ws), _stream(stream)),
           "dflash2_cycle_fused_init")


def dflash2_cycle_fused(logits, target, emb, h, w_a, w_b, w_h, last_tok, path_mode, cand_idx, cand_val, scores,
                        path_rank, path_tok, q, path_score, accept_len, out_tok, status, ws,
                        gate=DF2_GATE_IDENTITY, stream=None):
    """top-K, pair scores, path (VITERBI / GREEDY) and greedy verification of
    a small batch in one launch; status [1] int32 receives 0 on success."""
    B, T, V = logits.shape
    K = cand_idx.shape[-1]
    d = emb.shape[1]
    r = w_a.shape[0]
    _check(lib().dflash2_cycle_fused(_ptr(logits), _dt(logits), _ptr(target), _dt(target), V, _ptr(emb), _dt(emb),
                                     _ptr(h), _ptr(w_a), _ptr(w_b), _ptr(w_h), _ptr(last_tok), B, T, K, d, r,
                                     int(gate), int(path_mode), _ptr(cand_idx), _ptr(cand_val), _ptr(scores),
                                     _ptr(path_rank), _ptr(path_tok), _ptr(q), _ptr(path_score), _ptr(accept_len),
                                     _ptr(out_tok), _ptr(status), _ptr(ws), _bytes(ws), _stream(stream)),
           "dflash2_cycle_fused")


def dflash2_verify_greedy_noalloc_max_bytes() -> int:
    return int(lib().dflash2_verify_greedy_noalloc_max_bytes())


def dflash2_verify_greedy_noalloc(target, path_tok, accept_len, out_tok, stream=None):
    """dflash2_verify_greedy with the library's fixed device scratch instead
    of a workspace (for callers that cannot allocate)."""
    B, T1, V = target.shape
    _check(lib().dflash2_verify_greedy_noalloc(_ptr(target), _dt(target), V, _ptr(path_tok), B, T1 - 1,
                                               _ptr(accept_len), _ptr(out_tok), _stream(stream)),
           "dflash2_verify_greedy_noalloc")


def dflash2_verify_reject(target, path_tok, path_rank, cand_idx, q, temperature, seed_dev,
                          accept_len, out_tok, ws, b0=0, stream=None):
    """b0: index of target[0]'s request in the batch the seed covers."""
    B, T1, V = target.shape
    K = cand_idx.shape[-1]
    _check(lib().dflash2_verify_reject(_ptr(target), _dt(target), V, _ptr(path_tok), _ptr(path_rank),
                                       _ptr(cand_idx), _ptr(q), B, T1 - 1, K, float(temperature),
                                       _ptr(seed_dev), int(b0), _ptr(accept_len), _ptr(out_tok), _ptr(ws),
                                       _bytes(ws), _stream(stream)), "dflash2_verify_reject")


def dflash2_philox4x64(seed_dev, b, t, out, stream=None):
    _check(lib().dflash2_philox4x64(_ptr(seed_dev), _ptr(b), _ptr(t), int(b.numel()), _ptr(out),
                                    _stream(stream)), "dflash2_philox4x64")


def dflash2_profile_start(kernel: str, max_launches: int):
    """Arm the kernel timing hook for one kernel tag (see include/dflash2.h)."""
    _check(lib().dflash2_profile_start(kernel.encode(), int(max_launches)), "dflash2_profile_start")


def dflash2_profile_stop(max_launches: int = 4096):
    """Per-launch durations (ms) of the armed kernel since profile_start."""
    import numpy as np
    ms = np.zeros(max_launches, np.float32)
    n = C.c_int(0)
    _check(lib().dflash2_profile_stop(ms.ctypes.data_as(C.c_void_p), max_launches, C.byref(n)),
           "dflash2_profile_stop")
    return ms[: n.value].astype(float).tolist()

"""One DFlash 2 verification cycle on the GPU, optionally captured as a HIP
graph.

Order of the steps (the cycle of "DFlash2 并行投机解码解读" §二 and of
"DFlash 2: Keep Drafting Parallel", Fig. 1): the two-tap convolution sites
of the drafter (dflash2_dynconv2), top-K candidates of the drafter's block
logits (dflash2_topk), all adjacent pair scores (dflash2_pair_scores), one
path (dflash2_path_viterbi), and verification against the target's logits
(dflash2_verify_greedy / dflash2_verify_reject, or both on two halves of the
batch).  The drafter and target forward passes themselves are outside this
library; their outputs (block logits, hidden states, target logits) are
inputs here.

All output and scratch buffers are allocated once, before any capture, so a
captured cycle allocates nothing.  With `tables=True` the per-token A/B
table [V, 2r] is built once at construction (dflash2_selector_tables) and
each cycle scores pairs from it (dflash2_pair_scores_tab), on one stream:
running H = W_H h_t on a second stream beside top-K measured slower (its
work-groups take CU slots from top-K's rows, and the join costs time in
the replayed graph).  The sampling seed lives in device memory
(`seed`), so a replay can run with a fresh seed written between replays.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import (DF2_GATE_IDENTITY, DF2_PATH_GREEDY, DF2_PATH_SAMPLE, DF2_PATH_VITERBI,
               dflash2_cycle_fused, dflash2_cycle_fused_init, dflash2_cycle_fused_workspace_bytes,
               dflash2_dynconv2, dflash2_dynconv2_workspace_bytes, dflash2_init,
               dflash2_pair_scores, dflash2_pair_scores_tab, dflash2_pair_scores_tab_workspace_bytes,
               dflash2_pair_scores_workspace_bytes, dflash2_path_viterbi, dflash2_selector_tables,
               dflash2_topk, dflash2_topk_workspace_bytes, dflash2_verify_greedy,
               dflash2_verify_reject, dflash2_verify_workspace_bytes)

PATH_MODES = {"viterbi": DF2_PATH_VITERBI, "greedy": DF2_PATH_GREEDY, "sample": DF2_PATH_SAMPLE}


@dataclasses.dataclass
class ConvSite:
    x: torch.Tensor                  # [B, L, d] bf16
    x_prev: Optional[torch.Tensor]   # [B, d] bf16
    w: torch.Tensor                  # [2G, d] bf16
    base: Optional[torch.Tensor]     # [2, d] fp32
    y: torch.Tensor                  # [B, L, d] bf16 or fp32


def _ws(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


class Cycle:
    """Static-buffer cycle for fixed shapes.

    verify: "greedy" | "reject" | "mixed" (first `greedy_rows` requests greedy,
    the rest rejection sampling).  tables: score pairs from per-token A/B
    tables built once here, instead of projecting the candidates' embedding
    rows every cycle.  fused: run top-K, pair scores, path and verification
    as one persistent launch (dflash2_cycle_fused; greedy verification,
    VITERBI or GREEDY paths, bf16 logits, B T <= 1024), with the same results.
    """

    def __init__(self, *, logits, target, emb, h, w_a, w_b, w_h, last_tok, K: int,
                 path_mode: str, verify: str, tau: float = 1.0, gate: int = DF2_GATE_IDENTITY,
                 conv_sites: Optional[List[ConvSite]] = None, greedy_rows: Optional[int] = None,
                 seed: int = 0, tables: bool = False, fused: bool = False):
        dflash2_init()
        dev = logits.device
        self.B, self.T, self.V = logits.shape
        self.K, self.d, self.r = K, emb.shape[1], w_a.shape[0]
        self.logits, self.target, self.emb, self.h = logits, target, emb, h
        self.w_a, self.w_b, self.w_h, self.last_tok = w_a, w_b, w_h, last_tok
        self.path_mode, self.verify, self.tau, self.gate = PATH_MODES[path_mode], verify, tau, gate
        self.greedy_rows = self.B // 2 if greedy_rows is None else greedy_rows
        self.conv_sites = conv_sites or []
        B, T, V = self.B, self.T, self.V
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.cand_idx = torch.empty((B, T, K), **i32)
        self.cand_val = torch.empty((B, T, K), **f32)
        self.scores = torch.empty((B, T, K, K), **f32)
        self.path_rank = torch.empty((B, T), **i32)
        self.path_tok = torch.empty((B, T), **i32)
        self.q = torch.empty((B, T, K), **f32)
        self.path_score = torch.empty((B,), **f32)
        self.accept_len = torch.empty((B,), **i32)
        self.out_tok = torch.empty((B, T + 1), **i32)
        self.seed = torch.full((1,), int(seed), dtype=torch.int64, device=dev)
        self.ws_topk = _ws(dflash2_topk_workspace_bytes(B * T, V, K), dev)
        self.tab = None
        if tables:
            self.tab = torch.empty((V, 2 * self.r), **f32)
            dflash2_selector_tables(emb, w_a, w_b, self.tab)
            self.ws_pair = _ws(dflash2_pair_scores_tab_workspace_bytes(B, T, self.d, self.r), dev)
        else:
            self.ws_pair = _ws(dflash2_pair_scores_workspace_bytes(B, T, K, self.d, self.r), dev)
        self.ws_verify = _ws(dflash2_verify_workspace_bytes(B, T, V), dev)
        self.fused = fused
        if fused:
            if verify != "greedy" or path_mode == "sample" or tables:
                raise ValueError("the fused cycle runs greedy verification with VITERBI or GREEDY paths")
            self.status = torch.zeros((1,), **i32)
            self.ws_fused = _ws(dflash2_cycle_fused_workspace_bytes(B, T, K, V, self.d, self.r), dev)
            dflash2_cycle_fused_init(B, T, K, V, self.d, self.r, self.ws_fused)
        conv_bytes = 0
        for s in self.conv_sites:
            Bc, L, dc = s.x.shape
            conv_bytes = max(conv_bytes, dflash2_dynconv2_workspace_bytes(Bc, L, dc))
        self.ws_conv = _ws(conv_bytes, dev)
        self.graph = None

    # -- the steps -----------------------------------------------------------
    def run_conv(self):
        for s in self.conv_sites:
            dflash2_dynconv2(s.x, s.x_prev, s.w, s.base, s.y, self.ws_conv)

    def run_topk(self):
        dflash2_topk(self.logits, self.K, self.cand_idx, self.cand_val, self.ws_topk)

    def run_pair_scores(self):
        if self.tab is not None:
            dflash2_pair_scores_tab(self.cand_idx, self.cand_val, self.last_tok, self.tab, self.h, self.w_h,
                                    self.scores, self.ws_pair, gate=self.gate)
            return
        dflash2_pair_scores(self.cand_idx, self.cand_val, self.last_tok, self.emb, self.h, self.w_a,
                            self.w_b, self.w_h, self.scores, self.ws_pair, gate=self.gate)

    def run_path(self):
        dflash2_path_viterbi(self.scores, self.cand_idx, self.path_mode, self.path_rank, self.path_tok,
                             self.q, self.path_score, temperature=self.tau, seed_dev=self.seed)

    def run_verify(self):
        if self.verify == "greedy":
            dflash2_verify_greedy(self.target, self.path_tok, self.accept_len, self.out_tok,
                                  self.ws_verify)
        elif self.verify == "reject":
            dflash2_verify_reject(self.target, self.path_tok, self.path_rank, self.cand_idx, self.q,
                                  self.tau, self.seed, self.accept_len, self.out_tok, self.ws_verify)
        elif self.verify == "mixed":
            g = self.greedy_rows
            if g > 0:
                dflash2_verify_greedy(self.target[:g], self.path_tok[:g], self.accept_len[:g],
                                      self.out_tok[:g], self.ws_verify)
            if g < self.B:
                dflash2_verify_reject(self.target[g:], self.path_tok[g:], self.path_rank[g:],
                                      self.cand_idx[g:], self.q[g:], self.tau, self.seed,
                                      self.accept_len[g:], self.out_tok[g:], self.ws_verify, b0=g)
        else:
            raise ValueError(self.verify)

    def run_fused(self):
        dflash2_cycle_fused(self.logits, self.target, self.emb, self.h, self.w_a, self.w_b, self.w_h,
                            self.last_tok, self.path_mode, self.cand_idx, self.cand_val, self.scores,
                            self.path_rank, self.path_tok, self.q, self.path_score, self.accept_len,
                            self.out_tok, self.status, self.ws_fused, gate=self.gate)

    def run(self, conv: bool = True):
        if conv:
            self.run_conv()
        if self.fused:
            self.run_fused()
            return
        self.run_topk()
        self.run_pair_scores()
        self.run_path()
        self.run_verify()

    # -- graph ---------------------------------------------------------------
    def capture(self, conv: bool = True):
        """Record one whole cycle as a HIP graph (after one eager warm-up)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run(conv)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run(conv)
        torch.cuda.synchronize()
        return self.graph

    def replay(self):
        self.graph.replay()

    def set_seed(self, seed: int):
        self.seed.fill_(int(seed))

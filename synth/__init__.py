"""Seeded synthetic inputs for the DFlash 2 draft-block cycle.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark.  It draws random tensors and nothing else: it holds none of the
method's arithmetic (no top-k, no pair scores, no path search, no
verification, no convolution).  Everything is drawn with a seeded
``torch.Generator`` on the requested device, so a workload is reproducible
from its name and seed alone.

Shapes and value distributions follow the workloads the pages run on:

* block 8 (7 drafts) and block 16 (15 drafts); concurrency 1 / 8 / 32
  ("DFlash2 并行投机解码解读" §二 and §六; "DFlash 2: Keep Drafting Parallel"
  §"A lightweight local convolution" puts blocks at 4-16 tokens);
* a true token that sits in the drafter's top-16 at a rate falling from
  99.5 % to 87.8 % over the block, and at top-1 at a rate falling from
  85.4 % to 72.9 % ("DFlash 2: Keep Drafting Parallel", Table 1, Recall@16
  and Recall@1 rows);
* vocabulary 151,936 or 262,144, hidden size 5120, selector rank 256
  (the rank is stated in §"A lightweight path selector").

None of the pages' evaluation sets is used or reproduced; these tensors
stand in for the drafter and target logits those runs produced.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

# Table 1 of "DFlash 2: Keep Drafting Parallel" (Recall@1 / Recall@16 at the
# first and the last of seven draft positions).  The generator interpolates
# linearly between the endpoints for any block length.
RECALL16_FIRST, RECALL16_LAST = 0.995, 0.878
RECALL1_FIRST, RECALL1_LAST = 0.854, 0.729
PLANT_BOOST = 4.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # concurrent requests (batch rows)
    block: int             # block size; T = block - 1 draft positions
    K: int                 # candidates kept per position
    V: int                 # vocabulary
    d: int                 # hidden size
    r: int                 # selector rank
    logits_dtype: str      # "fp32" | "bf16"
    drafter: str           # "tiny_planted" | "normal3" | "gumbel3"
    target: str            # "tiny_agree" | "planted_argmax" | "correlated" | "mixed"
    path_mode: str         # "viterbi" | "greedy" | "sample" | "both"
    verify: str            # "greedy" | "reject" | "mixed"
    tau: float             # temperature for sampled paths / rejection verify
    seed: int
    conv_sites: int = 0    # independent two-tap conv applications per cycle
    conv_base: bool = False

    @property
    def T(self) -> int:
        return self.block - 1

    @property
    def G(self) -> int:
        return self.d // 16


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_b1_blk4_v1000", B=1, block=4, K=4, V=1000, d=64, r=16,
                 logits_dtype="fp32", drafter="tiny_planted", target="tiny_agree",
                 path_mode="both", verify="greedy", tau=0.0, seed=0),
        Workload("b1_blk8_v151936", B=1, block=8, K=16, V=151936, d=5120, r=256,
                 logits_dtype="bf16", drafter="normal3", target="planted_argmax",
                 path_mode="viterbi", verify="greedy", tau=0.0, seed=1),
        Workload("b8_blk8_v151936_sampled", B=8, block=8, K=16, V=151936, d=5120, r=256,
                 logits_dtype="bf16", drafter="normal3", target="correlated",
                 path_mode="sample", verify="reject", tau=1.0, seed=2),
        Workload("b32_blk16_v151936_conv", B=32, block=16, K=16, V=151936, d=5120, r=256,
                 logits_dtype="bf16", drafter="normal3", target="planted_argmax",
                 path_mode="viterbi", verify="greedy", tau=0.0, seed=3, conv_sites=20),
        Workload("b64_blk16_v262144_stress", B=64, block=16, K=16, V=262144, d=5120, r=256,
                 logits_dtype="bf16", drafter="gumbel3", target="mixed",
                 path_mode="viterbi", verify="mixed", tau=1.0, seed=4, conv_sites=20),
        # the remaining points of the batch x block sweep
        Workload("b32_blk8_v151936", B=32, block=8, K=16, V=151936, d=5120, r=256,
                 logits_dtype="bf16", drafter="normal3", target="planted_argmax",
                 path_mode="viterbi", verify="greedy", tau=0.0, seed=11),
        Workload("b1_blk16_v151936", B=1, block=16, K=16, V=151936, d=5120, r=256,
                 logits_dtype="bf16", drafter="normal3", target="planted_argmax",
                 path_mode="viterbi", verify="greedy", tau=0.0, seed=12),
        Workload("b8_blk16_v151936", B=8, block=16, K=16, V=151936, d=5120, r=256,
                 logits_dtype="bf16", drafter="normal3", target="planted_argmax",
                 path_mode="viterbi", verify="greedy", tau=0.0, seed=13),
    ]
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(w, **changes)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device) -> torch.Tensor:
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def _uniform(shape, g, device) -> torch.Tensor:
    return torch.rand(*shape, generator=g, device=device, dtype=torch.float32)


def _randint(high: int, shape, g, device) -> torch.Tensor:
    return torch.randint(0, high, shape, generator=g, device=device, dtype=torch.int64)


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """fp32 -> storage dtype; bf16 uses PyTorch's round-to-nearest-even."""
    if dtype == "fp32":
        return x.float().contiguous()
    if dtype == "bf16":
        return x.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def recall_rates(T: int):
    """Per-position (top-1 rate, top-16 rate), linear between Table 1's ends."""
    out = []
    for t in range(T):
        f = 0.0 if T == 1 else t / (T - 1)
        r1 = RECALL1_FIRST + (RECALL1_LAST - RECALL1_FIRST) * f
        r16 = RECALL16_FIRST + (RECALL16_LAST - RECALL16_FIRST) * f
        out.append((r1, r16))
    return out


def drafter_logits(w: Workload, device="cpu", B: Optional[int] = None, seed_offset: int = 0):
    """Drafter block logits [B, T, V] in the workload's dtype, plus the
    planted "true" token per position and the rank it was planted at.

    tiny_planted: N(0,1) with +4 on one uniform token per position.
    normal3 / gumbel3: 3*N(0,1) or 3*Gumbel(0,1); per position a rank rho is
    drawn (0 with the top-1 rate, 1..15 with the top-16 rate minus that,
    otherwise outside the top 16) and the token at that rank is the true
    token; a rank-0 true token gets +4 on its logit.
    """
    B = w.B if B is None else B
    T, V = w.T, w.V
    g = _gen(w.seed * 1000 + 1 + seed_offset, device)
    if w.drafter == "tiny_planted":
        z = _randn((B, T, V), g, device)
        tok = _randint(V, (B, T), g, device)
        z.scatter_add_(2, tok[..., None], torch.full((B, T, 1), PLANT_BOOST, device=device))
        rank = torch.zeros((B, T), dtype=torch.int64, device=device)
        return to_storage(z, w.logits_dtype), tok, rank
    if w.drafter == "normal3":
        z = 3.0 * _randn((B, T, V), g, device)
    elif w.drafter == "gumbel3":
        u = _uniform((B, T, V), g, device).clamp_(min=1e-12, max=1.0 - 1e-7)
        z = 3.0 * (-torch.log(-torch.log(u)))
    else:
        raise ValueError(w.drafter)
    top = torch.topk(z, 16, dim=-1).indices            # [B,T,16]
    rates = torch.tensor(recall_rates(T), device=device, dtype=torch.float32)  # [T,2]
    u = _uniform((B, T), g, device)
    in1 = u < rates[:, 0]
    in16 = u < rates[:, 1]
    rank_in = 1 + _randint(15, (B, T), g, device)
    rank = torch.where(in1, torch.zeros_like(rank_in), rank_in)
    tok = torch.gather(top, 2, rank[..., None]).squeeze(-1)
    # outside the top 16: uniform among the other tokens (rejection draws)
    out_tok = _randint(V, (B, T), g, device)
    for _ in range(8):
        clash = (out_tok[..., None] == top).any(-1)
        if not bool(clash.any()):
            break
        out_tok = torch.where(clash, _randint(V, (B, T), g, device), out_tok)
    tok = torch.where(in16, tok, out_tok)
    rank = torch.where(in16, rank, torch.full_like(rank, 16))
    boost = torch.where(rank == 0, PLANT_BOOST, 0.0).to(torch.float32)
    z.scatter_add_(2, tok[..., None], boost[..., None])
    return to_storage(z, w.logits_dtype), tok, rank


def target_logits(w: Workload, drafter: torch.Tensor, true_tok: torch.Tensor, device="cpu",
                  kind: Optional[str] = None, seed_offset: int = 0) -> torch.Tensor:
    """Target verify logits [B, T+1, V]; row T supplies the bonus token.

    tiny_agree: N(0,1); for t < T the argmax is moved (max + 4) to the
      drafter's top-1 token with probability 0.85, else to a uniform other
      token; row T gets a uniform argmax.
    planted_argmax: 3*N(0,1) with the true token of position t at max + 4;
      row T gets a uniform argmax.
    correlated: rows t < T are the drafter's logits plus N(0,1) noise;
      row T is 3*N(0,1).
    mixed: requests 0 .. B/2 - 1 planted_argmax (the greedy-verified half),
      the rest correlated with the next seed offset (the rejection half).
    """
    kind = kind or w.target
    B, T, V = drafter.shape[0], w.T, w.V
    if kind == "mixed":
        h = B // 2
        return torch.cat([target_logits(w, drafter[:h], true_tok[:h], device, "planted_argmax", seed_offset),
                          target_logits(w, drafter[h:], true_tok[h:], device, "correlated", seed_offset + 1)],
                         0)
    g = _gen(w.seed * 1000 + 2 + seed_offset, device)
    if kind == "tiny_agree":
        z = _randn((B, T + 1, V), g, device)
        top1 = drafter.float().argmax(-1)
        agree = _uniform((B, T), g, device) < 0.85
        other = (top1 + 1 + _randint(V - 1, (B, T), g, device)) % V
        y = torch.cat([torch.where(agree, top1, other), _randint(V, (B, 1), g, device)], 1)
        zmax = z.amax(-1, keepdim=True)
        z.scatter_(2, y[..., None], zmax + PLANT_BOOST)
        return to_storage(z, w.logits_dtype)
    if kind == "planted_argmax":
        z = 3.0 * _randn((B, T + 1, V), g, device)
        y = torch.cat([true_tok, _randint(V, (B, 1), g, device)], 1)
        zmax = z.amax(-1, keepdim=True)
        z.scatter_(2, y[..., None], zmax + PLANT_BOOST)
        return to_storage(z, w.logits_dtype)
    if kind == "correlated":
        rows = drafter.float() + _randn((B, T, V), g, device)
        last = 3.0 * _randn((B, 1, V), g, device)
        return to_storage(torch.cat([rows, last], 1), w.logits_dtype)
    raise ValueError(kind)


def embeddings(w: Workload, device="cpu") -> torch.Tensor:
    """Token embedding table E [V, d] bf16, N(0, 0.02^2)."""
    g = _gen(w.seed * 1000 + 3, device)
    out = torch.empty((w.V, w.d), dtype=torch.bfloat16, device=device)
    step = max(1, (1 << 26) // w.d)
    for v0 in range(0, w.V, step):
        v1 = min(w.V, v0 + step)
        out[v0:v1] = (0.02 * _randn((v1 - v0, w.d), g, device)).to(torch.bfloat16)
    return out


def selector_weights(w: Workload, device="cpu"):
    """W_A, W_B ~ N(0, 1/(0.0004 d)) so that A(tok), B(tok) have unit
    variance; W_H ~ N(0, 1/(d r)) so that the bigram term has unit variance."""
    g = _gen(w.seed * 1000 + 4, device)
    sa = 1.0 / (0.02 * math.sqrt(w.d))
    sh = 1.0 / math.sqrt(w.d * w.r)
    wa = (sa * _randn((w.r, w.d), g, device)).to(torch.bfloat16)
    wb = (sa * _randn((w.r, w.d), g, device)).to(torch.bfloat16)
    wh = (sh * _randn((w.r, w.d), g, device)).to(torch.bfloat16)
    return wa, wb, wh


def context_hidden(w: Workload, device="cpu", B: Optional[int] = None) -> torch.Tensor:
    """Drafter hidden state h_t per draft position, [B, T, d] bf16 N(0,1)."""
    B = w.B if B is None else B
    g = _gen(w.seed * 1000 + 5, device)
    return _randn((B, w.T, w.d), g, device).to(torch.bfloat16)


def last_tokens(w: Workload, device="cpu", B: Optional[int] = None) -> torch.Tensor:
    """Last verified token per request, [B] int32 uniform over the vocab."""
    B = w.B if B is None else B
    g = _gen(w.seed * 1000 + 6, device)
    return _randint(w.V, (B,), g, device).to(torch.int32)


def conv_site(w: Workload, site: int, device="cpu", B: Optional[int] = None, base: Optional[bool] = None):
    """One two-tap conv application: x [B, L, d], x_prev [B, d] (N(0,1) bf16),
    tap weights W [2G, d] bf16 N(0, 0.02^2) (rows 0..G-1 drive the current
    tap, rows G..2G-1 the previous tap), and an optional learned base kernel
    [2, d] fp32 (1 + N(0, 0.02^2) for the current tap, N(0, 0.02^2) for the
    previous tap)."""
    B = w.B if B is None else B
    base = w.conv_base if base is None else base
    L, d = w.block, w.d
    g = _gen(w.seed * 1000 + 100 + site, device)
    x = _randn((B, L, d), g, device).to(torch.bfloat16)
    xp = _randn((B, d), g, device).to(torch.bfloat16)
    wt = (0.02 * _randn((2 * (d // 16), d), g, device)).to(torch.bfloat16)
    bs = None
    if base:
        bs = 0.02 * _randn((2, d), g, device)
        bs[0] += 1.0
    return x, xp, wt, bs


def pair_score_lattice(B: int, T: int, K: int, seed: int, device="cpu", spread: float = 3.0,
                       ties: bool = False) -> torch.Tensor:
    """A stand-alone score lattice S [B, T, K, K] fp32 for exercising the
    path search on its own: unigram-like columns plus N(0,1) pair terms; at
    t = 0 only predecessor row 0 is populated and rows 1..K-1 are -inf.
    With ties=True values are rounded to multiples of 0.25 so that equal
    scores occur often."""
    g = _gen(seed, device)
    u = spread * _randn((B, T, 1, K), g, device)
    s = u + _randn((B, T, K, K), g, device)
    if ties:
        s = torch.round(s * 4.0) / 4.0
    s[:, 0, 1:, :] = float("-inf")
    return s.contiguous()


def philox_seed(base: int, cycle: int = 0) -> int:
    return int(base) + int(cycle)

"""GPU parity of the persistent small-batch cycle (dflash2_cycle_fused).

The fused launch runs the stage kernels' own arithmetic (the same K split
and summation orders), so every output -- candidates, pair scores, path,
proposal, path score, accepted length, emitted tokens -- must equal the
multi-launch cycle's bit for bit on the same inputs; the fused cycle is also
checked against the oracle's own cycle with the rules of test_gpu_cycle.py.
Shapes: batch 1 / block 8 and block 16 at the full vocabulary and hidden
size, batch 8, a ragged vocabulary, rank 64 with K = 7, the sigmoid gate,
GREEDY paths, and graph replays (the control words are reset by each launch
for the next)."""
import numpy as np
import pytest
import torch

import synth
from draft_selection_bf16_amd.cycle import Cycle
from gpu_util import DEV, report
from test_gpu_cycle import build, check_cycle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

OUTS = ("cand_idx", "cand_val", "scores", "path_rank", "path_tok", "q", "path_score", "accept_len", "out_tok")


def fused_twin(cyc, gate=None):
    """A fused Cycle over the same input tensors as `cyc`."""
    pm = {0: "viterbi", 1: "greedy"}[cyc.path_mode]
    return Cycle(logits=cyc.logits, target=cyc.target, emb=cyc.emb, h=cyc.h, w_a=cyc.w_a, w_b=cyc.w_b,
                 w_h=cyc.w_h, last_tok=cyc.last_tok, K=cyc.K, path_mode=pm, verify="greedy",
                 gate=cyc.gate if gate is None else gate, fused=True)


def assert_same(a, b, label):
    torch.cuda.synchronize()
    assert int(b.status.item()) == 0, (label, "status", int(b.status.item()))
    for k in OUTS:
        x, y = getattr(a, k), getattr(b, k)
        assert torch.equal(x, y), (label, k, int((x != y).sum().item()))


def run_case(w, rows, label, gate=None):
    print(f"[case] fused {label}", flush=True)
    cyc, _ = build(w, with_conv=0)
    if gate is not None:
        cyc.gate = gate
    cyc.run()
    fz = fused_twin(cyc)
    fz.run()
    assert_same(cyc, fz, label)
    check_cycle(fz, w, rows, "fused " + label)
    return cyc, fz


def test_fused_b1_blk8_full_size():
    run_case(synth.WORKLOADS["b1_blk8_v151936"], [0], "b1_blk8_v151936")


def test_fused_b1_blk16_full_size():
    run_case(synth.WORKLOADS["b1_blk16_v151936"], [0], "b1_blk16_v151936")


def test_fused_b8_blk16_full_size():
    run_case(synth.WORKLOADS["b8_blk16_v151936"], [0, 3, 7], "b8_blk16_v151936")


@pytest.mark.parametrize("kw,label", [
    (dict(V=50021, d=1024), "ragged vocabulary"),
    (dict(V=20000, d=384, r=64, K=7), "rank 64, K 7"),
    (dict(V=3000, d=256, path_mode="greedy"), "greedy path"),
    (dict(B=4, block=2, V=4096, d=512), "T 1"),
    (dict(B=3, block=33, V=8192, d=256), "T 32"),
])
def test_fused_shapes(kw, label):
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], **kw)
    run_case(w, list(range(min(w.B, 3))), label)


def test_fused_sigmoid_gate():
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], B=2, V=10000, d=512)
    cyc, _ = build(w, with_conv=0)
    cyc.gate = 1
    cyc.run()
    fz = fused_twin(cyc, gate=1)
    fz.run()
    assert_same(cyc, fz, "sigmoid gate")
    check_cycle(fz, w, [0, 1], "fused sigmoid gate")


def test_fused_graph_replays_and_repeated_launches():
    """Captured and replayed 50 times, eager launches 200 times in a row:
    every launch leaves the control words zero for the next, and every
    result equals the multi-launch cycle's."""
    w = synth.WORKLOADS["b1_blk8_v151936"]
    cyc, _ = build(w, with_conv=0)
    cyc.run()
    fz = fused_twin(cyc)
    for _ in range(200):
        fz.run()
    assert_same(cyc, fz, "eager x200")
    fz.capture(conv=False)
    for rep in range(50):
        for k in OUTS:
            getattr(fz, k).fill_(-7)
        fz.replay()
        if rep % 10 == 0:
            assert_same(cyc, fz, f"replay {rep}")
            _ = torch.randn(1000, device=DEV).sum().item()    # eager work between replays
    assert_same(cyc, fz, "replay 49")
    report("fused graph", replays=50, eager_launches=200)

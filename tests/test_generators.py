"""The synthetic generators against the numbers the pages print: the Table 1
recall endpoints, realised top-1 / top-16 rates of the planted tokens, and
the parameter counts that fix the shapes of the selector and the conv."""
import json
import os

import numpy as np
import pytest
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_recall_endpoints_match_table1():
    t1 = _load("table1_recall.json")
    assert synth.RECALL1_FIRST == t1["recall_at_1"][0]
    assert synth.RECALL1_LAST == t1["recall_at_1"][-1]
    assert synth.RECALL16_FIRST == t1["recall_at_16"][0]
    assert synth.RECALL16_LAST == t1["recall_at_16"][-1]
    rates = synth.recall_rates(7)
    assert rates[0] == pytest.approx((0.854, 0.995))
    assert rates[-1] == pytest.approx((0.729, 0.878))


@pytest.mark.parametrize("drafter", ["normal3", "gumbel3"])
def test_realised_recall_rates(orc, drafter):
    w = synth.scaled(synth.WORKLOADS["b8_blk8_v151936_sampled"], B=600, V=4096,
                     drafter=drafter)
    z, tok, rank = synth.drafter_logits(w)
    idx, _ = orc.topk(z, 16)
    tok = tok.numpy()
    in1 = idx[..., 0] == tok
    in16 = (idx == tok[..., None]).any(-1)
    for t, (r1, r16) in enumerate(synth.recall_rates(w.T)):
        n = in1.shape[0]
        assert abs(in1[:, t].mean() - r1) < 5 * np.sqrt(r1 * (1 - r1) / n) + 0.01, t
        assert abs(in16[:, t].mean() - r16) < 5 * np.sqrt(r16 * (1 - r16) / n) + 0.01, t


def test_selector_parameter_count_pins_the_projection_reading():
    p = _load("param_counts.json")["selector"]
    d, r = p["hidden_size_assumed"], p["rank"]
    tol = p["printed_precision_millions"] / 2
    # A, B and H as d -> r linear maps: three r x d matrices
    assert abs(3 * r * d / 1e6 - p["params_millions"]) <= tol
    # per-token lookup tables for A and B would be far larger
    assert 2 * 151936 * r / 1e6 > 10 * p["params_millions"]


def test_conv_parameter_count_pins_the_grouped_reading():
    p = _load("param_counts.json")["conv"]
    d, grp = p["hidden_size_assumed"], p["group"]
    sites = p["layers"] * p["sites_per_layer"]
    tol = p["printed_precision_millions"] / 2
    per_site = d * 2 * (d // grp) + 2 * d            # d -> 2G correction map + 2 x d base
    assert abs(sites * per_site / 1e6 - p["params_millions"]) <= tol
    # without the base kernel the count prints as 16.4M, not 16.5M
    assert abs(sites * d * 2 * (d // grp) / 1e6 - p["params_millions"]) > tol
    # one correction per channel instead of per 16 channels is ruled out
    assert sites * d * 2 * d / 1e6 > 10 * p["params_millions"]


def test_generators_are_seeded():
    w = synth.scaled(synth.WORKLOADS["b1_blk8_v151936"], V=2048, d=64)
    a = synth.drafter_logits(w)[0]
    b = synth.drafter_logits(w)[0]
    assert torch.equal(a, b)
    assert a.dtype == torch.bfloat16 and a.shape == (1, 7, 2048)
    Z = synth.target_logits(w, a, synth.drafter_logits(w)[1])
    assert Z.shape == (1, 8, 2048)


def test_tiny_workload_matches_its_recipe():
    w = synth.WORKLOADS["tiny_b1_blk4_v1000"]
    z, tok, _ = synth.drafter_logits(w)
    assert z.dtype == torch.float32 and z.shape == (1, 3, 1000)
    E = synth.embeddings(w)
    assert E.shape == (1000, 64) and E.dtype == torch.bfloat16
    assert abs(E.float().std().item() - 0.02) < 0.002
    wa, wb, wh = synth.selector_weights(w)
    assert wa.shape == (16, 64)

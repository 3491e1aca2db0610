"""Accounting helpers pinned to the numbers the pages print."""
import json
import os

import numpy as np
import pytest

from mixture_experts_layer_gate_amd import roofline as rf
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_pins.json")


def _gold():
    with open(GOLD) as fh:
        return json.load(fh)


def test_util_worked_example():
    g = _gold()["util_example"]
    F, B = g["F_flops"], g["B_bytes_per_s"]
    assert rf.min_full_util_batch(B, F) == pytest.approx(g["min_batch"])
    assert g["min_batch"] * g["topk"] / g["experts"] == g["tokens_per_expert"]
    assert rf.util(g["topk"], g["experts"], B, F, g["min_batch"]) == pytest.approx(g["util_at_min_batch"])
    # saturates at 1 for a large batch
    assert rf.util(g["topk"], g["experts"], B, F, 10 * g["min_batch"]) == 1.0


@pytest.mark.parametrize("row", _gold()["table_iv"]["rows"], ids=lambda r: r["model"])
def test_table_iv_expert_bytes(row):
    b = rf.expert_weight_bytes(row["E"], row["d"], row["f"], 2)
    assert abs(b / 2**30 - row["gib"]) <= 0.0051
    # Table IV's own formula, 48*E*d*f/G with G = 8, is the same number of bytes
    assert b == 48 * row["E"] * row["d"] * row["f"] // 8


def test_mean_rows_per_expert(rng):
    # b_e * m = B * K / E: the mean of the per-expert counts is T*k/E exactly
    T, E, k = 96, 12, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, _, _ = oracle.dispatch(idx, E)
    assert counts.sum() == T * k and offsets[-1] == T * k
    assert counts.mean() == T * k / E


def test_kappa_uniform_is_one():
    assert rf.kappa([5, 5, 5, 5]) == 1.0
    assert rf.kappa([8, 0, 0, 0]) == 4.0

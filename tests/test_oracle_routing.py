"""Pins of the oracle's top-k selection, weights, dispatch and block plan."""
import collections
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "routing_cases.json")


def _gold():
    with open(GOLD) as fh:
        return json.load(fh)


def _brute_topk(row, k):
    """rank_e = #{e' : l_e' > l_e or (l_e' == l_e and e' < e)}; slot = rank, kept iff rank < k."""
    E = len(row)
    ranks = [sum(1 for q in range(E) if row[q] > row[e] or (row[q] == row[e] and q < e)) for e in range(E)]
    out = [None] * k
    for e, r in enumerate(ranks):
        if r < k:
            out[r] = e
    return out


def _tied_logits(rng, T, E):
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 1.0, 2.0], np.float32)
    return rng.choice(vals, size=(T, E)).astype(np.float32)


@pytest.mark.parametrize("E,k", [(1, 1), (4, 1), (8, 2), (8, 8), (16, 4), (33, 7)])
def test_topk_matches_brute_force_with_ties(rng, E, k):
    for logits in (_tied_logits(rng, 25, E), rng.standard_normal((25, E)).astype(np.float32)):
        idx = oracle.topk_select(logits, k)
        assert idx.dtype == np.int32 and idx.shape == (25, k)
        for t in range(25):
            assert idx[t].tolist() == _brute_topk(logits[t].tolist(), k)


def test_topk_golden_ties():
    c = _gold()["tie_case"]
    idx = oracle.topk_select(np.array(c["logits"], np.float32), c["k"])
    assert idx.tolist() == c["expected_idx"]


def test_k_equals_E_is_a_full_sort(rng):
    logits = rng.standard_normal((10, 9)).astype(np.float32)
    idx = oracle.topk_select(logits, 9)
    for t in range(10):
        assert idx[t].tolist() == sorted(range(9), key=lambda e: (-float(logits[t, e]), e))


def test_weights_golden():
    c = _gold()["softmax_case"]
    l = np.array(c["logits"], np.float32)
    idx = oracle.topk_select(l, c["k"])
    assert idx.tolist() == c["expected_idx"]
    np.testing.assert_allclose(oracle.topk_weights(l, idx), c["expected_w"], rtol=1e-7)


def test_weights_k1_is_exactly_one(rng):
    l = rng.standard_normal((20, 6)).astype(np.float32) * 30
    idx = oracle.topk_select(l, 1)
    assert np.all(oracle.topk_weights(l, idx) == 1.0)


def test_weights_k_equals_E_is_textbook_softmax(rng):
    l = rng.standard_normal((20, 6)).astype(np.float32) * 3
    idx = oracle.topk_select(l, 6)
    w = oracle.topk_weights(l, idx)
    ref = np.take_along_axis(softmax(l.astype(np.float64), axis=1), idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, ref, rtol=2e-7, atol=0)


def test_weights_sum_to_one_and_descend(rng):
    l = rng.standard_normal((50, 16)).astype(np.float32) * 5
    idx = oracle.topk_select(l, 4)
    w = oracle.topk_weights(l, idx)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_forced_routing_by_bias(rng):
    T, d, E, k = 40, 64, 8, 3
    x = ((rng.standard_normal((T, d)).astype(np.float32).view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    wg = (((rng.standard_normal((E, d)) / 8).astype(np.float32).view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    bias = np.zeros(E, np.float32)
    bias[:k] = 1e4
    _, idx, _ = oracle.route(x, wg, bias, k, "bf16")
    counts, _, _, _ = oracle.dispatch(idx, E)
    assert counts.tolist() == [T] * k + [0] * (E - k)


def test_dispatch_golden():
    c = _gold()["dispatch_case"]
    counts, offsets, perm, inv = oracle.dispatch(np.array(c["topk_idx"], np.int32), c["E"])
    assert counts.tolist() == c["counts"]
    assert offsets.tolist() == c["offsets"]
    assert perm.tolist() == c["perm"]
    assert inv.tolist() == c["inv_perm"]


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 3, 2), (64, 8, 2), (100, 16, 4), (50, 256, 8)])
def test_dispatch_brute_force_and_invariants(rng, T, E, k):
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.dispatch(idx, E)
    # brute force: positions from sorting (expert, token, slot)
    order = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    assert perm.tolist() == [t * k + j for (_, t, j) in order]
    cnt = collections.Counter(int(e) for e in idx.reshape(-1))
    assert counts.tolist() == [cnt.get(e, 0) for e in range(E)]
    # invariants
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert sorted(perm.tolist()) == list(range(T * k))
    assert np.all(inv[perm] == np.arange(T * k)) and np.all(perm[inv] == np.arange(T * k))
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(idx.reshape(-1)[seg] == e)
        assert np.all(np.diff(seg) > 0)


def test_block_plan_golden():
    c = _gold()["plan_case"]
    assert [list(b) for b in oracle.block_plan(np.array(c["counts"]), c["beta"])] == c["blocks"]


@pytest.mark.parametrize("beta", [1, 7, 32, 128])
def test_block_plan_invariants(rng, beta):
    counts = rng.integers(0, 300, size=20)
    counts[3] = 0
    blocks = oracle.block_plan(counts, beta)
    covered = np.zeros(int(counts.sum()), np.int32)
    start = np.concatenate([[0], np.cumsum(counts)])
    partial = collections.Counter()
    for e, r0, n in blocks:
        assert 1 <= n <= beta and start[e] <= r0 and r0 + n <= start[e + 1]
        covered[r0:r0 + n] += 1
        partial[e] += n < beta
    assert np.all(covered == 1)
    assert all(v <= 1 for v in partial.values())
    assert len(blocks) == sum(math.ceil(c / beta) for c in counts)

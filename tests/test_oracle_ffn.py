"""Pins of the oracle's expert FFN and combine."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import moe_inputs
from conftest import to_numpy

GOLD = os.path.join(os.path.dirname(__file__), "golden", "routing_cases.json")


def _small(T, d, f, E, k, dtype="f32", seed=0, s=0.0):
    inp = moe_inputs.random_inputs(T, d, f, E, k, dtype, s, seed)
    return {n: to_numpy(v, dtype) for n, v in inp.items()}


def _direct_python(x, idx, w, w1, w3, w2):
    """out[t] straight from the definition, scalar Python loops (tiny shapes only)."""
    T, d = x.shape
    k = idx.shape[1]
    f = w1.shape[1]
    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            h = []
            for n in range(f):
                g = sum(float(x[t, i]) * float(w1[e, n, i]) for i in range(d))
                u = sum(float(x[t, i]) * float(w3[e, n, i]) for i in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for o in range(d):
                out[t][o] += float(w[t, j]) * sum(h[n] * float(w2[e, o, n]) for n in range(f))
    return np.array(out)


def test_swiglu_golden():
    c = json.load(open(GOLD))["swiglu_case"]
    x = np.array([[c["x"]]], np.float32)
    wg = np.array([[1.0]], np.float32)
    w1 = np.array([[[c["w1"]]]], np.float32)
    w3 = np.array([[[c["w3"]]]], np.float32)
    w2 = np.array([[[c["w2"]]]], np.float32)
    r = oracle.layer_forward(x, wg, None, w1, w3, w2, 1, "f32")
    assert r["out"][0, 0] == pytest.approx(c["expected_out"], rel=1e-14)


@pytest.mark.parametrize("T,d,f,E,k", [(5, 6, 7, 4, 2), (3, 4, 5, 3, 3), (4, 8, 3, 5, 1)])
def test_layer_matches_direct_python(T, d, f, E, k):
    a = _small(T, d, f, E, k)
    r = oracle.layer_forward(a["x"], a["wg"], a["bias"], a["w1"], a["w3"], a["w2"], k, "f32")
    ref = _direct_python(a["x"], r["topk_idx"], r["topk_w"], a["w1"], a["w3"], a["w2"])
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_identical_experts_reduce_to_dense_ffn():
    T, d, f, E, k = 12, 16, 24, 6, 3
    a = _small(T, d, f, E, k, seed=3)
    for n in ("w1", "w3", "w2"):
        a[n] = np.repeat(a[n][:1], E, axis=0)
    r = oracle.layer_forward(a["x"], a["wg"], a["bias"], a["w1"], a["w3"], a["w2"], k, "f32")
    xt = torch.from_numpy(a["x"]).double()
    dense = (torch.nn.functional.silu(xt @ torch.from_numpy(a["w1"][0]).double().T)
             * (xt @ torch.from_numpy(a["w3"][0]).double().T)) @ torch.from_numpy(a["w2"][0]).double().T
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-6, atol=1e-9)  # weights stored fp32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_expert_is_dense_swiglu(dtype):
    T, d, f = 9, 32, 48
    a = _small(T, d, f, 1, 1, dtype=dtype, seed=5)
    r = oracle.layer_forward(a["x"], a["wg"], a["bias"], a["w1"], a["w3"], a["w2"], 1, dtype)
    assert np.all(r["topk_w"] == 1.0)
    dec = lambda v: torch.from_numpy(oracle.decode(v, dtype)).double()  # noqa: E731
    xt = dec(a["x"])
    dense = (torch.nn.functional.silu(xt @ dec(a["w1"][0]).T) * (xt @ dec(a["w3"][0]).T)) @ dec(a["w2"][0]).T
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-12, atol=1e-12)


def test_swapping_gate_and_up_changes_the_result():
    """W1 is the gated projection: exchanging W1 and W3 must change the output."""
    a = _small(6, 8, 10, 4, 2, seed=9)
    r1 = oracle.layer_forward(a["x"], a["wg"], None, a["w1"], a["w3"], a["w2"], 2, "f32")
    r2 = oracle.layer_forward(a["x"], a["wg"], None, a["w3"], a["w1"], a["w2"], 2, "f32")
    assert np.max(np.abs(r1["out"] - r2["out"])) > 1e-3


def test_token_outputs_equal_full_layer():
    T, d, f, E, k = 30, 24, 40, 8, 2
    a = _small(T, d, f, E, k, dtype="bf16", seed=2, s=1.0)
    r = oracle.layer_forward(a["x"], a["wg"], a["bias"], a["w1"], a["w3"], a["w2"], k, "bf16")
    toks = [0, 3, 17, 29]
    o = oracle.token_outputs(a["x"], r["topk_idx"], r["topk_w"], a["w1"], a["w3"], a["w2"], toks, "bf16")
    np.testing.assert_allclose(o, r["out"][toks], rtol=1e-12, atol=1e-12)


def test_combine_weights_each_slot():
    """Combine: out[t] = sum_j w[t,j] * y[inv_perm[t*k+j]] -- checked on a y whose rows are one-hot."""
    T, k = 3, 2
    inv = np.array([2, 0, 1, 4, 3, 5], np.int32)
    w = np.array([[0.75, 0.25], [0.5, 0.5], [0.9, 0.1]], np.float32)
    y = np.eye(6)
    out = oracle.combine(y, inv, w, k)
    for t in range(T):
        for j in range(k):
            assert out[t, inv[t * k + j]] == pytest.approx(float(w[t, j]))
    assert out.sum() == pytest.approx(float(w.sum()))

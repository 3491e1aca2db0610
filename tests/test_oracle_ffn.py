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


def _small_shared(T, d, f, E, k, S, dtype="f32", seed=0, s=0.0):
    inp = moe_inputs.random_inputs(T, d, f, E, k, dtype, s, seed, n_shared=S)
    return {n: to_numpy(v, dtype) for n, v in inp.items()}


def _direct_dense_python(x, w1, w3, w2):
    """One SwiGLU expert applied to every token, scalar Python loops (tiny shapes only)."""
    T, d = x.shape
    f = w1.shape[0]
    out = np.zeros((T, d))
    for t in range(T):
        h = []
        for n in range(f):
            g = sum(float(x[t, i]) * float(w1[n, i]) for i in range(d))
            u = sum(float(x[t, i]) * float(w3[n, i]) for i in range(d))
            h.append(g / (1.0 + math.exp(-g)) * u)
        for o in range(d):
            out[t, o] = sum(h[n] * float(w2[o, n]) for n in range(f))
    return out


@pytest.mark.parametrize("T,d,f,E,k,S", [(5, 6, 7, 4, 2, 1), (3, 4, 5, 3, 1, 2)])
def test_shared_layer_matches_direct_python(T, d, f, E, k, S):
    """Shared experts: every token's output gains each shared expert's SwiGLU output, weight 1."""
    a = _small_shared(T, d, f, E, k, S, seed=4)
    r = oracle.layer_forward_shared(a["x"], a["wg"], a["bias"], a["w1"], a["w3"], a["w2"],
                                    a["sw1"], a["sw3"], a["sw2"], k, "f32")
    ref = _direct_python(a["x"], r["topk_idx"], r["topk_w"], a["w1"], a["w3"], a["w2"])
    for s in range(S):
        ref = ref + _direct_dense_python(a["x"], a["sw1"][s], a["sw3"][s], a["sw2"][s])
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def test_shared_layer_with_zero_routed_output_is_dense_swiglu():
    """Zero down projections for the routed experts leave the shared expert alone."""
    T, d, f, E, k = 10, 32, 40, 8, 2
    a = _small_shared(T, d, f, E, k, 1, dtype="bf16", seed=6)
    a["w2"] = np.zeros_like(a["w2"])
    r = oracle.layer_forward_shared(a["x"], a["wg"], a["bias"], a["w1"], a["w3"], a["w2"],
                                    a["sw1"], a["sw3"], a["sw2"], k, "bf16")
    dec = lambda v: torch.from_numpy(oracle.decode(v, "bf16")).double()  # noqa: E731
    xt = dec(a["x"])
    dense = (torch.nn.functional.silu(xt @ dec(a["sw1"][0]).T) * (xt @ dec(a["sw3"][0]).T)) @ dec(a["sw2"][0]).T
    np.testing.assert_allclose(r["out"], dense.numpy(), rtol=1e-12, atol=1e-12)


def test_shared_expert_equals_a_single_routed_expert_layer():
    """A shared expert's output equals a one-expert, top-1 layer with that expert's weights
    (whose weight is exactly 1)."""
    T, d, f = 7, 16, 24
    a = _small_shared(T, d, f, 4, 2, 2, seed=8)
    ys = oracle.shared_expert_ffn(a["x"], a["sw1"], a["sw3"], a["sw2"], "f32")
    for s in range(2):
        r1 = oracle.layer_forward(a["x"], a["wg"][:1], None, a["sw1"][s:s + 1], a["sw3"][s:s + 1],
                                  a["sw2"][s:s + 1], 1, "f32")
        np.testing.assert_array_equal(ys[s], r1["out"])

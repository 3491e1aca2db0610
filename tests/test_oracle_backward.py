"""Pins of the backward oracle (``oracle.moe_backward``).

Each pin comes from outside the oracle's own formulas:
* torch.autograd in fp64 on the forward written per token (a library routine);
* central finite differences of the forward oracle along random directions
  of every input (calculus, no derivative code at all);
* invariants the softmax over the selected logits forces: the logit
  gradients of a token sum to zero, so the bias gradient sums to zero;
* special cases: k = 1 and identical experts give no gate gradient.
"""
import numpy as np
import pytest
import torch

import oracle
import moe_inputs
from conftest import to_numpy


def _inputs(T, d, f, E, k, dtype="f32", s=0.0, seed=0):
    inp = moe_inputs.random_inputs(T, d, f, E, k, dtype, s, seed)
    return {n: to_numpy(v, dtype) for n, v in inp.items()}


def _dout(T, d, seed=7):
    return np.random.default_rng(seed).standard_normal((T, d))


def _loss(inp, k, dtype, dout):
    r = oracle.layer_forward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, dtype)
    return float(np.sum(dout * r["out"])), r["topk_idx"]


def _autograd(inp, k, dout, idx):
    """Gradients of sum(dout * out) by torch.autograd, fp64, with the selection fixed to idx."""
    f64 = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, wg, bias = f64(inp["x"]), f64(inp["wg"]), f64(inp["bias"])
    w1, w3, w2 = f64(inp["w1"]), f64(inp["w3"]), f64(inp["w2"])
    T = x.shape[0]
    logits = x @ wg.T + bias
    sel = torch.tensor(idx, dtype=torch.int64)
    w = torch.softmax(torch.gather(logits, 1, sel), dim=1)
    outs = []
    for t in range(T):
        o = 0
        for j in range(k):
            e = int(idx[t, j])
            h = torch.nn.functional.silu(w1[e] @ x[t]) * (w3[e] @ x[t])
            o = o + w[t, j] * (w2[e] @ h)
        outs.append(o)
    out = torch.stack(outs)
    (out * torch.tensor(dout)).sum().backward()
    return {"dx": x.grad.numpy(), "dwg": wg.grad.numpy(), "dbias": bias.grad.numpy(),
            "dw1": w1.grad.numpy(), "dw3": w3.grad.numpy(), "dw2": w2.grad.numpy()}


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("shape", [(6, 8, 12, 4, 2), (5, 16, 8, 3, 3), (4, 8, 8, 5, 1), (3, 8, 8, 1, 1)])
def test_backward_matches_autograd(shape):
    T, d, f, E, k = shape
    inp = _inputs(T, d, f, E, k, s=0.5)
    dout = _dout(T, d)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "f32", dout)
    ref = _autograd(inp, k, dout, g["topk_idx"])
    for name in ("dx", "dw1", "dw3", "dw2"):
        assert _rel(g[name], ref[name]) < 1e-6, name
    # the gate gradients are zero at k = 1 (the weight is exactly 1); compare absolutely then
    for name in ("dwg", "dbias"):
        scale = max(np.max(np.abs(ref[name])), 1e-3)
        assert np.max(np.abs(g[name] - ref[name])) / scale < 1e-5, name


@pytest.mark.parametrize("which", ["x", "wg", "bias", "w1", "w3", "w2"])
def test_backward_finite_differences(which):
    """Central difference of the forward oracle along a random direction V:
    L(P + eps V) - L(P - eps V) = <dL/dP, (P + eps V) - (P - eps V)> + O(eps^3)."""
    T, d, f, E, k = 6, 8, 12, 4, 2
    inp = _inputs(T, d, f, E, k, s=0.5)
    dout = _dout(T, d)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "f32", dout)
    grad = {"x": g["dx"], "wg": g["dwg"], "bias": g["dbias"], "w1": g["dw1"], "w3": g["dw3"], "w2": g["dw2"]}[which]
    P = inp[which].astype(np.float32)
    V = np.random.default_rng(3).standard_normal(P.shape)
    eps = 1e-2 * float(np.sqrt(np.mean(P.astype(np.float64) ** 2)))
    plus, minus = dict(inp), dict(inp)
    plus[which] = (P + eps * V).astype(np.float32)
    minus[which] = (P - eps * V).astype(np.float32)
    lp, ip = _loss(plus, k, "f32", dout)
    lm, im = _loss(minus, k, "f32", dout)
    assert np.array_equal(ip, im) and np.array_equal(ip, g["topk_idx"]), "selection must not change"
    delta = plus[which].astype(np.float64) - minus[which].astype(np.float64)
    pred = float(np.sum(grad * delta))
    assert abs((lp - lm) - pred) <= 1e-3 * abs(pred) + 1e-9, (lp - lm, pred)


def test_selected_logit_gradients_sum_to_zero():
    T, d, f, E, k = 16, 8, 8, 6, 3
    inp = _inputs(T, d, f, E, k, s=1.0)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "f32",
                              _dout(T, d))
    # sum_j dl = (sum_i w_i dw_i) (1 - sum_j w_j): zero up to the fp32 weights' sum
    wsum_err = np.max(np.abs(g["topk_w"].astype(np.float64).sum(axis=1) - 1.0))
    assert wsum_err < 1e-6
    bound = (wsum_err + 1e-15) * np.max(np.abs(g["dtopk_w"]))
    assert np.max(np.abs(g["dlogits"].sum(axis=1))) <= bound * 1.01
    assert abs(g["dbias"].sum()) <= T * bound * 1.01
    # unselected logits get nothing
    mask = np.zeros_like(g["dlogits"], bool)
    mask[np.repeat(np.arange(T), k), g["topk_idx"].reshape(-1)] = True
    assert np.all(g["dlogits"][~mask] == 0)


def test_top1_has_no_gate_gradient():
    T, d, f, E, k = 8, 8, 8, 4, 1
    inp = _inputs(T, d, f, E, k, s=1.0)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "f32",
                              _dout(T, d))
    assert np.all(g["dlogits"] == 0) and np.all(g["dwg"] == 0) and np.all(g["dbias"] == 0)
    assert np.all(g["topk_w"] == 1.0)


def test_identical_experts_have_no_gate_gradient():
    """Identical experts make out = FFN(x) * sum(w) = FFN(x): the gate cannot matter,
    and the expert gradients of the layer are those of one dense SwiGLU, split
    over the experts by the routing weights."""
    T, d, f, E, k = 7, 8, 12, 4, 2
    inp = _inputs(T, d, f, E, k, s=0.5)
    for n in ("w1", "w3", "w2"):
        inp[n] = np.repeat(inp[n][:1], E, axis=0)
    dout = _dout(T, d)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "f32", dout)
    # dw is the same for every slot, so dl = w dw (1 - sum w): zero up to the fp32 weights' sum
    np.testing.assert_array_equal(g["dtopk_w"][:, 0], g["dtopk_w"][:, 1])
    wsum_err = np.max(np.abs(g["topk_w"].astype(np.float64).sum(axis=1) - 1.0))
    assert np.max(np.abs(g["dlogits"])) <= (wsum_err + 1e-15) * np.max(np.abs(g["dtopk_w"])) * 1.01
    # dense SwiGLU by autograd: the summed expert gradients match it
    x = torch.tensor(inp["x"].astype(np.float64), requires_grad=True)
    W1 = torch.tensor(inp["w1"][0].astype(np.float64), requires_grad=True)
    W3 = torch.tensor(inp["w3"][0].astype(np.float64), requires_grad=True)
    W2 = torch.tensor(inp["w2"][0].astype(np.float64), requires_grad=True)
    out = (torch.nn.functional.silu(x @ W1.T) * (x @ W3.T)) @ W2.T
    (out * torch.tensor(dout)).sum().backward()
    assert _rel(g["dx"], x.grad.numpy()) < 1e-6
    assert _rel(g["dw1"].sum(axis=0), W1.grad.numpy()) < 1e-5
    assert _rel(g["dw3"].sum(axis=0), W3.grad.numpy()) < 1e-5
    assert _rel(g["dw2"].sum(axis=0), W2.grad.numpy()) < 1e-5


def test_dsilu_closed_form():
    # d/dg [g sigmoid(g)] at 0 is 1/2; tends to 1 for large g and 0 for very negative g
    assert oracle.dsilu(np.array([0.0]))[0] == 0.5
    assert abs(oracle.dsilu(np.array([40.0]))[0] - 1.0) < 1e-12
    assert abs(oracle.dsilu(np.array([-40.0]))[0]) < 1e-12
    z = np.linspace(-6, 6, 25)
    h = 1e-5
    silu = lambda v: v / (1 + np.exp(-v))
    assert np.max(np.abs(oracle.dsilu(z) - (silu(z + h) - silu(z - h)) / (2 * h))) < 1e-8


def test_bf16_inputs_decode_like_forward():
    """bf16 inputs: the backward sees the same decoded values as the forward."""
    T, d, f, E, k = 5, 16, 16, 4, 2
    inp = _inputs(T, d, f, E, k, dtype="bf16", s=0.5)
    dout = _dout(T, d)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "bf16", dout)
    dec = {n: oracle.decode(inp[n], "bf16") if inp[n].dtype == np.uint16 else inp[n] for n in inp}
    ref = _autograd(dec, k, dout, g["topk_idx"])
    for name in ("dx", "dw1", "dw3", "dw2"):
        assert _rel(g[name], ref[name]) < 1e-6, name


def test_sampled_helpers_agree_with_full_backward():
    """The sampled forms used at full size give the same numbers as the full backward."""
    T, d, f, E, k = 9, 16, 24, 4, 2
    inp = _inputs(T, d, f, E, k, dtype="bf16", s=0.7)
    dout = _dout(T, d)
    g = oracle.layer_backward(inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], k, "bf16", dout)
    toks = np.array([0, 4, 8])
    tb = oracle.token_backward(inp["x"][toks], g["topk_idx"][toks], g["topk_w"][toks], inp["w1"], inp["w3"],
                               inp["w2"], inp["wg"], dout[toks], "bf16")
    assert _rel(tb["dx"], g["dx"][toks]) < 1e-12
    assert _rel(tb["dtopk_w"], g["dtopk_w"][toks]) < 1e-12
    rows = np.repeat(np.arange(toks.size), k)
    assert _rel(tb["dl"].reshape(-1), g["dlogits"][toks[rows], g["topk_idx"][toks].reshape(-1)]) < 1e-12
    _, offsets, perm, _ = oracle.dispatch(g["topk_idx"], E)
    cols = np.array([1, 7, 23])
    for e in range(E):
        sl = oracle.expert_grad_slices(inp["x"], dout, g["topk_w"], perm, offsets, inp["w1"][e], inp["w3"][e],
                                       inp["w2"][e], k, e, cols, "bf16")
        np.testing.assert_allclose(sl["dw1"], g["dw1"][e][cols], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sl["dw3"], g["dw3"][e][cols], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sl["dw2"], g["dw2"][e][:, cols], rtol=1e-12, atol=1e-14)

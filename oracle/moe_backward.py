"""Plain CPU oracle of the MoE expert layer's backward pass (gradients of the
forward defined in ``moe_oracle``).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU-baseline
leg use this module. It shares no code with the HIP path and imports nothing
from it.

The pages name the backward's parts without printing its formulas: token blocks
stream through DGrad (gradients of the activations) and WGrad (gradients of the
expert weights), and the final top-k sum is a step of its own (MegaFlux,
section 2.1, and section 3.2 with Figure 2); routing keeps each assignment's
token, slot and weight for that sum (MegaFlux, appendix A.2). What follows is
the chain rule applied to the forward's plain definition, for a scalar loss
whose gradient with respect to the layer output is ``dout``:

    out[t]  = sum_j w[t,j] * y[t,j],   y = W2_e h,  h = SiLU(g) * u,
              g = W1_e x_t,  u = W3_e x_t,  e = S_t[j]
    w[t,:]  = softmax over the k selected logits l[t, S_t[j]],
    l[t,e]  = x_t . Wg_e + bias_e.

Per assignment (t, j) of expert e:
    dw[t,j] = dout_t . y[t,j]                    (routing-weight gradient)
    dy      = w[t,j] * dout_t
    dW2_e  += dy (outer) h
    dh      = W2_e^T dy
    dg      = dh * u * s * (1 + g * (1 - s)),  s = sigmoid(g)   (d SiLU / dg)
    du      = dh * SiLU(g)
    dW1_e  += dg (outer) x_t,   dW3_e += du (outer) x_t
    dx_t   += W1_e^T dg + W3_e^T du
Softmax over the selected logits:
    dl[t,j] = w[t,j] * (dw[t,j] - sum_i w[t,i] * dw[t,i]);  unselected logits get 0
Gate:
    dbias_e = sum_t dl[t,e],  dWg_e = sum_t dl[t,e] * x_t,  dx_t += sum_e dl[t,e] * Wg_e.

Readings (listed with the other readings in the design notes):
* the routing (which experts, and their slot order) is a piecewise-constant
  function of the logits; its derivative is taken as zero, so gradients flow
  only through the weights of the selected experts;
* every gradient is computed in fp64 from the exactly decoded inputs, with the
  routing weights the forward produced (fp32, from fp32 logits);
* the bias enters the logits, so it receives the logits' gradient.

Arrays: bf16 data is passed as its raw uint16 bit patterns and decoded exactly;
fp32 data as float32. Expert weight layouts as in ``moe_oracle``:
w1, w3 [E, f, d], w2 [E, d, f], wg [E, d].
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import decode, route, dispatch

__all__ = ["layer_backward", "routing_backward", "expert_backward_sorted", "dsilu", "token_backward",
           "expert_grad_slices"]


def _sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def dsilu(g: np.ndarray) -> np.ndarray:
    """d/dg of g * sigmoid(g) = s * (1 + g * (1 - s))."""
    s = _sigmoid(g)
    return s * (1.0 + g * (1.0 - s))


def expert_backward_sorted(x, dout, w, perm, offsets, w1, w3, w2, k: int, dtype: str) -> dict:
    """DGrad and WGrad of every expert over its sorted rows, fp64.

    Row p of expert e (offsets[e] <= p < offsets[e+1]) is assignment a = perm[p]
    of token t = a // k and slot j = a % k; w is [T, k]. Returns
    dw [T, k] (dout . y per assignment), dx_ffn [T, d] (the experts' part of
    dx), dw1, dw3 [E, f, d] and dw2 [E, d, f].
    """
    xf = decode(x, dtype).astype(np.float64)
    df = np.asarray(dout, np.float64) if dout.dtype != np.uint16 else decode(dout, dtype).astype(np.float64)
    E, f, d = w1.shape
    T = xf.shape[0]
    perm = np.asarray(perm, np.int64)
    wf = np.asarray(w, np.float64).reshape(-1)
    dw = np.zeros(T * k, np.float64)
    dx = np.zeros((T, d), np.float64)
    dw1 = np.zeros((E, f, d), np.float64)
    dw3 = np.zeros((E, f, d), np.float64)
    dw2 = np.zeros((E, d, f), np.float64)
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        a = perm[p0:p1]
        t = a // k
        W1 = decode(w1[e], dtype).astype(np.float64)
        W3 = decode(w3[e], dtype).astype(np.float64)
        W2 = decode(w2[e], dtype).astype(np.float64)
        X = xf[t]
        G = X @ W1.T
        U = X @ W3.T
        S = _sigmoid(G)
        H = G * S * U
        Y = H @ W2.T
        D = df[t]
        dw[a] = np.sum(D * Y, axis=1)
        dY = wf[a][:, None] * D
        dw2[e] = dY.T @ H
        dH = dY @ W2
        dG = dH * U * dsilu(G)
        dU = dH * G * S
        dw1[e] = dG.T @ X
        dw3[e] = dU.T @ X
        np.add.at(dx, t, dG @ W1 + dU @ W3)
    return {"dw": dw.reshape(T, k), "dx_ffn": dx, "dw1": dw1, "dw3": dw3, "dw2": dw2}


def routing_backward(x, wg, idx, w, dw, dtype: str) -> dict:
    """Softmax over the selected logits, then the gate GEMM + bias, fp64.

    dl[t,j] = w[t,j] * (dw[t,j] - sum_i w[t,i] dw[t,i]); dlogits [T, E] holds dl at
    the selected experts and zero elsewhere. Returns dlogits, dbias [E],
    dwg [E, d] and dx_gate [T, d]."""
    xf = decode(x, dtype).astype(np.float64)
    wgf = decode(wg, dtype).astype(np.float64)
    T, k = idx.shape
    E = wgf.shape[0]
    wf = np.asarray(w, np.float64)
    dwf = np.asarray(dw, np.float64)
    dl = wf * (dwf - np.sum(wf * dwf, axis=1, keepdims=True))
    dlogits = np.zeros((T, E), np.float64)
    rows = np.repeat(np.arange(T), k)
    dlogits[rows, np.asarray(idx, np.int64).reshape(-1)] = dl.reshape(-1)
    return {"dl": dl, "dlogits": dlogits, "dbias": dlogits.sum(axis=0), "dwg": dlogits.T @ xf,
            "dx_gate": dlogits @ wgf}


def layer_backward(x, wg, bias, w1, w3, w2, k: int, dtype: str, dout, routing: dict | None = None) -> dict:
    """Gradients of the whole layer for output gradient dout [T, d].

    ``routing`` may carry the forward's topk_idx / topk_w / perm / offsets; they
    are recomputed with the forward oracle otherwise. Returns dx [T, d],
    dwg [E, d], dbias [E], dw1, dw3 [E, f, d], dw2 [E, d, f], dlogits [T, E],
    dtopk_w [T, k] (dout . y per assignment), all fp64."""
    E = wg.shape[0]
    if routing is None:
        _, idx, w = route(x, wg, bias, k, dtype)
        _, offsets, perm, _ = dispatch(idx, E)
    else:
        idx, w, perm, offsets = routing["topk_idx"], routing["topk_w"], routing["perm"], routing["offsets"]
    ex = expert_backward_sorted(x, dout, w, perm, offsets, w1, w3, w2, k, dtype)
    rt = routing_backward(x, wg, idx, w, ex["dw"], dtype)
    return {"dx": ex["dx_ffn"] + rt["dx_gate"], "dwg": rt["dwg"], "dbias": rt["dbias"],
            "dw1": ex["dw1"], "dw3": ex["dw3"], "dw2": ex["dw2"], "dlogits": rt["dlogits"],
            "dtopk_w": ex["dw"], "topk_idx": idx, "topk_w": w}


def token_backward(x_rows, idx_rows, w_rows, w1, w3, w2, wg, dout_rows, dtype: str) -> dict:
    """dx, dtopk_w and dlogits of a few tokens, straight from the definition
    (sampled checks at sizes where the full backward is too slow).

    x_rows [n, d], idx_rows / w_rows [n, k], dout_rows [n, d] belong to the
    sampled tokens; w1, w3, w2 index by expert (whole tensors or lazy per-expert
    lookups) and wg is [E, d]. Returns fp64 dx [n, d], dtopk_w [n, k], dl [n, k]."""
    xf = decode(x_rows, dtype).astype(np.float64)
    df = np.asarray(dout_rows, np.float64) if dout_rows.dtype != np.uint16 else decode(dout_rows, dtype).astype(np.float64)
    wgf = decode(wg, dtype).astype(np.float64)
    n, k = idx_rows.shape
    wf = np.asarray(w_rows, np.float64)
    dx = np.zeros_like(xf)
    dw = np.zeros((n, k))
    for r in range(n):
        for j in range(k):
            e = int(idx_rows[r, j])
            W1 = decode(w1[e], dtype).astype(np.float64)
            W3 = decode(w3[e], dtype).astype(np.float64)
            W2 = decode(w2[e], dtype).astype(np.float64)
            g = W1 @ xf[r]
            u = W3 @ xf[r]
            s = _sigmoid(g)
            h = g * s * u
            dw[r, j] = df[r] @ (W2 @ h)
            dh = W2.T @ (wf[r, j] * df[r])
            dx[r] += W1.T @ (dh * u * dsilu(g)) + W3.T @ (dh * g * s)
    dl = wf * (dw - np.sum(wf * dw, axis=1, keepdims=True))
    for r in range(n):
        for j in range(k):
            dx[r] += dl[r, j] * wgf[int(idx_rows[r, j])]
    return {"dx": dx, "dtopk_w": dw, "dl": dl}


def expert_grad_slices(x, dout, w, perm, offsets, w1e, w3e, w2e, k: int, e: int, cols, dtype: str) -> dict:
    """Slices of expert e's weight gradients along FFN columns `cols` (sampled
    checks): dW1_e[cols, :], dW3_e[cols, :] (rows of [f, d]) and dW2_e[:, cols]
    (columns of [d, f]); each needs only the FFN columns `cols` of every row of
    expert e. w1e, w3e [f, d] and w2e [d, f] are expert e's matrices. fp64."""
    xf = decode(x, dtype).astype(np.float64)
    df = np.asarray(dout, np.float64) if dout.dtype != np.uint16 else decode(dout, dtype).astype(np.float64)
    cols = np.asarray(cols, np.int64)
    p0, p1 = int(offsets[e]), int(offsets[e + 1])
    a = np.asarray(perm, np.int64)[p0:p1]
    X = xf[a // k]
    D = np.asarray(w, np.float64).reshape(-1)[a][:, None] * df[a // k]
    W1c = decode(w1e[cols], dtype).astype(np.float64)            # [c, d]
    W3c = decode(w3e[cols], dtype).astype(np.float64)
    W2c = decode(w2e[:, cols], dtype).astype(np.float64)         # [d, c]
    G = X @ W1c.T
    U = X @ W3c.T
    S = _sigmoid(G)
    H = G * S * U
    dH = D @ W2c
    dG = dH * U * dsilu(G)
    dU = dH * G * S
    return {"dw1": dG.T @ X, "dw3": dU.T @ X, "dw2": D.T @ H}

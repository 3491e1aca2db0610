"""A model of where the HIP backward rounds, for a white-box check (test infrastructure).

The oracle is exact (fp64); the HIP backward stores g and u in bf16 and feeds
bf16 operands w*h, dg and du to its weight-gradient products, everything else
in fp32. This module repeats the backward in fp64 with exactly those bf16
roundings (round to nearest even), so that the HIP results can be held to a
much tighter bound than the one against the exact oracle: what remains is
fp32-versus-fp64 arithmetic and the rare bf16 rounding decision that the two
take differently. It imports nothing from the HIP path.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _bf16(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(a, np.float64)).float().to(torch.bfloat16).double().numpy()


def backward_with_roundings(h: dict, dout: np.ndarray, routing: dict, k: int) -> dict:
    """h: host inputs (bf16 bit patterns) x, wg, w1, w3, w2; dout bf16 bits;
    routing: topk_idx, topk_w, perm, offsets (the oracle's). Returns dw1, dw3,
    dw2, dtopk_w, dl [T, k] and dx with the HIP path's bf16 roundings."""
    dec = lambda a: oracle.decode(a, "bf16").astype(np.float64)
    X, D = dec(h["x"]), dec(dout)
    W1, W3, W2 = dec(h["w1"]), dec(h["w3"]), dec(h["w2"])
    E = W1.shape[0]
    w = np.asarray(routing["topk_w"], np.float64).reshape(-1)
    perm, offsets = np.asarray(routing["perm"], np.int64), routing["offsets"]
    dw1, dw3, dw2 = np.zeros_like(W1), np.zeros_like(W3), np.zeros_like(W2)
    dx = np.zeros_like(X)
    dw = np.zeros_like(w)
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        a = perm[p0:p1]
        t = a // k
        g = _bf16(X[t] @ W1[e].T)
        u = _bf16(X[t] @ W3[e].T)
        s = 1.0 / (1.0 + np.exp(-g))
        hh = g * s * u
        q = D[t] @ W2[e]
        dw[a] = np.sum(q * hh, axis=1)
        dh = w[a][:, None] * q
        dg = _bf16(dh * u * s * (1.0 + g * (1.0 - s)))
        du = _bf16(dh * g * s)
        np.add.at(dx, t, dg @ W1[e] + du @ W3[e])
        dw2[e] = D[t].T @ _bf16(w[a][:, None] * hh)
        dw1[e] = dg.T @ X[t]
        dw3[e] = du.T @ X[t]
    T = X.shape[0]
    wt, dwt = w.reshape(T, k), dw.reshape(T, k)
    dl = wt * (dwt - np.sum(wt * dwt, axis=1, keepdims=True))
    Wg = dec(h["wg"])
    idx = np.asarray(routing["topk_idx"], np.int64)
    for j in range(k):
        dx += dl[:, j:j + 1] * Wg[idx[:, j]]
    return {"dw1": dw1, "dw3": dw3, "dw2": dw2, "dtopk_w": dwt, "dl": dl, "dx": dx}

"""A model of where the HIP backward rounds, for a white-box check (test infrastructure).

The oracle is exact (fp64); the HIP backward stores g and u in bf16 and feeds
bf16 operands w*h, dg and du to its weight-gradient products, everything else
in fp32. This module repeats the backward in fp64 with exactly those bf16
roundings (round to nearest even), so that the HIP results can be held to a
much tighter bound than the one against the exact oracle: what remains is
fp32-versus-fp64 arithmetic and the rare bf16 rounding decision that the two
take differently. It imports nothing from the HIP path.

Next to each result it returns the result's componentwise error scale: for
every element the sum of the magnitudes of the terms it is made of (for dg,
whose factor SiLU'(g) = s (1 + g (1 - s)) crosses zero near g = -1.28, the sum
of its two terms' magnitudes; for a gradient of the logits, which can be a
difference of larger numbers, that scale carried on instead of |dl|). A
rounding step perturbs each term by a fraction of itself, so the error of an
element is a fraction of its scale, whatever cancellation the sum has.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle


def _bf16_near(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(a, np.float64)).float().to(torch.bfloat16).double().numpy()


def _bf16_other(a: np.ndarray, r: np.ndarray) -> np.ndarray:
    """The bf16 neighbour of a on the other side from its nearest value r (r where a == r)."""
    bits = torch.from_numpy(r.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int32) & 0xFFFF
    up = np.where(r >= 0, bits + 1, bits - 1)      # one bf16 step towards +inf
    down = np.where(r > 0, bits - 1, bits + 1)     # one bf16 step towards -inf
    down = np.where(r == 0, 0x8001, down)          # below +0: the smallest negative subnormal
    nb = np.where(a > r, up, down).astype(np.uint32) & 0xFFFF
    other = (nb << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.where(a == r, r, other)


def _rounder(flip):
    """bf16 rounding, to nearest even; with flip = (rng, p) each value is instead
    rounded to its other neighbour with probability p (a rounding decision taken
    the other way, as an fp32 sum that lands on the other side of a bf16 midpoint
    from the exact sum does)."""
    def rnd(a):
        a = np.asarray(a, np.float64)
        r = _bf16_near(a)
        if flip is None:
            return r
        rng, p = flip
        return np.where(rng.random(a.shape) < p, _bf16_other(a, r), r)
    return rnd


def _dec(a):
    return oracle.decode(a, "bf16").astype(np.float64)


def _rows(X, D, wa, W1c, W3c, W2c, rnd):
    """The backward of one expert's rows on FFN columns c: X [n][d] token rows, D
    [n][d] their output gradients, wa [n] routing weights, W1c, W3c [c][d] and W2c
    [d][c] the expert's matrices restricted to the columns. Returns the per-row
    intermediates (bf16 where the HIP path rounds) and their scales."""
    g = rnd(X @ W1c.T)
    u = rnd(X @ W3c.T)
    s = 1.0 / (1.0 + np.exp(-g))
    hh = g * s * u
    q = D @ W2c
    dh = wa[:, None] * q
    dg = rnd(dh * u * s * (1.0 + g * (1.0 - s)))
    du = rnd(dh * g * s)
    hw = rnd(wa[:, None] * hh)
    return {"hh": hh, "q": q, "dg": dg, "du": du, "hw": hw,
            "dgs": np.abs(dh * u * s) * (1.0 + np.abs(g * (1.0 - s)))}


def backward_with_roundings(h: dict, dout: np.ndarray, routing: dict, k: int, flip=None) -> dict:
    """h: host inputs (bf16 bit patterns) x, wg, w1, w3, w2; dout bf16 bits;
    routing: topk_idx, topk_w, perm, offsets (the oracle's). Returns dw1, dw3,
    dw2, dtopk_w, dl [T, k], dx, dwg and dbias with the HIP path's bf16
    roundings, and under "scale" each result element's componentwise error
    scale; flip = (numpy Generator, p) takes each rounding decision the other
    way with probability p."""
    rnd = _rounder(flip)
    X, D = _dec(h["x"]), _dec(dout)
    W1, W3, W2 = _dec(h["w1"]), _dec(h["w3"]), _dec(h["w2"])
    E = W1.shape[0]
    w = np.asarray(routing["topk_w"], np.float64).reshape(-1)
    perm, offsets = np.asarray(routing["perm"], np.int64), routing["offsets"]
    dw1, dw3, dw2 = np.zeros_like(W1), np.zeros_like(W3), np.zeros_like(W2)
    a1, a3, a2 = np.zeros_like(W1), np.zeros_like(W3), np.zeros_like(W2)
    dx, ax = np.zeros_like(X), np.zeros_like(X)
    dw, adw = np.zeros_like(w), np.zeros_like(w)
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        a = perm[p0:p1]
        t = a // k
        r = _rows(X[t], D[t], w[a], W1[e], W3[e], W2[e], rnd)
        dw[a] = np.sum(r["q"] * r["hh"], axis=1)
        adw[a] = np.sum(np.abs(r["q"]) * np.abs(r["hh"]), axis=1)
        np.add.at(dx, t, r["dg"] @ W1[e] + r["du"] @ W3[e])
        np.add.at(ax, t, r["dgs"] @ np.abs(W1[e]) + np.abs(r["du"]) @ np.abs(W3[e]))
        dw2[e] = D[t].T @ r["hw"]
        dw1[e] = r["dg"].T @ X[t]
        dw3[e] = r["du"].T @ X[t]
        a2[e] = np.abs(D[t]).T @ np.abs(r["hw"])
        a1[e] = r["dgs"].T @ np.abs(X[t])
        a3[e] = np.abs(r["du"]).T @ np.abs(X[t])
    T = X.shape[0]
    wt, dwt, adwt = w.reshape(T, k), dw.reshape(T, k), adw.reshape(T, k)
    dl = wt * (dwt - np.sum(wt * dwt, axis=1, keepdims=True))
    adl = wt * (adwt + np.sum(wt * adwt, axis=1, keepdims=True))
    Wg = _dec(h["wg"])
    idx = np.asarray(routing["topk_idx"], np.int64)
    dwg, dbias = np.zeros_like(Wg), np.zeros(E)
    awg, abias = np.zeros_like(Wg), np.zeros(E)
    for j in range(k):
        dx += dl[:, j:j + 1] * Wg[idx[:, j]]
        # dl can be a difference of larger terms: its own scale adl, not |dl|, carries on
        ax += adl[:, j:j + 1] * np.abs(Wg[idx[:, j]])
        np.add.at(dwg, idx[:, j], dl[:, j:j + 1] * X)
        np.add.at(awg, idx[:, j], adl[:, j:j + 1] * np.abs(X))
        np.add.at(dbias, idx[:, j], dl[:, j])
        np.add.at(abias, idx[:, j], adl[:, j])
    return {"dw1": dw1, "dw3": dw3, "dw2": dw2, "dtopk_w": dwt, "dl": dl, "dx": dx, "dwg": dwg, "dbias": dbias,
            "scale": {"dw1": a1, "dw3": a3, "dw2": a2, "dtopk_w": adwt, "dl": adl, "dx": ax, "dwg": awg,
                      "dbias": abias}}


def token_backward_with_roundings(x_rows, dout_rows, idx_rows, w_rows, w1, w3, w2, wg) -> dict:
    """dx, dtopk_w and dl [n, k] of a few tokens with the HIP path's roundings, and
    their scales (sampled checks at sizes where the whole model is too slow).
    x_rows, dout_rows [n][d] bf16 bits; idx_rows, w_rows [n][k]; w1, w3, w2 index
    by expert (bf16 bits); wg [E][d] bf16 bits."""
    rnd = _rounder(None)
    X, D = _dec(x_rows), _dec(dout_rows)
    Wg = _dec(wg)
    n, k = idx_rows.shape
    wt = np.asarray(w_rows, np.float64)
    dwt, adwt = np.zeros((n, k)), np.zeros((n, k))
    dx, ax = np.zeros_like(X), np.zeros_like(X)
    for j in range(k):
        for e in sorted(set(int(v) for v in idx_rows[:, j])):
            rs = np.flatnonzero(idx_rows[:, j] == e)
            W1e, W3e, W2e = _dec(w1[e]), _dec(w3[e]), _dec(w2[e])
            r = _rows(X[rs], D[rs], wt[rs, j], W1e, W3e, W2e, rnd)
            dwt[rs, j] = np.sum(r["q"] * r["hh"], axis=1)
            adwt[rs, j] = np.sum(np.abs(r["q"]) * np.abs(r["hh"]), axis=1)
            dx[rs] += r["dg"] @ W1e + r["du"] @ W3e
            ax[rs] += r["dgs"] @ np.abs(W1e) + np.abs(r["du"]) @ np.abs(W3e)
    dl = wt * (dwt - np.sum(wt * dwt, axis=1, keepdims=True))
    adl = wt * (adwt + np.sum(wt * adwt, axis=1, keepdims=True))
    for j in range(k):
        dx += dl[:, j:j + 1] * Wg[idx_rows[:, j]]
        ax += adl[:, j:j + 1] * np.abs(Wg[idx_rows[:, j]])
    return {"dx": dx, "dtopk_w": dwt, "dl": dl, "scale": {"dx": ax, "dtopk_w": adwt, "dl": adl}}


def expert_slices_with_roundings(x, dout, topk_w, perm, offsets, w1e, w3e, w2e, k: int, e: int, cols) -> dict:
    """Expert e's weight-gradient slices along FFN columns cols -- dW1_e[cols, :],
    dW3_e[cols, :] and dW2_e[:, cols] -- with the HIP path's roundings, and their
    scales. x, dout bf16 bits [T][d]; w1e, w3e [f][d], w2e [d][f] bf16 bits."""
    cols = np.asarray(cols, np.int64)
    p0, p1 = int(offsets[e]), int(offsets[e + 1])
    a = np.asarray(perm, np.int64)[p0:p1]
    t = a // k
    X, D = _dec(x[t]), _dec(dout[t])
    wa = np.asarray(topk_w, np.float64).reshape(-1)[a]
    r = _rows(X, D, wa, _dec(w1e[cols]), _dec(w3e[cols]), _dec(w2e[:, cols]), _rounder(None))
    return {"dw1": r["dg"].T @ X, "dw3": r["du"].T @ X, "dw2": D.T @ r["hw"],
            "scale": {"dw1": r["dgs"].T @ np.abs(X), "dw3": np.abs(r["du"]).T @ np.abs(X),
                      "dw2": np.abs(D).T @ np.abs(r["hw"])}}


def comp_err(got, ref, scale) -> float:
    """Componentwise error: max over elements of |got - ref| / scale (the scales
    above). An element whose scale is 0 has no terms and must be exactly 0 (error
    infinite otherwise)."""
    got, ref, scale = (np.asarray(v, np.float64) for v in (got, ref, scale))
    diff = np.abs(got - ref)
    zero = scale == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    return float(np.max(diff[~zero] / scale[~zero])) if np.any(~zero) else 0.0

"""Plain, slow, obviously-correct CPU oracle of one MoE expert layer's forward pass.

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU-baseline
leg use this module. It shares no code with the HIP path and imports nothing
from it.

What the layer computes (the plain definition). With S_t the ordered top-k
experts of token t and w_{t,j} their renormalised softmax weights,

    out[t] = sum_{j<k} w_{t,j} * W2_e^T ( SiLU(W1_e^T x_t) * (W3_e^T x_t) ),  e = S_t[j]

Sources on the pages:
* gating network decides each token's experts (MegaScale-Infer, 3.2 Big-Picture
  Architecture, item 2);
* the routing steps -- top-k selection from the gate output, per-expert token
  counts, weight normalisation, scatter of tokens into per-expert buffers
  (MegaScale-Infer, Supporting Implementation Details, "Fused Kernels");
* per-expert assignment order: by source and local token, then top-k position,
  with token identity, slot and weight kept for the final combine (MegaFlux,
  appendix A.2, last item);
* tile-aligned token blocks of at most beta rows, at most one partial block per
  expert (MegaFlux, section 3.1);
* SwiGLU expert with gate, up and down matrices (Piper, section III-A and
  Table III); FC1 then FC2 per expert and a separate final top-k sum (MegaFlux,
  section 2.1);
* shared experts, always active besides the routed ones (Piper, Table III
  notation; DeepSeek-V3: 256 routed + 1 shared, Piper Table I, note b).

Readings where the pages are silent (each one is listed in the design notes):
* logits are x . Wg_e plus a per-expert bias, added once after the dot product;
* the fp32 summation order of each logit is fixed (see ``gate_logits``), so that
  routing is reproducible bit for bit;
* top-k order: logit descending, ties to the lower expert index, -0 == +0;
* weights: softmax over the k selected logits (bias included);
* W1 is the gated (SiLU) projection, W3 the up projection;
* SiLU(z) = z / (1 + exp(-z));
* FFN and combine are computed in fp64 with no intermediate rounding;
* a shared expert is a SwiGLU expert of the same sizes that every token passes
  through; its output is added with weight 1, outside the renormalised softmax
  (shared experts in ascending order after the routed sum).

Arrays: bf16 data is passed as its raw uint16 bit patterns and decoded exactly
(fp32 bits = u16 << 16); fp32 data as float32.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode", "gate_logits", "topk_select", "topk_weights", "route", "dispatch",
    "block_plan", "expert_ffn_sorted", "combine", "layer_forward", "token_outputs",
    "shared_expert_ffn", "layer_forward_shared", "WAVE",
]

WAVE = 64  # lane classes of the fixed logit summation order


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of stored data: bf16 as uint16 bit patterns, or fp32."""
    if dtype == "bf16":
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint16:
            a = a.view(np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def gate_logits(x: np.ndarray, wg: np.ndarray, bias, dtype: str, token_chunk: int = 256) -> np.ndarray:
    """Gate logits l[t, e] = fl32(dot(x_t, Wg_e) + bias_e) in the fixed fp32 order.

    The pages only say that a gating network scores every token against every
    expert (MegaScale-Infer, 3.2 item 2). The summation order is this
    library's contract, chosen so that top-k routing is reproducible bit for
    bit:
      1. product p_i = fl32(x[t,i] * Wg[e,i]) (exact for bf16 operands);
      2. 64 lane classes: s_j = sequential fp32 sum, starting from +0.0, of the
         p_i with i = j (mod 64) in increasing i;
      3. butterfly: for off = 32, 16, 8, 4, 2, 1: s_j = fl32(s_j + s_{j+off})
         for every j < off;
      4. l = fl32(s_0 + bias_e).
    x: [T, d]; wg: [E, d]; bias: [E] float32 or None. Returns float32 [T, E].
    """
    xf = decode(x, dtype)
    wf = decode(wg, dtype)
    T, d = xf.shape
    E = wf.shape[0]
    assert wf.shape[1] == d
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    out = np.empty((T, E), np.float32)
    for t0 in range(0, T, token_chunk):
        xs = xf[t0:t0 + token_chunk]
        s = np.zeros((xs.shape[0], E, WAVE), np.float32)
        for i0 in range(0, d, WAVE):
            n = min(WAVE, d - i0)
            # step 1 (float32 multiply) and step 2 (float32 add), one lane class per column
            p = xs[:, None, i0:i0 + n] * wf[None, :, i0:i0 + n]
            s[:, :, :n] += p
        off = WAVE // 2
        while off >= 1:
            s[:, :, :off] = s[:, :, :off] + s[:, :, off:2 * off]
            off //= 2
        out[t0:t0 + token_chunk] = s[:, :, 0] + b[None, :]
    return out


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert indices per token, slot j = j-th largest logit.

    Order: logit descending, equal logits (with -0 == +0) to the lower expert
    index (MegaScale-Infer, "Fused Kernels", step 1: top-k from the gate output).
    A stable sort of the negated logits gives exactly this order.
    Returns int32 [T, k].
    """
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Renormalised softmax over the k selected logits, fp64, stored as fp32.

    w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), l_0 the largest selected logit
    (MegaScale-Infer, "Fused Kernels", step 3: normalise the token weights).
    """
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def route(x, wg, bias, k: int, dtype: str):
    """Gate GEMM + bias, top-k and renormalised weights. Returns (logits, idx, w)."""
    logits = gate_logits(x, wg, bias, dtype)
    idx = topk_select(logits, k)
    return logits, idx, topk_weights(logits, idx)


def dispatch(idx: np.ndarray, E: int):
    """Per-expert counts, exclusive offsets and the stable assignment permutation.

    Assignment a = t*k + j. counts[e] = #{a : idx[a] = e}; offsets = exclusive
    prefix sum with offsets[E] = T*k; perm[p] = a sorts assignments by expert,
    keeping token-then-slot order inside each expert (MegaScale-Infer "Fused
    Kernels" steps 2 and 4; MegaFlux appendix A.2 assignment order);
    inv_perm[a] = p. All int32.
    """
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")
    inv_perm = np.empty_like(perm)
    inv_perm[perm] = np.arange(perm.size)
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv_perm.astype(np.int32))


def block_plan(counts: np.ndarray, beta: int):
    """Tile-aligned token blocks: each expert's sorted rows cut into blocks of at
    most beta rows, only the last one partial (MegaFlux, section 3.1).
    Returns a list of (expert, first_row, rows) in expert order."""
    blocks = []
    start = 0
    for e, c in enumerate(np.asarray(counts).tolist()):
        for r0 in range(0, c, beta):
            blocks.append((e, start + r0, min(beta, c - r0)))
        start += c
    return blocks


def _silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn_sorted(x, perm, offsets, w1, w3, w2, k: int, dtype: str) -> np.ndarray:
    """y[p] = W2_e^T (SiLU(W1_e^T x_t) * W3_e^T x_t) for every sorted row p, fp64.

    Row p belongs to expert e with offsets[e] <= p < offsets[e+1] and to token
    t = perm[p] // k. SwiGLU expert: Piper section III-A; FC1/FC2 per expert:
    MegaFlux section 2.1. W1 = gate (SiLU) projection, W3 = up projection.
    w1, w3: [E, f, d]; w2: [E, d, f]. Returns float64 [T*k, d].
    """
    xf = decode(x, dtype).astype(np.float64)
    E = w1.shape[0]
    d = xf.shape[1]
    perm = np.asarray(perm, np.int64)
    y = np.zeros((perm.size, d), np.float64)
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        xe = xf[perm[p0:p1] // k]
        g = xe @ decode(w1[e], dtype).astype(np.float64).T
        u = xe @ decode(w3[e], dtype).astype(np.float64).T
        h = _silu(g) * u
        y[p0:p1] = h @ decode(w2[e], dtype).astype(np.float64).T
    return y


def combine(y_sorted: np.ndarray, inv_perm, w: np.ndarray, k: int) -> np.ndarray:
    """out[t] = sum_{j<k} w[t,j] * y[inv_perm[t*k+j]], j ascending, fp64
    (MegaFlux section 2.1: the final top-k sum is its own step)."""
    T = w.shape[0]
    inv = np.asarray(inv_perm, np.int64).reshape(T, k)
    out = np.zeros((T, y_sorted.shape[1]), np.float64)
    for j in range(k):
        out += w[:, j:j + 1].astype(np.float64) * y_sorted[inv[:, j]]
    return out


def layer_forward(x, wg, bias, w1, w3, w2, k: int, dtype: str) -> dict:
    """The whole layer: route, dispatch, expert FFN, combine."""
    E = wg.shape[0]
    logits, idx, w = route(x, wg, bias, k, dtype)
    counts, offsets, perm, inv_perm = dispatch(idx, E)
    y = expert_ffn_sorted(x, perm, offsets, w1, w3, w2, k, dtype)
    out = combine(y, inv_perm, w, k)
    return {"logits": logits, "topk_idx": idx, "topk_w": w, "counts": counts, "offsets": offsets,
            "perm": perm, "inv_perm": inv_perm, "y_sorted": y, "out": out}


def token_outputs(x, idx, w, w1, w3, w2, tokens, dtype: str) -> np.ndarray:
    """out[t] for the listed tokens straight from the definition (no permutation).

    Used for sampled checks at sizes where the full oracle is too slow; each
    needed expert's weights are decoded once. Returns float64 [len(tokens), d].
    """
    tokens = np.asarray(tokens, np.int64)
    xf = decode(x[tokens], dtype).astype(np.float64)
    k = idx.shape[1]
    ys = np.zeros((tokens.size, k, xf.shape[1]), np.float64)
    need = {}
    for r, t in enumerate(tokens.tolist()):
        for j in range(k):
            need.setdefault(int(idx[t, j]), []).append((r, j))
    for e, uses in sorted(need.items()):
        W1 = decode(w1[e], dtype).astype(np.float64)
        W3 = decode(w3[e], dtype).astype(np.float64)
        W2 = decode(w2[e], dtype).astype(np.float64)
        xe = xf[[r for r, _ in uses]]
        y = (_silu(xe @ W1.T) * (xe @ W3.T)) @ W2.T
        for n, (r, j) in enumerate(uses):
            ys[r, j] = y[n]
    out = np.zeros((tokens.size, xf.shape[1]), np.float64)
    for j in range(k):
        out += w[tokens, j:j + 1].astype(np.float64) * ys[:, j]
    return out


def shared_expert_ffn(x, sw1, sw3, sw2, dtype: str) -> np.ndarray:
    """y_s[t] = W2_s^T (SiLU(W1_s^T x_t) * W3_s^T x_t) for every shared expert s
    and token t, fp64 (every token passes through every shared expert: Piper,
    Table III notation). sw1, sw3: [S, f, d]; sw2: [S, d, f]. Returns [S, T, d]."""
    xf = decode(x, dtype).astype(np.float64)
    S = sw1.shape[0]
    y = np.zeros((S, xf.shape[0], xf.shape[1]), np.float64)
    for s in range(S):
        g = xf @ decode(sw1[s], dtype).astype(np.float64).T
        u = xf @ decode(sw3[s], dtype).astype(np.float64).T
        y[s] = (_silu(g) * u) @ decode(sw2[s], dtype).astype(np.float64).T
    return y


def layer_forward_shared(x, wg, bias, w1, w3, w2, sw1, sw3, sw2, k: int, dtype: str) -> dict:
    """The layer with shared experts: the routed layer's output plus, with weight
    1 and in ascending order, every shared expert's output for the token."""
    r = layer_forward(x, wg, bias, w1, w3, w2, k, dtype)
    ys = shared_expert_ffn(x, sw1, sw3, sw2, dtype)
    out = r["out"].copy()
    for s in range(ys.shape[0]):
        out += ys[s]
    r["routed_out"] = r["out"]
    r["y_shared"] = ys
    r["out"] = out
    return r

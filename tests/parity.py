"""Shared helpers of the parity tests (test infrastructure)."""
from __future__ import annotations

import numpy as np
import torch

import moe_inputs
import oracle
from conftest import to_numpy

# Output tolerance: max over elements of |gpu - ref| / max(|ref|, rms(ref)).
# bf16 inputs with fp32 accumulation; the intermediate h and y are rounded to
# bf16 on the GPU and not in the fp64 oracle (about 2^-9 relative each).
OUT_TOL = 2e-2
# Combine weights: fp32 exp/divide on the GPU against the fp64 oracle.
W_TOL = 1e-5


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


def gpu_float(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_inputs(inp: dict, dtype: str) -> dict:
    """Host copies (oracle format) of the small tensors; weights are fetched per expert on demand."""
    return {n: to_numpy(inp[n], dtype) for n in ("x", "wg", "bias")}


class LazyExperts:
    """Index by expert -> host numpy copy of one expert's weight matrix (oracle format)."""

    def __init__(self, t: torch.Tensor, dtype: str):
        self.t, self.dtype, self.cache = t, dtype, {}
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = to_numpy(self.t[e], self.dtype)
        return self.cache[e]


def oracle_logits_threaded(x, wg, bias, dtype, threads=16, chunk=128):
    """The oracle's gate logits, token slices computed in parallel threads (rows are independent)."""
    from concurrent.futures import ThreadPoolExecutor
    T = x.shape[0]
    parts = [(t0, min(T, t0 + chunk)) for t0 in range(0, T, chunk)]
    with ThreadPoolExecutor(threads) as ex:
        outs = list(ex.map(lambda p: oracle.gate_logits(x[p[0]:p[1]], wg, bias, dtype), parts))
    return np.concatenate(outs, axis=0) if outs else np.zeros((0, wg.shape[0]), np.float32)


def oracle_routing(h: dict, k: int, dtype: str, threads=16):
    logits = oracle_logits_threaded(h["x"], h["wg"], h["bias"], dtype, threads)
    idx = oracle.topk_select(logits, k)
    w = oracle.topk_weights(logits, idx)
    counts, offsets, perm, inv = oracle.dispatch(idx, h["wg"].shape[0])
    return {"logits": logits, "topk_idx": idx, "topk_w": w, "counts": counts, "offsets": offsets,
            "perm": perm, "inv_perm": inv}


def assert_routing_equal(gpu: dict, ref: dict, names=("logits", "topk_idx", "counts", "offsets", "perm", "inv_perm")):
    for n in names:
        g = gpu[n].detach().cpu().numpy()
        r = np.asarray(ref[n]).reshape(g.shape)
        if n == "logits":
            bad = np.flatnonzero(g.view(np.uint32).ravel() != r.astype(np.float32).view(np.uint32).ravel())
        else:
            bad = np.flatnonzero(g.ravel() != r.ravel())
        assert bad.size == 0, f"{n}: {bad.size} mismatches, first at flat index {bad[:5].tolist()}"
    if "topk_w" in gpu:
        g = gpu["topk_w"].detach().cpu().numpy().astype(np.float64)
        r = np.asarray(ref["topk_w"], np.float64)
        assert np.max(np.abs(g - r) / np.maximum(np.abs(r), 1e-30)) <= W_TOL


def make_case(cfg, seed=0, device="cuda"):
    inp = moe_inputs.make_layer_inputs(cfg, seed, device)
    return inp


class OneExpert:
    """A single expert's matrix presented as a one-expert stack (shape [1, ...], index 0)."""

    def __init__(self, m: np.ndarray):
        self.m = m
        self.shape = (1,) + tuple(m.shape)

    def __getitem__(self, e):
        assert int(e) == 0
        return self.m


def oracle_outputs_threaded(h: dict, w1, w3, w2, idx, w, tokens, k: int, dtype: str, threads=16):
    """out[t] for the listed tokens (all tokens when tokens is None), computed by the oracle's
    own functions: each expert's rows through oracle.expert_ffn_sorted (one call per expert,
    the experts spread over threads), then oracle.combine over the (token, slot) rows.
    w1, w3, w2: host arrays [E][...] in the oracle's format. Returns float64 [len(tokens), d]."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    T = idx.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    sel = idx[tokens]                                  # [n, k] experts of the sampled tokens
    # assignment a = r*k + j of sampled token r, slot j; its row of x is tokens[r]
    flat = sel.reshape(-1).astype(np.int64)
    x_rows = h["x"][tokens]
    y = np.zeros((flat.size, x_rows.shape[1]), np.float64)

    def one(e):
        a = np.flatnonzero(flat == e)                  # assignments of expert e, in order
        ye = oracle.expert_ffn_sorted(x_rows, a.astype(np.int32), np.array([0, a.size], np.int32),
                                      OneExpert(w1[e]), OneExpert(w3[e]), OneExpert(w2[e]), k, dtype)
        y[a] = ye
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, sorted(set(flat.tolist()))))
    inv = np.arange(flat.size, dtype=np.int32)        # row r*k + j holds (token r, slot j)
    return oracle.combine(y, inv, np.asarray(w)[tokens], k)


def check_plan(blocks: np.ndarray, counts, offsets, beta: int, n_rows: int):
    """Invariants of a tile plan (MegaFlux, section 3.1): every sorted row of every expert
    is covered by exactly one m-block of that expert, every block has 1..beta rows and at
    most one per expert has fewer than beta, the rows add up to n_rows, and the tile-group
    field names a run of at most 8 m-blocks of one expert that contains the block."""
    blocks = np.asarray(blocks, np.int64).reshape(-1, 4)
    counts = np.asarray(counts, np.int64)
    offsets = np.asarray(offsets, np.int64)
    E = counts.size
    assert blocks[:, 2].sum() == n_rows, "rows do not add up to T*k"
    cover = np.zeros(n_rows, np.int64)
    partial = np.zeros(E, np.int64)
    for i, (e, r0, rows, info) in enumerate(blocks.tolist()):
        assert 0 <= e < E, f"block {i}: expert {e}"
        assert 1 <= rows <= beta, f"block {i}: {rows} rows"
        assert offsets[e] <= r0 and r0 + rows <= offsets[e + 1], f"block {i} leaves expert {e}'s rows"
        cover[r0:r0 + rows] += 1
        partial[e] += rows < beta
        m0, gs = info >> 4, info & 15
        assert 1 <= gs <= 8 and m0 <= i < m0 + gs <= len(blocks), f"block {i}: group ({m0}, {gs})"
        assert (blocks[m0:m0 + gs, 0] == e).all(), f"block {i}: group spans experts"
    assert (cover == 1).all(), f"rows covered {cover.min()}..{cover.max()} times"
    assert (partial <= 1).all(), f"experts with {partial.max()} partial blocks"
    assert len(blocks) == sum(-(-int(c) // beta) for c in counts)

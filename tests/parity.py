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

"""The training pair through the C ABI: moe_layer_forward_train keeps FC1's
g | u rows, and moe_layer_backward_saved reads them instead of recomputing FC1.

* routing arrays: bit for bit those of moe_layer_forward (the same kernels);
* out: the forward's 2e-2 bar against the fp64 oracle (h is formed from the
  fp32 sums, as in the plain forward);
* gu: g = x W1_e^T and u = x W3_e^T of every sorted row, in fp64, within
  2e-2 with the rms floor (one bf16 rounding of an fp32 sum);
* every gradient of moe_layer_backward_saved bit for bit moe_layer_backward's
  (whose parity with the backward oracle is tested on its own), so the kept
  g | u is exactly the backward's recompute.
Small shapes check every element; the Mixtral prefill and DeepSeek-shaped
workloads check sampled tokens and rows (the first, middle and last row of
each expert, of up to 16 experts including the largest), and every gradient
element bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
import mixture_experts_layer_gate_amd as moe
from conftest import to_numpy
from parity import LazyExperts, gpu_float, host_inputs, oracle_outputs_threaded, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
ROUTING = ("logits", "topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm")
GRADS = ("dx", "dwg", "dbias", "dw1", "dw3", "dw2", "dlogits", "dtopk_w")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gu_reference(x, w1, w3, perm, offsets, k, rows, dtype):
    """fp64 g | u of the listed sorted rows: expert e owns offsets[e] <= p < offsets[e+1],
    row p is token perm[p] // k."""
    xf = oracle.decode(x, dtype).astype(np.float64)
    offsets = np.asarray(offsets, np.int64)
    rows = np.asarray(list(rows), np.int64)
    experts = np.searchsorted(offsets, rows, side="right") - 1
    out = np.zeros((rows.size, 2 * w1.shape[1]), np.float64)
    for e in np.unique(experts):
        sel = np.flatnonzero(experts == e)
        xe = xf[np.asarray(perm, np.int64)[rows[sel]] // k]
        out[sel] = np.concatenate([xe @ oracle.decode(w1[int(e)], dtype).astype(np.float64).T,
                                   xe @ oracle.decode(w3[int(e)], dtype).astype(np.float64).T], axis=1)
    return out


def _train_and_plain(dims, inp, dout):
    out_p, r_p = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                                   return_routing=True)
    out_t, r_t, gu = moe.layer_forward_train(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"],
                                             inp["w2"])
    for n in ROUTING:
        assert torch.equal(r_t[n], r_p[n]), n
    ws = torch.empty(moe.backward_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    g_re = moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r_t, dout, ws=ws,
                              want_dlogits=True, want_dtopk_w=True)
    g_sv = moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r_t, dout, ws=ws,
                              want_dlogits=True, want_dtopk_w=True, gu=gu)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g_sv[n], g_re[n]), n
    return out_p, out_t, r_t, gu


SHAPES = [
    # T, d, f, E, k, bias scale
    (200, 256, 512, 8, 2, 0.0),      # one partial m-block per expert
    (300, 512, 768, 4, 2, 1.0),      # skewed, f = 3 x 256
    (64, 256, 256, 16, 4, 2.0),      # experts without rows
    (1500, 256, 512, 4, 2, 1.0),     # experts over several 256-row m-blocks, ragged tails
    (700, 1024, 512, 2, 1, 0.0),     # k = 1
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_train_pair_small(shape):
    T, d, f, E, k, s = shape
    _say(f"case train pair {shape}")
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, 0, device="cuda")
    dout = moe_inputs.output_grad(T, d, "bf16", 0, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    _, out_t, r, gu = _train_and_plain(dims, inp, dout)
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    ref = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")
    assert rel_err(gpu_float(out_t), ref["out"]) <= TOL
    perm, offsets = r["perm"].cpu().numpy(), r["offsets"].cpu().numpy()
    gu_ref = _gu_reference(h["x"], h["w1"], h["w3"], perm, offsets, k, range(T * k), "bf16")
    assert rel_err(gpu_float(gu), gu_ref) <= TOL


def test_train_pair_twice_on_one_workspace():
    """A second training forward on the same workspace, with fewer tokens, gives
    the result of a fresh call."""
    d, f, E, k = 256, 512, 8, 2
    ws = torch.empty(moe.workspace_bytes(moe.Dims(600, d, f, E, k, torch.bfloat16)), dtype=torch.uint8,
                     device="cuda")
    for T in (600, 250):
        inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", 1.0, T, device="cuda")
        dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
        a = moe.layer_forward_train(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"], ws=ws)
        b = moe.layer_forward_train(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"])
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_prefill_skew", "deepseek_skew"])
def test_train_pair_full_size_sampled(name):
    cfg = moe_inputs.config(name)
    _say(f"case train pair full {cfg.name}: generating inputs on the GPU")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dout = moe_inputs.output_grad(cfg.T, cfg.d, cfg.dtype, 0, device="cuda")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    _say("  forwards and both backwards")
    _, out_t, r, gu = _train_and_plain(dims, inp, dout)
    h = host_inputs(inp, cfg.dtype)
    w1, w3, w2 = (LazyExperts(inp[n], cfg.dtype) for n in ("w1", "w3", "w2"))
    idx, w = r["topk_idx"].cpu().numpy(), r["topk_w"].cpu().numpy()
    toks = np.unique(np.linspace(0, cfg.T - 1, 8).astype(np.int64))
    _say("  oracle on sampled tokens")
    ref = oracle_outputs_threaded(h, w1, w3, w2, idx, w, toks, cfg.k, cfg.dtype)
    assert rel_err(gpu_float(out_t[toks]), ref) <= TOL
    perm, offsets = r["perm"].cpu().numpy(), r["offsets"].cpu().numpy()
    rows = []
    counts = np.diff(offsets)
    experts = range(cfg.E) if cfg.E <= 16 else sorted(
        set(np.linspace(0, cfg.E - 1, 15).astype(int).tolist()) | {int(np.argmax(counts))})
    for e in experts:
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 > p0:
            rows += sorted({p0, (p0 + p1) // 2, p1 - 1})
    gu_ref = _gu_reference(h["x"], w1, w3, perm, offsets, cfg.k, rows, cfg.dtype)
    assert rel_err(gpu_float(gu[rows]), gu_ref) <= TOL

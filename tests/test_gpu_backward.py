"""Parity of the HIP backward pass with the CPU oracle, through the C ABI.

Bars. The backward is outside the forward's 2e-2 statement. Its bars are
derived on the CPU in tests/backward_bars.py from the backward's arithmetic,
without looking at GPU results: the rounding model (tests/rounding_model.py)
repeats the GPU's bf16 roundings (g and u stored in bf16; w*h, dg and du
rounded to bf16 as matrix-product operands) in fp64, and the same model with
a fraction of its rounding decisions flipped stands for the decisions fp32
accumulation takes the other way. Over the test shapes and five seeds, twice
the largest spread gives:
* NORM_TOL, every gradient normwise against the exact oracle;
* ACT_TOL and ACT_MODEL_TOL, the per-token results (dx, dtopk_w, the selected
  logits' gradients) elementwise with the forward's rms floor, against the
  exact oracle and against the rounding model: a wrong token row is off by
  about its own size;
* COMP_TOL and MODEL_TOL, the per-expert sums (dw1, dw3, dw2, dwg, dbias)
  componentwise, the error of an element over its sum of |terms| (the model's
  scale), against the oracle and against the model: sums with cancellation
  (the gradients of experts with few rows) do not inflate it, and a swapped
  row of such a sum is off by about its scale.
Small shapes compare every element of every gradient; the full-size workloads
compare sampled tokens (dx, dtopk_w, the selected logits' gradients) and
sampled FFN columns of the weight gradients the same ways (the rounding model
computes just those), and check the gate gradients against the GPU's own
dlogits (dbias = column sums, dwg = dlogits^T x, fp64).
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs
import oracle
import mixture_experts_layer_gate_amd as moe
from conftest import to_numpy
from parity import LazyExperts, assert_routing_equal, gpu_float, host_inputs, oracle_routing, rel_err
from rounding_model import (backward_with_roundings, comp_err, expert_slices_with_roundings,
                            token_backward_with_roundings)

pytestmark = pytest.mark.gpu

GRADS = ("dx", "dwg", "dbias", "dw1", "dw3", "dw2", "dlogits", "dtopk_w")
WEIGHT_GRADS = ("dw1", "dw3", "dw2")
PER_TOKEN = ("dx", "dtopk_w", "dl")
PER_EXPERT = ("dw1", "dw3", "dw2", "dwg", "dbias")   # sums over one expert's rows
# derived bars (tests/backward_bars.py: twice the largest spread of the rounding
# model over the test shapes and seeds 0-4)
NORM_TOL = 2e-2
ACT_TOL = 7e-2
ACT_MODEL_TOL = 3e-2
COMP_TOL = 5e-2
MODEL_TOL = 3e-2


def norm_err(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def elem_errs(n: str, got, ref, model, scale) -> tuple:
    """(error against the oracle, bar, error against the rounding model, bar) of gradient
    n: per-token results with the rms floor, per-expert sums componentwise."""
    if n in PER_TOKEN:
        return rel_err(got, ref), ACT_TOL, rel_err(got, model), ACT_MODEL_TOL
    return comp_err(got, ref, scale), COMP_TOL, comp_err(got, model, scale), MODEL_TOL


def check_grads(g: dict, ref: dict, model: dict, idx: np.ndarray) -> dict:
    """Every gradient against the exact oracle (normwise and elementwise) and against
    the rounding model (elementwise); the logits that were not selected get exactly 0.
    Returns the errors."""
    T, k = idx.shape
    got = {n: gpu_float(g[n]) for n in GRADS}
    for n, v in got.items():
        assert np.all(np.isfinite(v)), n
    dlog = got.pop("dlogits")
    rows = np.arange(T)[:, None]
    got["dl"] = dlog[rows, idx]
    unsel = np.ones_like(dlog, dtype=bool)
    unsel[rows, idx] = False
    assert not np.any(dlog[unsel]), "gradient on a logit that was not selected"
    ref = dict(ref, dl=ref["dlogits"][rows, idx])
    errs = {}
    for n, v in got.items():
        if np.any(ref[n]):
            errs[n + "_norm"] = norm_err(v, ref[n])
            assert errs[n + "_norm"] <= NORM_TOL, n
        errs[n], bar, errs[n + "_model"], mbar = elem_errs(n, v, ref[n], model[n], model["scale"][n])
        assert errs[n] <= bar, n
        assert errs[n + "_model"] <= mbar, n
    return errs


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _forward_backward(T, d, f, E, k, s, seed=0, forced=False):
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed, device="cuda")
    if forced:
        inp["bias"] = inp["bias"].clone()
        inp["bias"][:k] += 1e4
    dout = moe_inputs.output_grad(T, d, "bf16", seed, device="cuda")
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    _, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                             return_routing=True)
    g = moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r, dout,
                           want_dlogits=True, want_dtopk_w=True)
    torch.cuda.synchronize()
    return inp, dout, r, g


BWD_SHAPES = [
    # T, d, f, E, k, bias scale
    (200, 256, 512, 8, 2, 0.0),     # several n-blocks, one partial m-block per expert
    (300, 512, 768, 4, 2, 1.0),     # skewed: K windows of 1..6 steps, f = 3 x 256
    (64, 256, 256, 16, 4, 2.0),     # many experts, some with no rows (zero gradients)
    (129, 256, 512, 8, 1, 0.5),     # top-1: no gate gradient
    (40, 256, 256, 8, 8, 0.0),      # k = E: every expert selected
    (1, 256, 256, 4, 2, 0.0),       # a single token
    (600, 256, 256, 2, 2, 0.0),     # 600 rows per expert: three m-blocks, ten K steps
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_backward_small_shapes(shape):
    T, d, f, E, k, s = shape
    _say(f"case backward {shape}")
    inp, dout, r, g = _forward_backward(T, d, f, E, k, s)
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    fw = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")
    assert_routing_equal(r, fw)
    ref = oracle.layer_backward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16",
                                to_numpy(dout, "bf16"), routing=fw)
    model = backward_with_roundings(h, to_numpy(dout, "bf16"), fw, k)
    errs = check_grads(g, ref, model, np.asarray(fw["topk_idx"]))
    _say("  " + " ".join(f"{n}={v:.2e}" for n, v in errs.items()))
    # experts without rows get exactly zero weight gradients
    counts = r["counts"].cpu().numpy()
    for e in np.nonzero(counts == 0)[0]:
        for name in ("dw1", "dw3", "dw2"):
            assert not torch.any(g[name][int(e)]), (name, e)


def _random_bwd_shapes(n=16, seed=20261203):
    """Seeded random shapes: tokens 1..500, d and f multiples of 256 up to 768,
    1..64 experts, top-1..4, gate bias 0, 1 or 2 times -ln(rank)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
        k = int(rng.integers(1, min(E, 4) + 1))
        out.append((int(rng.integers(1, 501)), 256 * int(rng.integers(1, 4)), 256 * int(rng.integers(1, 4)),
                    E, k, float(rng.choice([0.0, 1.0, 2.0]))))
    return out


@pytest.mark.parametrize("shape", _random_bwd_shapes(), ids=lambda s: "T{}_d{}_f{}_E{}_k{}_s{}".format(*s))
def test_backward_random_shapes(shape):
    test_backward_small_shapes(shape)


def test_backward_forced_routing():
    """All tokens on experts 0..k-1 (bias +1e4): one expert per slot, the rest empty."""
    T, d, f, E, k = 300, 256, 512, 8, 2
    _say("case backward forced routing")
    inp, dout, r, g = _forward_backward(T, d, f, E, k, 0.0, forced=True)
    counts = r["counts"].cpu().numpy()
    assert list(counts) == [T] * k + [0] * (E - k)
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    fw = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")
    ref = oracle.layer_backward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16",
                                to_numpy(dout, "bf16"), routing=fw)
    model = backward_with_roundings(h, to_numpy(dout, "bf16"), fw, k)
    errs = check_grads(g, ref, model, np.asarray(fw["topk_idx"]))
    _say("  " + " ".join(f"{n}={v:.2e}" for n, v in errs.items()))


def test_backward_deterministic_and_zero_batch():
    T, d, f, E, k = 150, 256, 256, 8, 2
    _say("case backward determinism")
    inp, dout, r, g1 = _forward_backward(T, d, f, E, k, 1.0)
    dims = moe.Dims(T, d, f, E, k, torch.bfloat16)
    g2 = moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r, dout,
                            want_dlogits=True, want_dtopk_w=True)
    torch.cuda.synchronize()
    for name in GRADS:
        assert torch.equal(g1[name], g2[name]), name
    # T = 0: the weight gradients are written as zeros
    dims0 = moe.Dims(0, d, f, E, k, torch.bfloat16)
    z = {n: torch.empty(0, dtype=torch.int32, device="cuda") for n in ("perm", "inv_perm")}
    z["topk_idx"] = torch.empty((0, k), dtype=torch.int32, device="cuda")
    z["topk_w"] = torch.empty((0, k), dtype=torch.float32, device="cuda")
    z["counts"] = torch.zeros(E, dtype=torch.int32, device="cuda")
    z["offsets"] = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    filled = {n: torch.full_like(g1[n], 7.0) for n in ("dwg", "dbias", "dw1", "dw3", "dw2")}
    filled["dx"] = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    x0 = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    out = moe.layer_backward(dims0, x0, inp["wg"], inp["w1"], inp["w3"], inp["w2"], z, x0, grads=filled)
    torch.cuda.synchronize()
    for n in ("dwg", "dbias", "dw1", "dw3", "dw2"):
        assert not torch.any(out[n]), n


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_prefill_skew", "deepseek_skew"])
def test_backward_full_size_sampled(name):
    cfg = moe_inputs.config(name)
    _say(f"case backward full {name}: generating inputs on the GPU")
    inp = moe_inputs.make_layer_inputs(cfg, 0, "cuda")
    dout = moe_inputs.output_grad(cfg.T, cfg.d, cfg.dtype, 0, device="cuda")
    dims = moe.Dims(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.torch_dtype)
    _, r = moe.layer_forward(dims, inp["x"], inp["wg"], inp["bias"], inp["w1"], inp["w3"], inp["w2"],
                             return_routing=True)
    _say("  backward")
    g = moe.layer_backward(dims, inp["x"], inp["wg"], inp["w1"], inp["w3"], inp["w2"], r, dout,
                           want_dlogits=True, want_dtopk_w=True)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.isfinite(g[n].float()).all(), n
    h = host_inputs(inp, cfg.dtype)
    _say("  oracle routing")
    ref = oracle_routing(h, cfg.k, cfg.dtype)
    assert_routing_equal(r, ref)
    dout_h = to_numpy(dout, cfg.dtype)
    w1, w3, w2 = (LazyExperts(inp[n], cfg.dtype) for n in ("w1", "w3", "w2"))
    # sampled tokens: dx, dtopk_w and the selected logits' gradients
    toks = np.unique(np.linspace(0, cfg.T - 1, 6).astype(np.int64))
    _say(f"  oracle and rounding-model token gradients for {toks.size} tokens")
    tb = oracle.token_backward(h["x"][toks], ref["topk_idx"][toks], ref["topk_w"][toks], w1, w3, w2, h["wg"],
                               dout_h[toks], cfg.dtype)
    tm = token_backward_with_roundings(h["x"][toks], dout_h[toks], ref["topk_idx"][toks], ref["topk_w"][toks],
                                       w1, w3, w2, h["wg"])
    tt = torch.from_numpy(toks).cuda()
    got = {"dx": gpu_float(g["dx"][tt]), "dtopk_w": gpu_float(g["dtopk_w"][tt]),
           "dl": gpu_float(g["dlogits"][tt])[np.arange(toks.size)[:, None], ref["topk_idx"][toks]]}
    for n, v in got.items():
        e_n = norm_err(v, tb[n])
        e_o, bar, e_m, mbar = elem_errs(n, v, tb[n], tm[n], tm["scale"][n])
        _say(f"  sampled {n}: normwise {e_n:.2e}, elementwise {e_o:.2e} (oracle) {e_m:.2e} (rounding model)")
        assert e_n <= NORM_TOL and e_o <= bar and e_m <= mbar, n
    # sampled FFN columns of the weight gradients of the busiest, a middle and the least busy active expert
    counts = ref["counts"]
    active = np.nonzero(counts > 0)[0]
    order = active[np.argsort(-counts[active], kind="stable")]
    experts = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1])})
    cols = np.unique(np.linspace(0, cfg.f - 1, 4).astype(np.int64))
    perm = ref["perm"]
    for e in experts:
        sl = oracle.expert_grad_slices(h["x"], dout_h, ref["topk_w"], perm, ref["offsets"], w1[e], w3[e], w2[e],
                                       cfg.k, e, cols, cfg.dtype)
        sm = expert_slices_with_roundings(h["x"], dout_h, ref["topk_w"], perm, ref["offsets"], w1[e], w3[e], w2[e],
                                          cfg.k, e, cols)
        ct = torch.from_numpy(cols).cuda()
        got = {"dw1": gpu_float(g["dw1"][e][ct]), "dw3": gpu_float(g["dw3"][e][ct]),
               "dw2": gpu_float(g["dw2"][e][:, ct])}
        ne = {n: norm_err(got[n], sl[n]) for n in WEIGHT_GRADS}
        eo = {n: comp_err(got[n], sl[n], sm["scale"][n]) for n in WEIGHT_GRADS}
        em = {n: comp_err(got[n], sm[n], sm["scale"][n]) for n in WEIGHT_GRADS}
        _say(f"  expert {e} ({counts[e]} rows): " +
             " ".join(f"{n}={ne[n]:.2e}/{eo[n]:.2e}/{em[n]:.2e}" for n in WEIGHT_GRADS))
        for n in WEIGHT_GRADS:
            assert ne[n] <= NORM_TOL and eo[n] <= COMP_TOL and em[n] <= MODEL_TOL, n
    # gate gradients from the GPU's own dlogits (a property at any size)
    dlog = gpu_float(g["dlogits"])
    xf = oracle.decode(h["x"], cfg.dtype).astype(np.float64)
    e_b = rel_err(gpu_float(g["dbias"]), dlog.sum(axis=0))
    e_g = rel_err(gpu_float(g["dwg"]), dlog.T @ xf)
    _say(f"  dbias={e_b:.2e} dwg={e_g:.2e} (from the GPU dlogits)")
    assert e_b <= 1e-3 and e_g <= 1e-3

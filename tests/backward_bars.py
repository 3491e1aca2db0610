"""Where the backward's tolerance bars come from (test infrastructure).

The HIP backward differs from the exact (fp64) oracle in two ways:
1. bf16 roundings at fixed places: g and u stored in bf16, and the matrix-product
   operands w*h, dg and du rounded to bf16. The rounding model
   (rounding_model.backward_with_roundings) repeats exactly these in fp64.
2. fp32 instead of fp64 accumulation. Its direct effect is about 2^-24 * sqrt(K)
   relative, negligible next to the bf16 steps. Its visible effect is indirect:
   an fp32 sum that lands on the other side of a bf16 rounding midpoint from the
   exact sum flips that rounding decision. The model with flip = (rng, P_FLIP)
   takes a random fraction P_FLIP of its rounding decisions the other way. With
   K of 256 .. 16384 terms, fp32 sums are off by up to about 2^-24 * sqrt(K) *
   (a few), against a bf16 midpoint spacing of 2^-8: a flip probability of order
   1e-4. P_FLIP = 1e-3 leaves a factor of about ten.

Errors are measured normwise, ||g - r|| / ||r||, for every gradient, and
elementwise in the way that suits each kind of gradient:
* per-token results (dx, dtopk_w, the selected logits' gradients dl) with the
  forward's metric, max |g - r| / max(|r|, rms(r)): a wrong or swapped token
  row is off by about its own size, far above the rounding spread;
* per-expert sums (dw1, dw3, dw2, dwg, dbias) componentwise, max |g - r| /
  scale with scale the element's sum of |terms| (the rounding model's
  "scale"), the natural unit of a rounding error: the sums of an expert with a
  few rows are differences of larger terms, and on the rms-floor metric the
  model alone is 0.29 from the exact result there, while a swapped row of
  such a sum is off by about its scale. (For a long sum such as dx the scale
  is about sqrt(K) times a typical result, which is why dx is not measured
  that way.)

The bars are taken from these differences measured on the CPU over the test
shapes and several seeds, times a safety factor, without looking at any GPU
result:
* NORM_TOL (every gradient) covers the model against the exact oracle;
* ACT_TOL (per-token results, GPU against the oracle) covers the model
  against the oracle plus the flipped model against the model: the GPU's
  result differs from the exact one by the model's roundings and by the
  decisions fp32 takes the other way; ACT_MODEL_TOL (GPU against the model)
  covers the flipped model against the model;
* COMP_TOL and MODEL_TOL, the same for the per-expert sums, componentwise.

Run as a script to print the table (python tests/backward_bars.py).
"""
from __future__ import annotations

import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import moe_inputs  # noqa: E402
import oracle  # noqa: E402
from conftest import to_numpy  # noqa: E402
from parity import rel_err  # noqa: E402
from rounding_model import backward_with_roundings, comp_err  # noqa: E402

P_FLIP = 1e-3
SAFETY = 2.0
ACT = ("dx", "dtopk_w", "dl")
SUM = ("dw1", "dw3", "dw2", "dwg", "dbias")
MODEL = ("dw1", "dw3", "dw2", "dx", "dtopk_w", "dl")


def norm_err(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def spread(shape, seed: int) -> dict:
    """Errors of one case, keyed '<kind>:<gradient>': the rounding model against the exact
    oracle normwise ('norm'), elementwise with the rms floor ('rms') and componentwise
    ('comp'); the model with flipped rounding decisions against the model, componentwise
    ('flip') and elementwise with the rms floor ('fliprms')."""
    T, d, f, E, k, s = shape
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed, device="cpu")
    dout = to_numpy(moe_inputs.output_grad(T, d, "bf16", seed, device="cpu"), "bf16")
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    fw = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")
    ref = oracle.layer_backward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16", dout,
                                routing=fw)
    idx = np.asarray(fw["topk_idx"], np.int64)
    ref["dl"] = ref["dlogits"][np.arange(T)[:, None], idx]
    model = backward_with_roundings(h, dout, fw, k)
    flip = backward_with_roundings(h, dout, fw, k, flip=(np.random.default_rng(seed + 7919), P_FLIP))
    out = {}
    for g in ACT + SUM:
        if np.any(ref[g]):  # (top-1 gate gradients are exact zeros)
            out["norm:" + g] = norm_err(model[g], ref[g])
            out["rms:" + g] = rel_err(model[g], ref[g])
        if np.any(model[g]):
            out["fliprms:" + g] = rel_err(flip[g], model[g])
        if g in SUM:
            out["comp:" + g] = comp_err(model[g], ref[g], model["scale"][g])
            out["flip:" + g] = comp_err(flip[g], model[g], model["scale"][g])
    return out


def derive(shapes, seeds) -> dict:
    """Largest differences over the cases per kind (the rms-floor kinds split into
    'act' for dx, dtopk_w, dl and 'sum' for the per-expert sums), and the bars:
    SAFETY times them, rounded up to one significant digit."""
    worst = {}
    for shape in shapes:
        for seed in seeds:
            for key, v in spread(shape, seed).items():
                kind, g = key.split(":")
                if kind in ("rms", "fliprms"):
                    kind += "_act" if g in ACT else "_sum"
                worst[kind] = max(worst.get(kind, 0.0), v)

    def up(v):
        e = math.floor(math.log10(v))
        return round(math.ceil(v / 10 ** e - 1e-9) * 10 ** e, 12)

    bars = {"NORM_TOL": up(SAFETY * worst["norm"]),
            "ACT_TOL": up(SAFETY * (worst["rms_act"] + worst["fliprms_act"])),
            "ACT_MODEL_TOL": up(SAFETY * worst["fliprms_act"]),
            "COMP_TOL": up(SAFETY * (worst["comp"] + worst["flip"])),
            "MODEL_TOL": up(SAFETY * worst["flip"])}
    return {"worst": worst, "bars": bars}


def test_shapes():
    """The backward GPU tests' hand-picked and seeded random shapes."""
    import test_gpu_backward as tb
    return list(tb.BWD_SHAPES) + list(tb._random_bwd_shapes())


GOLDEN = os.path.join(HERE, "golden", "backward_bars.json")


if __name__ == "__main__":
    # python tests/backward_bars.py [seeds]: derive the bars and record them in tests/golden/backward_bars.json
    import json
    seeds = [int(v) for v in (sys.argv[1] if len(sys.argv) > 1 else "0,1,2,3,4").split(",")]
    shapes = test_shapes()
    res = derive(shapes, seeds)
    print({k: round(v, 5) for k, v in res["worst"].items()})
    print(res["bars"])
    with open(GOLDEN, "w") as fh:
        json.dump({"about": "backward tolerance bars derived on the CPU by tests/backward_bars.py from the rounding "
                            "model against the oracle (no GPU result involved)",
                   "seeds": seeds, "shapes": [list(x) for x in shapes], "p_flip": P_FLIP, "safety": SAFETY,
                   "worst": res["worst"], "bars": res["bars"]}, fh, indent=1)

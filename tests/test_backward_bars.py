"""Host tests of the backward's error model (tests/rounding_model.py) and of the
bars derived from it (tests/backward_bars.py, tests/golden/backward_bars.json)."""
import json
import os

import numpy as np
import pytest

import backward_bars as bb
import moe_inputs
import oracle
import test_gpu_backward as tgb
from conftest import to_numpy
from parity import rel_err
from rounding_model import (_bf16_near, _bf16_other, backward_with_roundings, comp_err,
                            expert_slices_with_roundings, token_backward_with_roundings)


def _case(T=150, d=256, f=256, E=8, k=2, s=1.0, seed=3):
    inp = moe_inputs.random_inputs(T, d, f, E, k, "bf16", s, seed, device="cpu")
    dout = to_numpy(moe_inputs.output_grad(T, d, "bf16", seed, device="cpu"), "bf16")
    h = {n: to_numpy(v, "bf16") for n, v in inp.items()}
    fw = oracle.layer_forward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16")
    return h, dout, fw, k


def test_other_neighbour_rounding():
    a = np.array([1.0 + 2.0 ** -9 + 2.0 ** -12, -3.3, 0.1, 2.0, -0.0])
    r = _bf16_near(a)
    o = _bf16_other(a, r)
    inexact = a != r
    assert np.all((o[inexact] - a[inexact]) * (r[inexact] - a[inexact]) < 0)   # the other side of a
    assert np.all(o[~inexact] == r[~inexact])                                    # exact values stay
    # one bf16 step apart
    step = np.abs(o - r)[inexact] / np.abs(r[inexact])
    assert np.all((step > 2.0 ** -9) & (step <= 2.0 ** -7))


def test_sampled_model_functions_agree_with_the_whole_model():
    h, dout, fw, k = _case()
    full = backward_with_roundings(h, dout, fw, k)
    toks = np.array([0, 17, 149])
    tm = token_backward_with_roundings(h["x"][toks], dout[toks], fw["topk_idx"][toks], fw["topk_w"][toks],
                                       h["w1"], h["w3"], h["w2"], h["wg"])
    for n in ("dx", "dtopk_w", "dl"):
        # the same arithmetic on a different BLAS blocking: at most a rare rounding taken the other way
        assert comp_err(tm[n], full[n][toks], full["scale"][n][toks]) <= 1e-2, n
        np.testing.assert_allclose(tm["scale"][n], full["scale"][n][toks], rtol=1e-6)
    cols = np.array([0, 100, 255])
    e = int(np.argmax(fw["counts"]))
    sm = expert_slices_with_roundings(h["x"], dout, fw["topk_w"], fw["perm"], fw["offsets"], h["w1"][e], h["w3"][e],
                                      h["w2"][e], k, e, cols)
    pick = {"dw1": lambda a: a[e][cols], "dw3": lambda a: a[e][cols], "dw2": lambda a: a[e][:, cols]}
    for n, take in pick.items():
        assert comp_err(sm[n], take(full[n]), take(full["scale"][n])) <= 1e-2, n
        np.testing.assert_allclose(sm["scale"][n], take(full["scale"][n]), rtol=1e-6)


def test_each_metric_catches_an_index_error():
    """Two rows swapped (a plausible indexing mistake) stand out by far against the bar of
    the metric each gradient is held to, while the model itself is well inside it: one
    expert's dw1 rows componentwise, two tokens' dx rows with the rms floor."""
    h, dout, fw, k = _case()
    ref = oracle.layer_backward(h["x"], h["wg"], h["bias"], h["w1"], h["w3"], h["w2"], k, "bf16", dout, routing=fw)
    model = backward_with_roundings(h, dout, fw, k)
    assert comp_err(model["dw1"], ref["dw1"], model["scale"]["dw1"]) <= tgb.COMP_TOL / 2
    bad = model["dw1"].copy()
    e = int(np.argmax(fw["counts"]))
    bad[e, [3, 4]] = bad[e, [4, 3]]
    assert comp_err(bad, ref["dw1"], model["scale"]["dw1"]) > 10 * tgb.COMP_TOL
    assert rel_err(model["dx"], ref["dx"]) <= tgb.ACT_TOL / 2
    bad = model["dx"].copy()
    bad[[5, 6]] = bad[[6, 5]]
    assert rel_err(bad, ref["dx"]) > 10 * tgb.ACT_TOL


def test_committed_bars_are_the_derived_ones():
    rec = json.load(open(bb.GOLDEN))
    assert rec["bars"] == {"NORM_TOL": tgb.NORM_TOL, "ACT_TOL": tgb.ACT_TOL, "ACT_MODEL_TOL": tgb.ACT_MODEL_TOL,
                           "COMP_TOL": tgb.COMP_TOL, "MODEL_TOL": tgb.MODEL_TOL}
    assert rec["shapes"] == [list(x) for x in bb.test_shapes()]
    assert rec["p_flip"] == bb.P_FLIP and rec["safety"] == bb.SAFETY


@pytest.mark.timeout(300)
def test_recorded_spread_reproduces_on_a_sample():
    """A few of the recorded cases recomputed: each spread stays within the recorded worst."""
    rec = json.load(open(bb.GOLDEN))
    for shape in bb.test_shapes()[:3]:
        for key, v in bb.spread(shape, rec["seeds"][0]).items():
            kind, g = key.split(":")
            if kind in ("rms", "fliprms"):
                kind += "_act" if g in bb.ACT else "_sum"
            assert v <= rec["worst"][kind] * 1.05 + 1e-12, (shape, key, v)

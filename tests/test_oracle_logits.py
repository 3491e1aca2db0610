"""Pins of the oracle's gate logits (fixed fp32 summation order + bias)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "logit_order_cases.json")


def _gold():
    with open(GOLD) as fh:
        return json.load(fh)


def _bf16_bits(vals):
    """uint16 patterns of values that are exactly representable in bf16."""
    f = np.asarray(vals, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def _encode(vals, dtype):
    return _bf16_bits(vals) if dtype == "bf16" else np.asarray(vals, np.float32)


def _dense(sparse, d):
    v = np.zeros(d, np.float32)
    for i, val in sparse.items():
        v[int(i)] = val
    return v


@pytest.mark.parametrize("case", _gold()["cases"], ids=lambda c: c["name"])
def test_hand_worked_order_cases(case):
    d, dt = case["d"], case["dtype"]
    x = _encode(_dense(case["x"], d)[None, :], dt)
    w = _encode(_dense(case["w"], d)[None, :], dt)
    l = oracle.gate_logits(x, w, np.array([case["bias"]], np.float32), dt)
    assert l.dtype == np.float32
    assert l[0, 0] == np.float32(case["expected"]), (l[0, 0], case["why"])
    for name, v in case.get("other", {}).items():
        assert np.float32(v) != l[0, 0], f"contract must differ from {name}"


def test_index_case():
    c = _gold()["index_case"]
    d = c["d"]
    x = _encode(np.stack([_dense(r, d) for r in c["x"]]), c["dtype"])
    wg = _encode(np.stack([_dense(r, d) for r in c["wg"]]), c["dtype"])
    l = oracle.gate_logits(x, wg, np.array(c["bias"], np.float32), c["dtype"])
    np.testing.assert_array_equal(l, np.array(c["expected"], np.float32))


@pytest.mark.parametrize("d", [1, 63, 64, 65, 200])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_when_every_partial_sum_is_representable(rng, d, dtype):
    """Dyadic inputs whose partial sums all fit in fp32: any order gives the exact
    rational dot product, so this pins the pairing x[t,i]*Wg[e,i], the full index
    range and the bias, independently of the order."""
    T, E = 3, 5
    xv = rng.integers(-16, 17, size=(T, d)) / 8.0
    wv = rng.integers(-16, 17, size=(E, d)) / 8.0
    bv = rng.integers(-64, 65, size=E) / 4.0
    l = oracle.gate_logits(_encode(xv, dtype), _encode(wv, dtype), bv.astype(np.float32), dtype)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(xv[t, i])) * Fraction(float(wv[e, i])) for i in range(d)) + Fraction(float(bv[e]))
            assert Fraction(float(l[t, e])) == exact


@pytest.mark.parametrize("d", [128, 6144, 7168, 1000])
def test_error_bound_against_exact_sum(rng, d):
    """|l - exact| <= (ceil(d/64) + 7) * 2^-24 * (sum|p| + |b|): the recursive-sum bound
    of the contract's 64 lane sums, 6 tree levels and the bias add."""
    T, E = 4, 6
    xs = rng.standard_normal((T, d)).astype(np.float32)
    ws = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    xb = ((xs.view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    wb = ((ws.view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    b = rng.standard_normal(E).astype(np.float32)
    l = oracle.gate_logits(xb, wb, b, "bf16")
    xf = oracle.decode(xb, "bf16").astype(np.float64)
    wf = oracle.decode(wb, "bf16").astype(np.float64)
    exact = xf @ wf.T + b[None, :].astype(np.float64)   # products exact, fp64 sum of <= 7168 terms
    mag = np.abs(xf) @ np.abs(wf).T + np.abs(b)[None, :]
    bound = (-(-d // 64) + 7) * 2.0**-24 * mag * 1.01 + 1e-30
    err = np.abs(l.astype(np.float64) - exact)
    assert np.all(err <= bound)
    # and it is not trivially exact: a real rounding order is being exercised
    assert np.any(err > 0)


def test_order_sensitivity_is_real(rng):
    """On N(0,1) bf16 data the contract differs bitwise from a plain sequential sum
    for a sizeable share of logits: the order really must be fixed."""
    T, E, d = 16, 16, 6144
    xb = ((rng.standard_normal((T, d)).astype(np.float32).view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    wb = (((rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32).view(np.uint32) + np.uint32(0x8000)) >> 16).astype(np.uint16)
    l = oracle.gate_logits(xb, wb, None, "bf16")
    xf, wf = oracle.decode(xb, "bf16"), oracle.decode(wb, "bf16")
    seq = np.zeros((T, E), np.float32)
    for i in range(d):
        seq += xf[:, i:i + 1] * wf[None, :, i]
    assert 0.2 < np.mean(l != seq) < 1.0


def test_token_chunking_does_not_change_bits(rng):
    T, E, d = 37, 7, 300
    xb = rng.integers(0, 2**16, size=(T, d), dtype=np.uint16) & np.uint16(0xBFFF)  # finite, |v| < 2
    wb = rng.integers(0, 2**16, size=(E, d), dtype=np.uint16) & np.uint16(0xBFFF)
    a = oracle.gate_logits(xb, wb, None, "bf16", token_chunk=5)
    b = oracle.gate_logits(xb, wb, None, "bf16", token_chunk=1000)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))

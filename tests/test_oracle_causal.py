"""Pins of the oracle's scaled, causally masked softmax.

The causal function is checked against things other than itself: the plain
oracle on inputs where the mask is written in as -inf (a different code path
of the same definition), 50-digit decimal arithmetic, an exact power-of-two
scale applied to the input instead, and the closed forms of the first rows.
"""
import decimal
import math

import numpy as np
import pytest

from row_wise_softmax_amd import workloads as W

D = decimal.Decimal


def _decimal_softmax(vals):
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        finite = [D(v) for v in vals if math.isfinite(v)]
        if not finite:
            return [0.0] * len(vals)
        m = max(finite)
        e = [(D(v) - m).exp() if math.isfinite(v) else D(0) for v in vals]
        s = sum(e)
        return [float(v / s) for v in e]


def _scores(rows, cols, seed=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, cols)) * 3.0).astype(np.float32)


@pytest.mark.parametrize("diag", [0, -3, 5, 200])
def test_equals_plain_softmax_on_premasked_input(oracle_mod, diag):
    x = _scores(37, 64)
    got = oracle_mod.softmax_causal(x, "f32", scale=1.0, diag=diag)
    masked = x.copy()
    i = np.arange(37)[:, None]
    j = np.arange(64)[None, :]
    masked[j > i + diag] = -np.inf
    want = oracle_mod.softmax(masked, "f32")
    assert np.array_equal(got, want)


def test_c2_rows_equal_the_plain_oracle_on_the_masked_workload(oracle_mod):
    # The workload generator writes the mask itself; the causal oracle takes
    # the same scores unmasked (scale 1: the generator already divided by 8).
    wl = W.WORKLOADS["c2"]
    rng = np.random.default_rng([2])
    q = rng.standard_normal((2048, 64))
    k = rng.standard_normal((2048, 64))
    raw = W.cast((q[:128] @ k.T) / 8.0, "f32")
    got = oracle_mod.softmax_causal(np.ascontiguousarray(raw), "f32", scale=1.0, diag=0)
    want = oracle_mod.softmax(wl.generate(rows=128), "f32")
    assert np.array_equal(got, want)


def test_power_of_two_scale_equals_scaled_input(oracle_mod):
    x = _scores(9, 33)
    got = oracle_mod.softmax_causal(x, "f32", scale=0.25, diag=100)
    want = oracle_mod.softmax((x * np.float32(0.25)).astype(np.float32), "f32")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_brute_force_decimal(oracle_mod, dtype):
    x = W.random_matrix(seed=31, rows=7, cols=6, dtype=dtype, sigma=4.0)
    scale = 0.125
    got = oracle_mod.softmax_causal(x, dtype, scale=scale, diag=-1)
    if dtype == "f32":
        xd = x.astype(np.float64)
    elif dtype == "f16":
        xd = x.view(np.float16).astype(np.float64)
    else:
        xd = (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    for i in range(7):
        kept = max(0, min(6, i))  # diag = -1: columns 0 .. i-1
        want = np.zeros(6)
        if kept:
            want[:kept] = _decimal_softmax([scale * v for v in xd[i, :kept]])
        assert np.allclose(got[i], want, rtol=2e-15, atol=0.0), (i, got[i], want)


def test_first_rows_closed_forms(oracle_mod):
    x = np.array([[3.0, 9.0, 9.0], [0.0, math.log(3.0), 7.0], [1.0, 1.0, 1.0]], dtype=np.float32)
    got = oracle_mod.softmax_causal(x, "f32", scale=1.0, diag=0)
    assert got[0, 0] == 1.0 and got[0, 1] == 0.0 and got[0, 2] == 0.0      # one kept entry
    assert np.allclose(got[1, :2], [0.25, 0.75], rtol=1e-7) and got[1, 2] == 0.0  # ln 3 rounded to fp32
    assert np.all(np.abs(got[2] - 1.0 / 3.0) <= np.spacing(1.0 / 3.0))     # constant row


def test_rows_without_kept_columns_are_zero(oracle_mod):
    x = _scores(6, 10)
    got = oracle_mod.softmax_causal(x, "f32", scale=1.0, diag=-4)
    assert np.all(got[:4] == 0.0) and not np.signbit(got[:4]).any()
    assert got[4, 0] == 1.0 and np.all(got[4, 1:] == 0.0)
    got = oracle_mod.softmax_causal(x, "f32", scale=1.0, diag=-(2 ** 62))
    assert np.all(got == 0.0)
    got = oracle_mod.softmax_causal(x, "f32", scale=1.0, diag=2 ** 62)
    assert np.array_equal(got, oracle_mod.softmax(x, "f32"))


def test_masked_inputs_are_never_read(oracle_mod):
    x = _scores(8, 8)
    poisoned = x.copy()
    i = np.arange(8)[:, None]
    j = np.arange(8)[None, :]
    poisoned[j > i] = np.nan
    assert np.array_equal(oracle_mod.softmax_causal(poisoned, "f32", 1.0, 0),
                          oracle_mod.softmax_causal(x, "f32", 1.0, 0))


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan")])
def test_bad_scale_rejected(oracle_mod, scale):
    with pytest.raises(ValueError):
        oracle_mod.softmax_causal(_scores(2, 3), "f32", scale=scale)

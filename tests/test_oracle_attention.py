"""Pins of the oracle's attention forward (softmax(scale Q K^T) V, causal).

Expected values come from 50-digit decimal brute force, closed forms (uniform
attention, one kept key, constant values), exact symmetries (joint key/value
permutation, exact rescaling of the queries), and the independently pinned
softmax oracle (with d = 1 and q = 1 the score row is scale * k).
"""
import decimal

import numpy as np
import pytest

from row_wise_softmax_amd import workloads as W

D = decimal.Decimal


def _decode(x, dtype):
    if dtype == "f32":
        return x.astype(np.float64)
    if dtype == "f16":
        return x.view(np.float16).astype(np.float64)
    return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _qkv(b, h, nq, nk, d, dtype, seed, sigma=1.0):
    rng = np.random.default_rng(seed)
    q = W.cast(rng.standard_normal((b, h, nq, d)) * sigma, dtype)
    k = W.cast(rng.standard_normal((b, h, nk, d)) * sigma, dtype)
    v = W.cast(rng.standard_normal((b, h, nk, d)), dtype)
    return q, k, v


def _kept(i, nq, nk, causal):
    return nk if not causal else max(0, min(nk, i + (nk - nq) + 1))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_brute_force_decimal(oracle_mod, causal, dtype):
    b, h, nq, nk, d, scale = 1, 2, 3, 4, 3, 0.7
    q, k, v = _qkv(b, h, nq, nk, d, dtype, seed=81, sigma=2.0)
    got = oracle_mod.attention_fwd(q, k, v, dtype, scale, causal)
    qd, kd, vd = (_decode(t, dtype) for t in (q, k, v))
    with decimal.localcontext() as ctx:
        ctx.prec = 50
        for hh in range(h):
            for i in range(nq):
                kept = _kept(i, nq, nk, causal)
                if kept == 0:
                    assert np.all(got[0, hh, i] == 0.0)
                    continue
                s = [D(scale) * sum(D(qd[0, hh, i, c]) * D(kd[0, hh, j, c]) for c in range(d)) for j in range(kept)]
                m = max(s)
                e = [(x - m).exp() for x in s]
                tot = sum(e)
                for c in range(d):
                    want = float(sum(e[j] / tot * D(vd[0, hh, j, c]) for j in range(kept)))
                    assert abs(got[0, hh, i, c] - want) <= 1e-14 * (1 + abs(want))


def test_constant_values_give_that_constant(oracle_mod):
    q, k, _ = _qkv(2, 3, 17, 29, 8, "f16", seed=82, sigma=3.0)
    vals = np.linspace(-2, 2, 8)
    v = W.cast(np.broadcast_to(vals, (2, 3, 29, 8)).copy(), "f16")
    got = oracle_mod.attention_fwd(q, k, v, "f16", 0.3, causal=False)
    want = _decode(v, "f16")[0, 0, 0]
    assert np.allclose(got, np.broadcast_to(want, got.shape), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("nq,nk", [(16, 16), (5, 12), (12, 5)])
def test_zero_queries_give_the_running_mean(oracle_mod, nq, nk):
    _, k, v = _qkv(1, 2, nq, nk, 8, "bf16", seed=83)
    q = np.zeros((1, 2, nq, 8), dtype=np.uint16)
    got = oracle_mod.attention_fwd(q, k, v, "bf16", 1.0, causal=True)
    vd = _decode(v, "bf16")
    csum = np.cumsum(vd, axis=2)  # library prefix sum
    for i in range(nq):
        kept = _kept(i, nq, nk, True)
        want = np.zeros(8) if kept == 0 else csum[:, :, kept - 1] / kept
        assert np.allclose(got[:, :, i], want, rtol=1e-13, atol=1e-14)


def test_first_causal_row_copies_the_first_value(oracle_mod):
    q, k, v = _qkv(2, 2, 9, 9, 16, "f16", seed=84, sigma=4.0)
    got = oracle_mod.attention_fwd(q, k, v, "f16", 0.25, causal=True)
    assert np.array_equal(got[:, :, 0], _decode(v, "f16")[:, :, 0])


def test_joint_key_value_permutation(oracle_mod):
    q, k, v = _qkv(1, 1, 7, 23, 8, "f16", seed=85)
    perm = np.random.default_rng(0).permutation(23)
    a = oracle_mod.attention_fwd(q, k, v, "f16", 0.5, causal=False)
    bb = oracle_mod.attention_fwd(q, np.ascontiguousarray(k[:, :, perm]), np.ascontiguousarray(v[:, :, perm]),
                                  "f16", 0.5, causal=False)
    assert np.allclose(a, bb, rtol=1e-13, atol=1e-15)


def test_exact_rescaling_of_queries(oracle_mod):
    q, k, v = _qkv(1, 2, 6, 6, 8, "f16", seed=86)
    q2 = W.cast(_decode(q, "f16") * 2.0, "f16")  # doubling is exact in fp16 at these magnitudes
    assert np.array_equal(_decode(q2, "f16"), 2.0 * _decode(q, "f16"))
    a = oracle_mod.attention_fwd(q, k, v, "f16", 0.5, causal=True)
    bb = oracle_mod.attention_fwd(q2, k, v, "f16", 0.25, causal=True)
    assert np.array_equal(a, bb)


@pytest.mark.parametrize("causal", [False, True])
def test_one_dimensional_heads_match_the_softmax_oracle(oracle_mod, causal):
    # d = 1, q = 1: the score of key j is scale * k_j, so P is the softmax
    # oracle's (causal) softmax of the k column, and O = P V.
    nq = nk = 11
    rng = np.random.default_rng(87)
    k = W.cast(rng.standard_normal((1, 1, nk, 1)) * 3, "f16")
    v = W.cast(rng.standard_normal((1, 1, nk, 1)), "f16")
    q = W.cast(np.ones((1, 1, nq, 1)), "f16")
    got = oracle_mod.attention_fwd(q, k, v, "f16", 0.75, causal)[0, 0, :, 0]
    krow = np.ascontiguousarray(np.broadcast_to(k[0, 0, :, 0], (nq, nk)))
    p = oracle_mod.softmax_causal(krow, "f16", 0.75, diag=0 if causal else nk)
    want = p @ _decode(v, "f16")[0, 0, :, 0]  # library matrix-vector product
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


def test_huge_scores_keep_their_logistic_weights(oracle_mod):
    """Scores of 1000 and 999 (exp overflows fp64 past 709): only the shift by
    the row max keeps them finite.  With two keys the weights are the
    logistic 1/(1+e^-1) and e^-1/(1+e^-1) (closed form), so
    O = sigma(1) v0 + (1 - sigma(1)) v1 exactly up to rounding."""
    q = W.cast(np.array([[[[1.0, 0.0]]]]), "f32")
    k = W.cast(np.array([[[[1000.0, 0.0], [999.0, 0.0]]]]), "f32")
    v = W.cast(np.array([[[[2.0, -3.0], [5.0, 7.0]]]]), "f32")
    got = oracle_mod.attention_fwd(q, k, v, "f32", 1.0, causal=False)[0, 0, 0]
    w0 = 1.0 / (1.0 + np.exp(-1.0))
    want = w0 * np.array([2.0, -3.0]) + (1.0 - w0) * np.array([5.0, 7.0])
    assert np.all(np.isfinite(got))
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def test_bad_arguments(oracle_mod):
    q, k, v = _qkv(1, 1, 2, 2, 4, "f16", seed=88)
    with pytest.raises(ValueError):
        oracle_mod.attention_fwd(q, k, v, "f16", 0.0, True)
    with pytest.raises(ValueError):
        oracle_mod.attention_fwd(q, k[:, :, :1].copy(), v, "f16", 1.0, True)

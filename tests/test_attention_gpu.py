"""GPU parity of the fused attention forward (MFMA) against the CPU oracle.

Tolerance, from the arithmetic: P is rounded to the input type before the
second product (relative error <= 2^-(m+1) per weight, and the weights sum to
one) and O is rounded on the way out (<= 2^-(m+1) |O| <= 2^-(m+1) max|V|),
with m the mantissa width (11 for fp16, 8 for bf16); the fp32 products and
sums add far less.  So |O_gpu - O_oracle| <= 2^-m max|V|; the tests allow 4x.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import decode, to_device, to_host

pytestmark = pytest.mark.gpu

MANT = {"f16": 11, "bf16": 8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _qkv(b, h, nq, nk, d, dtype, seed):
    rng = np.random.default_rng([seed, b, h, nq, nk, d])
    q = W.cast(rng.standard_normal((b, h, nq, d)), dtype)
    k = W.cast(rng.standard_normal((b, h, nk, d)), dtype)
    v = W.cast(rng.standard_normal((b, h, nk, d)), dtype)
    return q, k, v


def _run(q, k, v, dtype, scale, causal):
    import torch
    b, h, nq, d = q.shape
    nk = k.shape[2]
    qd, kd, vd = (to_device(np.ascontiguousarray(t), dtype) for t in (q, k, v))
    od = torch.full_like(qd, float("nan"))
    binding.attention_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), od.data_ptr(), b, h, nq, nk, d, scale,
                          causal, W.dtype_code(dtype), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return decode(to_host(od, dtype), dtype)


SHAPES = [(1, 1, 64, 64, 64), (2, 3, 100, 100, 64), (1, 2, 128, 256, 128), (1, 1, 77, 33, 128),
          (2, 2, 200, 200, 128), (1, 4, 1, 130, 64), (1, 1, 130, 1, 64), (1, 2, 64, 0, 64), (3, 1, 257, 300, 64),
          (2, 5, 300, 300, 64), (1, 8, 512, 512, 128), (1, 2, 640, 520, 128)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{b}x{h}x{nq}x{nk}x{d}" for b, h, nq, nk, d in SHAPES])
def test_attention_matches_the_oracle(dtype, causal, shape):
    b, h, nq, nk, d = shape
    print(f"[gpu-case] attention {dtype} causal={causal} {shape}", file=sys.stderr, flush=True)
    q, k, v = _qkv(b, h, nq, nk, d, dtype, seed=91)
    scale = 1.0 / np.sqrt(d)
    got = _run(q, k, v, dtype, scale, causal)
    want = O.attention_fwd(q, k, v, dtype, scale, causal)
    vmax = float(np.max(np.abs(decode(v, dtype)))) if v.size else 1.0
    tol = 4 * 2.0 ** -MANT[dtype] * max(vmax, 1.0)
    assert not np.isnan(got).any()
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= tol, f"max abs error {err:.3e} > {tol:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_large_scale_and_peaked_rows(dtype):
    """A large scale makes every row nearly one-hot: the online max must track it."""
    q, k, v = _qkv(1, 2, 150, 150, 64, dtype, seed=92)
    got = _run(q, k, v, dtype, 2.0, True)
    want = O.attention_fwd(q, k, v, dtype, 2.0, True)
    tol = 4 * 2.0 ** -MANT[dtype] * float(np.max(np.abs(decode(v, dtype))))
    assert float(np.max(np.abs(got - want))) <= tol


def test_attention_first_causal_row_copies_v0():
    q, k, v = _qkv(2, 2, 64, 64, 128, "f16", seed=93)
    got = _run(q, k, v, "f16", 0.125, True)
    assert np.array_equal(got[:, :, 0], decode(v, "f16")[:, :, 0])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("direction", [1.0, -1.0])
def test_attention_scores_that_ramp_across_blocks(dtype, direction):
    """Scores that grow (or shrink) steadily with the key index: the running max
    moves a little in every key block, sometimes by less than the kernel lets
    the exponent offset lag, sometimes by more, so both the kept and the
    rescaled offsets are exercised against the oracle."""
    b, h, n, d = 1, 2, 520, 64
    rng = np.random.default_rng(94)
    q = np.zeros((b, h, n, d))
    q[..., 0] = 1.0
    q[..., 1:] = 0.05 * rng.standard_normal((b, h, n, d - 1))
    k = 0.05 * rng.standard_normal((b, h, n, d))
    k[..., 0] = direction * 0.26 * np.arange(n)  # log2-domain slope ~ 3 per 64 keys at scale 1/8
    v = rng.standard_normal((b, h, n, d))
    q, k, v = (W.cast(t, dtype) for t in (q, k, v))
    for causal in (False, True):
        got = _run(q, k, v, dtype, 0.125, causal)
        want = O.attention_fwd(q, k, v, dtype, 0.125, causal)
        tol = 4 * 2.0 ** -MANT[dtype] * float(np.max(np.abs(decode(v, dtype))))
        err = float(np.max(np.abs(got - want)))
        assert err <= tol, f"causal={causal}: max abs error {err:.3e} > {tol:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_benchmarked_shape_sampled(dtype):
    """The benchmarked shape (batch 4, 32 heads, 4096 queries and keys, head
    dim 128, causal, scale 1/sqrt(128)), run whole in the benchmark's launch
    configuration; 40 sampled queries checked against the oracle.  Query i of
    a causal head keeps keys 0..i, so the oracle takes that query alone with
    those keys (one query, i + 1 keys: the same kept set)."""
    b, h, n, d = 4, 32, 4096, 128
    print(f"[gpu-case] attention full size {dtype}", file=sys.stderr, flush=True)
    rng = np.random.default_rng(95)
    q, k, v = (W.cast(rng.standard_normal((b, h, n, d), dtype=np.float32), dtype) for _ in range(3))
    scale = 1.0 / np.sqrt(d)
    got = _run(q, k, v, dtype, scale, True)
    picks = [(0, 0, 0), (0, 0, 1), (1, 5, 127), (1, 5, 128), (3, 31, n - 1), (2, 17, n - 64)]
    picks += [tuple(int(t) for t in rng.integers((0, 0, 0), (b, h, n))) for _ in range(34)]
    vmax = float(np.max(np.abs(decode(v, dtype))))
    tol = 4 * 2.0 ** -MANT[dtype] * vmax
    worst = 0.0
    for bb, hh, i in picks:
        qi = np.ascontiguousarray(q[bb:bb + 1, hh:hh + 1, i:i + 1])
        ki = np.ascontiguousarray(k[bb:bb + 1, hh:hh + 1, :i + 1])
        vi = np.ascontiguousarray(v[bb:bb + 1, hh:hh + 1, :i + 1])
        want = O.attention_fwd(qi, ki, vi, dtype, scale, True)[0, 0, 0]
        err = float(np.max(np.abs(got[bb, hh, i] - want)))
        worst = max(worst, err)
        assert err <= tol, f"query ({bb}, {hh}, {i}): max abs error {err:.3e} > {tol:.3e}"
    assert not np.isnan(got).any()


def test_attention_tensors_beyond_4gib():
    """18000 heads of 1024 queries and keys, head dim 128, fp16: each of Q, K,
    V and O is 4.7 GB, so the heads past the 4 GiB mark test the 64-bit head
    offsets.  Inputs are made on the device by seeded torch ops; 12 sampled
    (head, query) pairs, the last head included, go back to the oracle."""
    import torch
    b, h, n, d = 1, 18000, 1024, 128
    print(f"[gpu-case] attention beyond 4 GiB: {b}x{h}x{n}x{d}", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda").manual_seed(96)
    q, k, v = (torch.randn((b, h, n, d), generator=g, device="cuda", dtype=torch.float16) for _ in range(3))
    o = torch.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    binding.attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), b, h, n, n, d, scale, True,
                          W.dtype_code("f16"), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    picks = [(h - 1, n - 1), (h - 1, 0), (h - 2, 517), (h // 2, 1000), (9000, 63), (17000, 64)]
    picks += [(int(a), int(c)) for a, c in zip(np.random.default_rng(99).integers(16400, h, 6),
                                               np.random.default_rng(100).integers(0, n, 6))]
    assert (h - 1) * n * d * 2 > (1 << 32)
    tol = 4 * 2.0 ** -MANT["f16"] * float(v.abs().max().item())
    for hh, i in picks:
        qi = to_host(q[:, hh:hh + 1, i:i + 1].contiguous(), "f16")
        ki = to_host(k[:, hh:hh + 1, :i + 1].contiguous(), "f16")
        vi = to_host(v[:, hh:hh + 1, :i + 1].contiguous(), "f16")
        want = O.attention_fwd(qi, ki, vi, "f16", scale, True)[0, 0, 0]
        got = decode(to_host(o[0, hh, i].contiguous(), "f16"), "f16")
        err = float(np.max(np.abs(got - want)))
        assert err <= tol, f"head {hh}, query {i}: max abs error {err:.3e} > {tol:.3e}"
    del q, k, v, o
    torch.cuda.empty_cache()


def test_attention_longest_benchmarked_context_sampled():
    """The longest context the benchmark times (batch 4, 32 heads, 32768
    queries and keys, head dim 128, causal, fp16), run whole; 10 sampled
    queries, the last ones of a head included, against the oracle.  Inputs are
    made on the device by seeded torch ops (3 GB)."""
    import torch
    b, h, n, d = 4, 32, 32768, 128
    print(f"[gpu-case] attention longest context: {b}x{h}x{n}x{d}", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda").manual_seed(101)
    q, k, v = (torch.randn((b, h, n, d), generator=g, device="cuda", dtype=torch.float16) for _ in range(3))
    o = torch.empty_like(q)
    scale = 1.0 / np.sqrt(d)
    binding.attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), b, h, n, n, d, scale, True,
                          W.dtype_code("f16"), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    picks = [(3, 31, n - 1), (0, 0, n - 2), (2, 7, 16383), (1, 20, 30000), (0, 5, 0)]
    rng = np.random.default_rng(102)
    picks += [(int(rng.integers(b)), int(rng.integers(h)), int(rng.integers(n))) for _ in range(5)]
    tol = 4 * 2.0 ** -MANT["f16"] * float(v.abs().max().item())
    for bb, hh, i in picks:
        qi = to_host(q[bb:bb + 1, hh:hh + 1, i:i + 1].contiguous(), "f16")
        ki = to_host(k[bb:bb + 1, hh:hh + 1, :i + 1].contiguous(), "f16")
        vi = to_host(v[bb:bb + 1, hh:hh + 1, :i + 1].contiguous(), "f16")
        want = O.attention_fwd(qi, ki, vi, "f16", scale, True)[0, 0, 0]
        got = decode(to_host(o[bb, hh, i].contiguous(), "f16"), "f16")
        err = float(np.max(np.abs(got - want)))
        assert err <= tol, f"query ({bb}, {hh}, {i}): max abs error {err:.3e} > {tol:.3e}"
    del q, k, v, o
    torch.cuda.empty_cache()


def _random_case(case):
    rng = np.random.default_rng([83, case])
    d = int(rng.choice([64, 128]))
    b, h = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    nq = int(rng.integers(1, 700))
    nk = int(rng.choice([nq, int(rng.integers(0, 700))]))
    dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
    causal = bool(rng.random() < 0.5)
    scale = float(rng.uniform(0.02, 0.4))
    sigma = float(rng.uniform(0.3, 3.0))
    return b, h, nq, nk, d, dtype, causal, scale, sigma


@pytest.mark.parametrize("case", range(40))
def test_attention_random_shapes(case):
    """Seeded random batch, heads, query and key counts (equal or not, keys
    possibly none), head dim, dtype, causality, scale and input spread."""
    b, h, nq, nk, d, dtype, causal, scale, sigma = _random_case(case)
    print(f"[gpu-case] attention random #{case}: {dtype} b{b} h{h} nq{nq} nk{nk} d{d} causal={causal}",
          file=sys.stderr, flush=True)
    rng = np.random.default_rng([84, case])
    q = W.cast(sigma * rng.standard_normal((b, h, nq, d)), dtype)
    k = W.cast(sigma * rng.standard_normal((b, h, nk, d)), dtype)
    v = W.cast(rng.standard_normal((b, h, nk, d)), dtype)
    got = _run(q, k, v, dtype, scale, causal)
    want = O.attention_fwd(q, k, v, dtype, scale, causal)
    vmax = float(np.max(np.abs(decode(v, dtype)))) if v.size else 1.0
    tol = 4 * 2.0 ** -MANT[dtype] * max(vmax, 1.0)
    assert not np.isnan(got).any()
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= tol, f"max abs error {err:.3e} > {tol:.3e}"

"""GPU parity of the scaled, causally masked softmax against the CPU oracle."""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import causal_mask, check, check_padding_untouched, decode, run

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _raw_scores(rows, cols, head_dim=64, seed=2):
    """q k^T in fp32 without the 1/sqrt(d) scale or the mask (the kernel applies both)."""
    rng = np.random.default_rng([seed])
    q = rng.standard_normal((cols, head_dim))
    k = rng.standard_normal((cols, head_dim))
    return W.cast(q[:rows] @ k.T, "f32")


def test_c2_scores_scaled_and_masked_in_the_kernel():
    """The c2 workload built the other way round: raw q k^T in, scale 1/8 and
    the causal mask applied by the kernel."""
    x = _raw_scores(2048, 2048)
    _say("causal c2 2048x2048 scale 1/8")
    y = run(x, "f32", causal=True, scale=0.125, diag=0)
    keep = causal_mask(2048, 2048, 0)
    err = check(y, x, "f32", O.softmax_causal(x, "f32", 0.125, 0), label="causal c2", keep=keep)
    _say(f"causal c2 max abs err {err:.3e}")
    yd = decode(y, "f32")
    assert yd[0, 0] == 1.0 and np.all(yd[~keep] == 0.0)


def test_c2_workload_rows_match_the_plain_path():
    """Causal kernel on unmasked scores vs the plain kernel on the c2 workload
    (the same fp32 scores with the mask written in as -inf)."""
    rows = 512
    rng = np.random.default_rng([2])
    q = rng.standard_normal((2048, 64))
    k = rng.standard_normal((2048, 64))
    scores = W.cast((q[:rows] @ k.T) / 8.0, "f32")
    y_causal = decode(run(scores, "f32", causal=True, scale=1.0, diag=0), "f32")
    y_plain = decode(run(W.WORKLOADS["c2"].generate(rows=rows), "f32"), "f32")
    assert np.max(np.abs(y_causal - y_plain)) <= 4e-6


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [8, 64, 100, 512, 1000, 1024, 2048, 4096, 8192, 16384, 100000])
@pytest.mark.parametrize("diag", [0, -5, 37])
def test_widths_and_diagonals(dtype, cols, diag):
    rows = max(8, min(300, 4_000_000 // cols))
    _say(f"causal {dtype} rows={rows} cols={cols} diag={diag}")
    x = W.random_matrix(seed=41, rows=rows, cols=cols, dtype=dtype, sigma=3.0)
    y = run(x, dtype, causal=True, scale=0.5, diag=diag)
    check(y, x, dtype, O.softmax_causal(x, dtype, 0.5, diag), label=f"causal {dtype} {cols} {diag}",
          keep=causal_mask(rows, cols, diag))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_masked_inputs_are_never_read(dtype):
    """NaN in every masked position: a read of one would poison its row."""
    rows, cols = 257, 1000
    x = W.random_matrix(seed=42, rows=rows, cols=cols, dtype=dtype)
    keep = causal_mask(rows, cols, 3)
    poisoned = x.copy()
    poisoned[~keep] = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}[dtype]
    y = run(poisoned, dtype, causal=True, scale=1.0, diag=3)
    check(y, x, dtype, O.softmax_causal(x, dtype, 1.0, 3), label=f"poisoned {dtype}", keep=keep)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cols,stride", [(1000, 1024), (1000, 1003), (4096, 4104)])
def test_stride_padding_and_in_place(dtype, cols, stride):
    x = W.random_matrix(seed=43, rows=64, cols=cols, dtype=dtype, row_stride=stride)
    keep = causal_mask(64, cols, 10)
    ref = O.softmax_causal(x, dtype, 2.0, 10, cols=cols)
    y = run(x, dtype, cols=cols, causal=True, scale=2.0, diag=10)
    check(y, x, dtype, ref, cols=cols, label="causal stride", keep=keep)
    check_padding_untouched(y, cols, dtype, label="causal stride")
    if stride % (16 // (4 if dtype == "f32" else 2)) == 0:
        yi = run(x, dtype, cols=cols, causal=True, scale=2.0, diag=10, inplace=True)
        check(yi, x, dtype, ref, cols=cols, label="causal in place", keep=keep)


@pytest.mark.parametrize("diag", [-(2 ** 62), -1000, 2 ** 62])
def test_extreme_diagonals(diag):
    x = W.random_matrix(seed=44, rows=50, cols=256, dtype="f32")
    y = decode(run(x, "f32", causal=True, scale=1.0, diag=diag), "f32")
    ref = O.softmax_causal(x, "f32", 1.0, diag)
    assert np.max(np.abs(y - ref)) <= 2e-6
    if diag < 0:
        assert np.all(y == 0.0)


def test_large_scale_and_huge_values():
    x64 = np.random.default_rng(45).standard_normal((6, 300))
    x64[0, 17] = 3.0e38
    x64[2, :] = -3.0e38
    x = W.cast(x64, "f32")
    for scale in (1.0, 8.0, 1e-3):
        y = run(x, "f32", causal=True, scale=scale, diag=400)
        check(y, x, "f32", O.softmax_causal(x, "f32", scale, 400), label=f"huge scale={scale}")


# ------------------------------------------- a batch of score matrices

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,diag", [((2, 3, 100, 100), 0), ((4, 5, 40, 40), 3), ((2, 2, 300, 320), 20),
                                        ((1, 2, 64, 4096), 4032), ((3, 1, 1000, 1000), -5),
                                        ((2, 3, 37, 53), 5)])  # odd width: every row at another chunk offset
def test_batched_causal_masks_each_matrix(dtype, shape, diag):
    """softmax_fwd_causal_batched: every matrix of [b][h][n][m] scores masked on
    its own row index, against the oracle run matrix by matrix; the torch call
    on the 4-D tensor gives the same bits."""
    import torch

    from gpu_util import to_device, to_host
    b, h, n, m = shape
    _say(f"batched causal {dtype} {shape} diag={diag}")
    x = W.random_matrix(seed=61, rows=b * h * n, cols=m, dtype=dtype, sigma=2.0)
    xd = to_device(x, dtype)
    out = torch.empty_like(xd)
    binding.softmax_fwd_causal_batched(xd.data_ptr(), out.data_ptr(), b * h * n, m, m, n, 0.5, diag,
                                       W.dtype_code(dtype), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    y = to_host(out, dtype)
    ref = np.concatenate([O.softmax_causal(np.ascontiguousarray(x[k * n:(k + 1) * n]), dtype, 0.5, diag)
                          for k in range(b * h)])
    keep = np.tile(causal_mask(n, m, diag), (b * h, 1))
    check(y, x, dtype, ref, label=f"batched causal {dtype} {shape}", keep=keep)
    y4 = binding.softmax(xd.view(b, h, n, m), causal=True, scale=0.5, diag=diag)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(y4.reshape(b * h * n, m), dtype), y)


def test_batched_causal_empty_shapes():
    """Empty [..., n, m] batches (no matrix, no rows, no columns) launch nothing and return."""
    import torch
    for shape in ((2, 0, 5), (0, 3, 4, 4), (2, 3, 4, 0)):
        x = torch.empty(shape, device="cuda")
        y = binding.softmax(x, causal=True, scale=0.5)
        torch.cuda.synchronize()
        assert y.shape == x.shape

"""GPU parity of the any-alignment kernels: rows whose start is not on a
16-byte boundary (widths that are not a multiple of 16 bytes, odd row
pitches, pointers inside a chunk), moved in aligned 16-byte chunks with the
elements of the neighbouring rows masked on load and left alone on store.

Each case compares every output element with the oracle and checks that no
element outside the rows (row padding, the elements before the first row and
after the last, the neighbours' elements in shared chunks) is written.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import causal_mask, check, check_every_row, decode, sentinel, to_device, to_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _run(x, dtype, cols, offset, inplace=False, causal=False, scale=1.0, diag=0):
    """softmax_fwd (or softmax_fwd_causal) on host array x (rows x row_stride) placed
    `offset` elements into device buffers whose other elements hold a NaN
    sentinel; returns (raw output buffer, the entry name softmax_select reports)."""
    import torch
    rows, stride = x.shape
    code = W.dtype_code(dtype)
    esz = 4 if dtype == "f32" else 2
    tail = 5
    full_in = np.full(offset + rows * stride + tail, sentinel(dtype), dtype=x.dtype)
    full_in[offset:offset + rows * stride] = x.ravel()
    xd = to_device(full_in, dtype)
    out = xd if inplace else to_device(np.full_like(full_in, sentinel(dtype)), dtype)
    pi, po = xd.data_ptr() + offset * esz, out.data_ptr() + offset * esz
    stream = torch.cuda.current_stream().cuda_stream
    if causal:
        kid = binding.softmax_select(pi, po, cols, stride, code, rows=rows, causal=True)
        binding.softmax_fwd_causal(pi, po, rows, cols, stride, scale, diag, code, stream)
    else:
        kid = binding.softmax_select(pi, po, cols, stride, code, rows=rows)
        binding.softmax_fwd(pi, po, rows, cols, stride, code, stream)
    torch.cuda.synchronize()
    name = "split" if kid == binding.SPLIT_KERNEL else binding.kernel_table()[kid].name
    return to_host(out, dtype), name


def _untouched(full, x, dtype, cols, offset, label):
    """Every element of the buffer outside the rows' first `cols` columns still
    holds what it held before the call (the sentinel, or in place the input)."""
    rows, stride = x.shape
    mask = np.ones(full.size, dtype=bool)
    for r in range(rows):
        mask[offset + r * stride: offset + r * stride + cols] = False
    got = full[mask]
    if dtype == "f32":
        assert np.isnan(got).all(), f"{label}: an element outside the rows was written"
    else:
        assert (got == sentinel(dtype)).all(), f"{label}: an element outside the rows was written"


@pytest.mark.parametrize("case", range(40))
def test_any_alignment_random_calls(case):
    """Seeded random dtype, rows (1..300), width (1..70000, log-uniform), row
    padding (0..9), offset of the first row in its chunk (0..7 elements), in
    place or not, plain or causal."""
    rng = np.random.default_rng([95, case])
    dtype = ["f32", "f16", "bf16"][int(rng.integers(0, 3))]
    cols = max(1, int(round(float(np.exp(rng.uniform(0.0, np.log(70000.0)))))))
    rows = int(rng.integers(1, 301))
    stride = cols + int(rng.integers(0, 10))
    offset = int(rng.integers(0, 8))
    inplace = bool(rng.random() < 0.2)
    causal = bool(rng.random() < 0.3)
    diag = int(rng.integers(-rows, cols + 1))
    label = (f"any #{case}: {dtype} rows={rows} cols={cols} stride={stride} offset={offset} inplace={inplace} "
             f"causal={causal} diag={diag}")
    _say(label)
    x = W.random_matrix(seed=960 + case, rows=rows, cols=cols, dtype=dtype, sigma=float(rng.uniform(0.5, 4.0)),
                        row_stride=stride)
    x[0, : cols // 3] = W.neg_inf(dtype)
    full, name = _run(x, dtype, cols, offset, inplace=inplace, causal=causal, scale=0.5, diag=diag)
    esz = 4 if dtype == "f32" else 2
    misaligned = (offset * esz) % 16 != 0 or (stride * esz) % 16 != 0 or (cols * esz) % 16 != 0
    if name != "split":
        assert ("any_" in name) == misaligned, f"{label}: picked {name}"
    y = full[offset:offset + x.size].reshape(x.shape)
    if causal:
        ref = O.softmax_causal(x, dtype, 0.5, diag, cols=cols)
        check(y, x, dtype, ref, cols=cols, label=label, keep=causal_mask(rows, cols, diag))
    else:
        check(y, x, dtype, O.softmax(x, dtype, cols=cols), cols=cols, label=label)
    if not inplace:
        _untouched(full, x, dtype, cols, offset, label)


@pytest.mark.parametrize("dtype,rows,cols", [("bf16", 8192, 4097), ("f32", 8192, 4097), ("f32", 50000, 1001),
                                             ("bf16", 2048, 50257), ("f16", 4096, 32001), ("bf16", 30000, 33)])
def test_odd_widths_every_row(dtype, rows, cols):
    """Contiguous tensors of odd widths (every row at another offset in its
    first chunk), every row against the oracle."""
    _say(f"odd width {dtype} {rows}x{cols}")
    x = W.random_matrix(seed=97, rows=rows, cols=cols, dtype=dtype, sigma=2.0)
    full, name = _run(x, dtype, cols, 0)
    assert "any_" in name, name
    y = full[:x.size].reshape(x.shape)
    check_every_row(y, x, dtype, label=f"odd width {dtype} {rows}x{cols}")
    _untouched(full, x, dtype, cols, 0, "odd width")


@pytest.mark.parametrize("case", range(24))
def test_wide_16bit_rows_random_calls(case):
    """16-bit rows of 32769..200000 columns (the stored-value kernels, plain,
    causal and at any offset, and the online kernel past them): seeded random
    width, 1..12 rows, row padding 0..9, offset 0..7 elements, in place or not,
    plain or causal; every output element against the oracle, and nothing
    outside the rows written."""
    rng = np.random.default_rng([96, case])
    dtype = ["f16", "bf16"][int(rng.integers(0, 2))]
    cols = int(round(float(np.exp(rng.uniform(np.log(32769.0), np.log(200000.0))))))
    if rng.random() < 0.4:
        cols = -(-cols // 8) * 8  # a whole number of 16-byte accesses
    rows = int(rng.integers(1, 13))
    stride = cols + int(rng.choice([0, 0, 0, 3, 8, 9]))
    offset = int(rng.choice([0, 0, 1, 3, 7]))
    inplace = bool(rng.random() < 0.2)
    causal = bool(rng.random() < 0.35)
    diag = int(rng.integers(-rows, cols + 1))
    label = (f"wide 16-bit #{case}: {dtype} rows={rows} cols={cols} stride={stride} offset={offset} "
             f"inplace={inplace} causal={causal} diag={diag}")
    _say(label)
    x = W.random_matrix(seed=980 + case, rows=rows, cols=cols, dtype=dtype, sigma=float(rng.uniform(0.5, 4.0)),
                        row_stride=stride)
    x[0, : cols // 5] = W.neg_inf(dtype)
    full, name = _run(x, dtype, cols, offset, inplace=inplace, causal=causal, scale=0.5, diag=diag)
    y = full[offset:offset + x.size].reshape(x.shape)
    if causal:
        ref = O.softmax_causal(x, dtype, 0.5, diag, cols=cols)
        check(y, x, dtype, ref, cols=cols, label=f"{label} ({name})", keep=causal_mask(rows, cols, diag))
    else:
        check(y, x, dtype, O.softmax(x, dtype, cols=cols), cols=cols, label=f"{label} ({name})")
    if not inplace:
        _untouched(full, x, dtype, cols, offset, label)

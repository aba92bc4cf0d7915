"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its C ABI, and compare with the CPU oracle.

Tolerances (max |y_gpu - y_oracle| over the whole output): 2e-6 for fp32,
1e-3 for fp16, 8e-3 for bf16; fp32 row sums within 1e-5 of 1 for every row
with a finite entry; every -inf input gives exactly 0; no NaN or Inf.
"""
from __future__ import annotations

import numpy as np

from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

TOL = {"f32": 2e-6, "f16": 1e-3, "bf16": 8e-3}
ROWSUM_TOL_F32 = 1e-5


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)) if dtype == "f32" else \
        torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch_dtype(dtype))
    return t.to("cuda")


def to_host(t, dtype: str) -> np.ndarray:
    import torch
    c = t.detach().cpu().contiguous()
    return c.numpy() if dtype == "f32" else c.view(torch.int16).numpy().view(np.uint16)


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64 (numpy's fp16 decoding; bf16 = upper half of fp32)."""
    if dtype == "f32":
        return raw.astype(np.float64)
    if dtype == "f16":
        return raw.view(np.float16).astype(np.float64)
    return (raw.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def sentinel(dtype: str):
    """A NaN bit pattern used to fill output padding that must stay untouched."""
    return {"f32": np.float32(np.nan), "f16": np.uint16(0x7E01), "bf16": np.uint16(0x7FC1)}[dtype]


def run(x: np.ndarray, dtype: str, cols: int | None = None, kernel_id: int | None = None,
        inplace: bool = False, prefill_out: bool = True, causal: bool = False, scale: float = 1.0,
        diag: int = 0):
    """Run the library on host array x (shape rows x row_stride); return the raw output (host).

    causal=True calls the scaled, causally masked entry points (row i keeps
    columns j <= i + diag, kept entries multiplied by scale)."""
    import torch
    rows, stride = x.shape
    cols = stride if cols is None else cols
    xd = to_device(x, dtype)
    if inplace:
        out = xd
    elif prefill_out:
        out = to_device(np.full_like(x, sentinel(dtype)), dtype)
    else:
        out = torch.empty_like(xd)
    stream = torch.cuda.current_stream().cuda_stream
    code = W.dtype_code(dtype)
    if causal and kernel_id is None:
        binding.softmax_fwd_causal(xd.data_ptr(), out.data_ptr(), rows, cols, stride, scale, diag, code, stream)
    elif causal:
        binding.softmax_fwd_causal_kernel(kernel_id, xd.data_ptr(), out.data_ptr(), rows, cols, stride, scale,
                                          diag, code, stream)
    elif kernel_id is None:
        binding.softmax_fwd(xd.data_ptr(), out.data_ptr(), rows, cols, stride, code, stream)
    else:
        binding.softmax_fwd_kernel(kernel_id, xd.data_ptr(), out.data_ptr(), rows, cols, stride, code, stream)
    torch.cuda.synchronize()
    return to_host(out, dtype)


def causal_mask(rows: int, cols: int, diag: int) -> np.ndarray:
    """True where row i keeps column j (j <= i + diag)."""
    i = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(cols, dtype=np.int64)[None, :]
    return j - i <= diag


def check(y_raw: np.ndarray, x: np.ndarray, dtype: str, ref: np.ndarray, cols: int | None = None,
          label: str = "", keep: np.ndarray | None = None) -> float:
    """Compare the raw GPU output with the oracle's float64 result; returns max abs error.

    ``keep`` (causal calls) marks the kept columns: masked ones count as -inf
    inputs (exact 0 expected), and row sums are taken over rows that keep a
    finite entry."""
    cols = x.shape[1] if cols is None else cols
    y = decode(np.ascontiguousarray(y_raw[:, :cols]), dtype)
    xin = decode(np.ascontiguousarray(x[:, :cols]), dtype)
    if keep is not None:
        xin = np.where(keep, xin, -np.inf)
    finite_rows = np.isfinite(xin).any(axis=1)
    assert not np.isnan(y).any(), f"{label}: NaN in output"
    assert np.isfinite(y[finite_rows]).all(), f"{label}: Inf in output"
    err = float(np.max(np.abs(y - ref))) if y.size else 0.0
    assert err <= TOL[dtype], f"{label}: max abs error {err:.3e} > {TOL[dtype]:.1e}"
    neg_inf = np.isneginf(xin)
    assert np.all(y[neg_inf] == 0.0), f"{label}: -inf input did not give exactly 0"
    if dtype == "f32" and finite_rows.any():
        sums = y[finite_rows].sum(axis=1)
        dev = float(np.max(np.abs(sums - 1.0)))
        assert dev <= ROWSUM_TOL_F32, f"{label}: fp32 row sum off by {dev:.3e}"
    return err


def check_padding_untouched(y_raw: np.ndarray, cols: int, dtype: str, label: str = "") -> None:
    pad = y_raw[:, cols:]
    if pad.size:
        want = sentinel(dtype)
        if dtype == "f32":
            same = pad.view(np.uint32) == np.float32(want).view(np.uint32)
        else:
            same = pad == want
        assert same.all(), f"{label}: output padding between cols and row_stride was written"


def check_every_row(y_raw: np.ndarray, x: np.ndarray, dtype: str, label: str = "",
                    chunk_elems: int = 1 << 21, threads: int = 16) -> float:
    """Element-by-element comparison of a large GPU output with the oracle, over every row.

    The rows are cut into chunks of about ``chunk_elems`` elements; each
    chunk is run through the oracle and compared with ``check`` on a pool of
    host threads (the oracle's C call and numpy's large-array loops release
    the interpreter lock).  Returns the largest absolute error."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O

    rows, cols = x.shape
    step = max(1, chunk_elems // max(cols, 1))
    starts = list(range(0, rows, step))

    def one(r0: int) -> float:
        r1 = min(rows, r0 + step)
        xs = x[r0:r1]
        return check(y_raw[r0:r1], xs, dtype, O.softmax(xs, dtype), label=f"{label} rows {r0}..{r1 - 1}")

    with ThreadPoolExecutor(max_workers=threads) as ex:
        errs = list(ex.map(one, starts))
    return max(errs) if errs else 0.0

"""The widest row the library takes: 2^30 columns (its width limit), one row.

A row this wide is 2-4 GiB, and the oracle's float64 output of it would not
fit the host many times over, so these cases check what holds at any size,
on the device (torch here is only the test's calculator):
  * every output is finite and >= 0, and each -inf input gives exactly 0;
  * the outputs sum to 1 (fp32: within 1e-5; bf16: within its unit
    roundoff u = 2^-8 -- 8 significant bits, round to nearest -- plus 1e-5);
  * for 4096 seeded pairs of finite entries the ratio of outputs equals
    exp(x_i - x_j) of the stored inputs, which pins the exponent of every
    sampled entry without the row's sum (fp32: relative 1e-5; bf16: two
    roundings, (1 + u) / (1 - u) - 1 = 7.84e-3, plus 1e-5).
The paths: softmax_fwd out of place (bf16: the split through the output,
131072 tiles merged by the merge kernel), softmax_fwd in place (fp32: one
workgroup streams the whole row twice) and softmax_fwd_split with a
workspace (fp32: the merge kernel on the workspace).
"""
import sys

import numpy as np
import pytest

from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu

COLS = 1 << 30


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _row(dtype, seed):
    """One seeded N(0, 2^2) row of COLS entries on the device, with -inf in
    columns 1000..4999 and in the first 2^16 columns (whole 16 KiB tiles)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((1, COLS), generator=g, device="cuda", dtype=torch.float32).mul_(2.0)
    x[0, 1000:5000] = float("-inf")
    x[0, : 1 << 16] = float("-inf")
    return x if dtype == "f32" else x.to(torch.bfloat16)


def _check_properties(x, y, dtype, label):
    import torch
    u = 2.0 ** -8  # bf16 unit roundoff
    sum_tol = 1e-5 if dtype == "f32" else u + 1e-5
    ratio_tol = 1e-5 if dtype == "f32" else (1 + u) / (1 - u) - 1 + 1e-5
    total = torch.zeros((), dtype=torch.float64, device="cuda")
    step = 1 << 26
    for a in range(0, COLS, step):
        yc = y[0, a:a + step].double()
        xc = x[0, a:a + step]
        assert not torch.isnan(yc).any(), f"{label}: NaN in columns {a}.."
        assert torch.isfinite(yc).all() and (yc >= 0).all(), f"{label}: negative or infinite output near {a}"
        masked = torch.isneginf(xc)
        assert (yc[masked] == 0).all(), f"{label}: a -inf input did not give exactly 0 near {a}"
        total += yc.sum()
    dev = abs(float(total) - 1.0)
    assert dev <= sum_tol, f"{label}: outputs sum to 1 + {dev:.3e}"
    rng = np.random.default_rng(92)
    idx = torch.from_numpy(rng.integers(1 << 16, COLS, size=(2, 4096))).to("cuda")
    xi, xj = x[0, idx[0]].double(), x[0, idx[1]].double()
    yi, yj = y[0, idx[0]].double(), y[0, idx[1]].double()
    keep = torch.isfinite(xi) & torch.isfinite(xj) & (yi > 1e-30) & (yj > 1e-30)
    assert int(keep.sum()) > 3000, f"{label}: too few usable pairs"
    rel = ((yi / yj)[keep] / torch.exp(xi - xj)[keep] - 1.0).abs().max().item()
    assert rel <= ratio_tol, f"{label}: y_i / y_j off exp(x_i - x_j) by {rel:.3e} (relative)"
    _say(f"{label}: sum - 1 = {float(total) - 1.0:.3e}, ratio error {rel:.3e}")


def test_widest_row_bf16_out_of_place():
    import torch
    _say("max width: bf16 1 x 2^30, softmax_fwd out of place")
    x = _row("bf16", 90)
    y = torch.empty_like(x)
    code = W.dtype_code("bf16")
    assert binding.softmax_select(x.data_ptr(), y.data_ptr(), COLS, COLS, code, rows=1) == binding.SPLIT_KERNEL
    binding.softmax_fwd(x.data_ptr(), y.data_ptr(), 1, COLS, COLS, code, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _check_properties(x, y, "bf16", "bf16 max width, split through the output")


def test_widest_row_fp32_in_place():
    import torch
    _say("max width: fp32 1 x 2^30, softmax_fwd in place")
    x = _row("f32", 91)
    x_in = x.clone()
    code = W.dtype_code("f32")
    assert binding.softmax_select(x.data_ptr(), x.data_ptr(), COLS, COLS, code, rows=1) != binding.SPLIT_KERNEL
    binding.softmax_fwd(x.data_ptr(), x.data_ptr(), 1, COLS, COLS, code, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _check_properties(x_in, x, "f32", "fp32 max width, in place")


def test_widest_row_fp32_split_with_workspace():
    import torch
    _say("max width: fp32 1 x 2^30, softmax_fwd_split with a workspace")
    x = _row("f32", 93)
    y = torch.empty_like(x)
    code = W.dtype_code("f32")
    nbytes = binding.split_workspace_bytes(1, COLS, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    binding.softmax_fwd_split(x.data_ptr(), y.data_ptr(), 1, COLS, COLS, code, ws.data_ptr(), nbytes, 1,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    _check_properties(x, y, "f32", "fp32 max width, split with a workspace")

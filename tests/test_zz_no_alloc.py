"""GPU: softmax_fwd_split_noalloc (the split path on the library's static
scratch, for callers that cannot allocate) against softmax_fwd_split with a
caller workspace, through the C ABI, on two calls in a row (the second
smaller), plus the oracle at the stated tolerances."""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import check, to_device, to_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def _pair(x, dtype, cols, stride):
    """Run the workspace entry point and the no-alloc one on the same input; return both raw outputs."""
    import torch
    rows = x.shape[0]
    code = W.dtype_code(dtype)
    xd = to_device(x, dtype)
    ref_out = torch.empty_like(xd)
    out = torch.empty_like(xd)
    nbytes = binding.split_workspace_bytes(rows, cols, code)
    assert 0 < nbytes <= binding.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    binding.softmax_fwd_split(xd.data_ptr(), ref_out.data_ptr(), rows, cols, stride, code, ws.data_ptr(), nbytes,
                              1, stream)
    binding.softmax_fwd_split_noalloc(xd.data_ptr(), out.data_ptr(), rows, cols, stride, code, 1, stream)
    torch.cuda.synchronize()
    return to_host(ref_out, dtype), to_host(out, dtype)


# (dtype, rows, cols, row_stride): the first call is the larger; the second,
# smaller one reuses scratch the first left behind.  The last pair takes the
# scalar path (ragged pitch).
CASES = [
    [("f32", 8, 1 << 20, 1 << 20), ("bf16", 3, 300_000, 300_000)],
    [("bf16", 32, 1 << 18, 1 << 18), ("f32", 2, 70_001, 70_003)],
]


@pytest.mark.parametrize("calls", CASES, ids=["f32-then-bf16", "bf16-then-scalar-f32"])
def test_noalloc_matches_workspace_entry(calls):
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    for dtype, rows, cols, stride in calls:
        _say(f"noalloc split {dtype} {rows}x{cols} stride {stride}")
        x = W.random_matrix(seed=41, rows=rows, cols=cols, dtype=dtype, sigma=2.0, row_stride=stride)
        want, got = _pair(x, dtype, cols, stride)
        assert np.array_equal(want[:, :cols], got[:, :cols]), f"{dtype} {rows}x{cols}: differs from the workspace call"
        check(got, x, dtype, O.softmax(x, dtype, cols=cols), cols=cols, label=f"noalloc {dtype} {rows}x{cols}")


def test_noalloc_rejects_beyond_the_scratch_limit():
    import torch
    code = W.dtype_code("f32")
    rows, cols = 512, 1 << 20  # 512 rows x 512 scalar tiles x 8 B = 2 MiB of pairs
    assert binding.split_workspace_bytes(rows, cols, code) > binding.NOALLOC_SCRATCH_BYTES
    x = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.SoftmaxError) as e:
        binding.softmax_fwd_split_noalloc(x.data_ptr(), x.data_ptr(), rows, cols, cols, code, 1,
                                          torch.cuda.current_stream().cuda_stream)
    assert e.value.status == 8

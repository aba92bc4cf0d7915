"""The library keeps no state between calls: several host threads calling it
at once, each on its own default-priority stream and buffers, and one thread
interleaving calls on two streams, must each get the oracle's results.  (The
only shared state is the per-device cache of resident-workgroup counts, an
array of atomics.)"""
import sys
import threading

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import causal_mask, check, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


# (dtype, rows, cols): shapes the dispatch sends to the packed, row, online and line-shifted row kernels
_JOBS = [("f32", 300, 96), ("bf16", 120, 4096), ("f16", 8, 70000), ("f32", 64, 3000)]


def test_threads_on_their_own_streams():
    import torch
    print("[gpu-case] concurrency: 4 host threads x 25 calls", file=sys.stderr, flush=True)
    inputs = [W.random_matrix(seed=140 + i, rows=r, cols=c, dtype=d, sigma=3.0) for i, (d, r, c) in enumerate(_JOBS)]
    wants = [O.softmax(x, d) for x, (d, _, _) in zip(inputs, _JOBS)]
    results, errors = [None] * len(_JOBS), []

    def worker(i):
        try:
            dtype, rows, cols = _JOBS[i]
            stream = torch.cuda.Stream()  # default priority
            with torch.cuda.stream(stream):
                xd = to_device(inputs[i], dtype)
                outs = [torch.empty_like(xd) for _ in range(25)]
            stream.synchronize()
            for out in outs:
                binding.softmax_fwd(xd.data_ptr(), out.data_ptr(), rows, cols, cols, W.dtype_code(dtype),
                                    stream.cuda_stream)
            stream.synchronize()
            results[i] = [to_host(o, dtype) for o in outs]
        except Exception as e:  # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(_JOBS))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, (dtype, _, _) in enumerate(_JOBS):
        first = results[i][0]
        check(first, inputs[i], dtype, wants[i], label=f"thread {i}")
        for y in results[i][1:]:
            assert np.array_equal(y.view(np.uint32 if dtype == "f32" else np.uint16),
                                  first.view(np.uint32 if dtype == "f32" else np.uint16)), f"thread {i}: calls differ"


def test_interleaved_streams_one_thread():
    import torch
    print("[gpu-case] concurrency: two streams interleaved", file=sys.stderr, flush=True)
    a = W.random_matrix(seed=150, rows=2048, cols=2048, dtype="f32", sigma=3.0)
    b = W.random_matrix(seed=151, rows=4096, cols=1000, dtype="bf16", sigma=3.0)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ad, bd = to_device(a, "f32"), to_device(b, "bf16")
    ya, yb = torch.empty_like(ad), torch.empty_like(bd)
    torch.cuda.synchronize()
    for _ in range(10):
        binding.softmax_fwd(ad.data_ptr(), ya.data_ptr(), 2048, 2048, 2048, W.dtype_code("f32"), s1.cuda_stream)
        binding.softmax_fwd_causal(bd.data_ptr(), yb.data_ptr(), 4096, 1000, 1000, 0.5, 0, W.dtype_code("bf16"),
                                   s2.cuda_stream)
    torch.cuda.synchronize()
    check(to_host(ya, "f32"), a, "f32", O.softmax(a, "f32"), label="stream 1")
    check(to_host(yb, "bf16"), b, "bf16", O.softmax_causal(b, "bf16", 0.5, 0), label="stream 2",
          keep=causal_mask(4096, 1000, 0))

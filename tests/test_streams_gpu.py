"""Concurrent calls: the library keeps no state between calls (apart from the
no-workspace split entry point's static array, which is documented to race),
so calls from several host threads on several streams at once must give the
bits each call gives alone.

Four host threads, each with its own stream (default priority) and its own
tensors, run softmax_fwd on a many-row shape (table kernel), softmax_fwd on
few, very wide rows (the split through the output), softmax_fwd_causal and
softmax_fwd_causal_batched, ten times each, interleaved; every result must equal
the same call made alone beforehand.  The ctypes calls release the
interpreter lock, so the threads' launches do overlap on the host.
"""
import sys
import threading

import pytest

from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _calls(t, stream):
    """The four calls of one thread, on its tensors `t`, enqueued on `stream`."""
    f16, bf16, f32 = W.dtype_code("f16"), W.dtype_code("bf16"), W.dtype_code("f32")
    binding.softmax_fwd(t["x"].data_ptr(), t["y"].data_ptr(), 2048, 4096, 4096, f16, stream)
    binding.softmax_fwd(t["w"].data_ptr(), t["yw"].data_ptr(), 8, 1 << 18, 1 << 18, bf16, stream)
    binding.softmax_fwd_causal(t["s"].data_ptr(), t["ys"].data_ptr(), 512, 512, 512, 0.25, 0, f32, stream)
    binding.softmax_fwd_causal_batched(t["b"].data_ptr(), t["yb"].data_ptr(), 4 * 128, 128, 128, 128, 0.5, 3, f32,
                                       stream)


def _tensors(seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    t = {"x": torch.randn((2048, 4096), generator=g, device="cuda").mul_(3).half(),
         "w": torch.randn((8, 1 << 18), generator=g, device="cuda").mul_(2).bfloat16(),
         "s": torch.randn((512, 512), generator=g, device="cuda"),
         "b": torch.randn((4 * 128, 128), generator=g, device="cuda")}
    for k, o in (("x", "y"), ("w", "yw"), ("s", "ys"), ("b", "yb")):
        t[o] = torch.empty_like(t[k])
    return t


OUTS = ("y", "yw", "ys", "yb")


def _bits(v):
    import torch
    return v.view(torch.int16 if v.element_size() == 2 else torch.int32)


def test_concurrent_streams_and_threads_match_calls_alone():
    import torch
    print("[gpu-case] four host threads on four streams", file=sys.stderr, flush=True)
    sets = [_tensors(300 + i) for i in range(4)]
    alone = []
    for t in sets:  # each thread's calls, alone, on the current stream
        _calls(t, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        alone.append({k: t[k].clone() for k in OUTS})
        for k in OUTS:
            t[k].fill_(float("nan"))
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in sets]
    errors = []
    barrier = threading.Barrier(len(sets))

    def worker(i):
        try:
            barrier.wait()
            with torch.cuda.stream(streams[i]):
                for _ in range(10):
                    _calls(sets[i], streams[i].cuda_stream)
            streams[i].synchronize()
        except Exception as e:  # reported after the join
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(sets))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, t in enumerate(sets):
        for k in OUTS:
            assert torch.equal(_bits(t[k]), _bits(alone[i][k])), f"thread {i}: {k} differs from the call alone"

"""The entry points inside a captured HIP graph.

They allocate nothing, never synchronise and issue no memset, so a caller may
record them in a graph.  One graph here holds a plain softmax, a scaled causal
softmax, the same over a batch of score matrices, a split-row softmax (caller
workspace), softmax_fwd's own split of few, very wide rows (two kernels, the
partials kept in the output), a vocabulary-width 16-bit softmax (the row kept
in registers as stored) and an attention forward.  It
is replayed three times on fresh inputs written between replays by ordinary
eager work, and after every replay each output must equal, bit for bit, the
same call made eagerly on the same inputs (every kernel here is
deterministic); the first replay is also checked against the oracle.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import TOL, check, decode, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _calls(bufs, stream):
    """The library calls, from the buffers in `bufs`, on `stream`."""
    r, c = bufs["shape"]
    f16 = W.dtype_code("f16")
    binding.softmax_fwd(bufs["x"].data_ptr(), bufs["y"].data_ptr(), r, c, c, f16, stream)
    binding.softmax_fwd_causal(bufs["s"].data_ptr(), bufs["ys"].data_ptr(), 256, 256, 256, 0.125, 0,
                               W.dtype_code("f32"), stream)
    binding.softmax_fwd_causal_batched(bufs["sb"].data_ptr(), bufs["ysb"].data_ptr(), 6 * 64, 64, 64, 64, 0.5, 2,
                                       W.dtype_code("f32"), stream)
    vr, vc = bufs["vshape"]
    binding.softmax_fwd(bufs["wide"].data_ptr(), bufs["ywide"].data_ptr(), vr, vc, vc, W.dtype_code("bf16"), stream)
    binding.softmax_fwd(bufs["voc"].data_ptr(), bufs["yvoc"].data_ptr(), 64, 50304, 50304, W.dtype_code("bf16"), stream)
    wr, wc = bufs["wshape"]
    binding.softmax_fwd_split(bufs["w"].data_ptr(), bufs["yw"].data_ptr(), wr, wc, wc, W.dtype_code("f32"),
                              bufs["ws"].data_ptr(), bufs["ws"].numel(), 1, stream)
    b, h, n, d = bufs["ashape"]
    binding.attention_fwd(bufs["q"].data_ptr(), bufs["k"].data_ptr(), bufs["v"].data_ptr(), bufs["o"].data_ptr(),
                          b, h, n, n, d, 1.0 / np.sqrt(d), True, f16, stream)


def _inputs(seed):
    rng = np.random.default_rng(seed)
    return {
        "x": W.cast(3.0 * rng.standard_normal((300, 4096)), "f16"),
        "s": W.cast(rng.standard_normal((256, 256)), "f32"),
        "sb": W.cast(rng.standard_normal((6 * 64, 64)), "f32"),
        "wide": W.cast(2.0 * rng.standard_normal((8, 1 << 18)), "bf16"),
        "voc": W.cast(2.0 * rng.standard_normal((64, 50304)), "bf16"),
        "w": W.cast(2.0 * rng.standard_normal((3, 70000)), "f32"),
        "q": W.cast(rng.standard_normal((1, 4, 200, 128)), "f16"),
        "k": W.cast(rng.standard_normal((1, 4, 200, 128)), "f16"),
        "v": W.cast(rng.standard_normal((1, 4, 200, 128)), "f16"),
    }


def _upload(dst, host):
    """Write host data into existing device tensors (eager copies, outside any graph)."""
    import torch
    for key, arr in host.items():
        src = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16 if arr.dtype == np.uint16 else np.float32))
        dst[key].view(src.dtype).copy_(src.view(dst[key].shape))


def test_captured_graph_replays_match_eager_calls():
    import torch
    host = _inputs(101)
    dev = {key: torch.empty(arr.shape, dtype=torch.float16 if arr.dtype == np.uint16 else torch.float32,
                            device="cuda") for key, arr in host.items()}
    dev["wide"] = torch.empty(host["wide"].shape, dtype=torch.bfloat16, device="cuda")
    dev["voc"] = torch.empty(host["voc"].shape, dtype=torch.bfloat16, device="cuda")
    bufs = dict(dev, shape=(300, 4096), wshape=(3, 70000), vshape=(8, 1 << 18), ashape=(1, 4, 200, 128))
    bufs["y"] = torch.empty_like(dev["x"])
    bufs["ys"] = torch.empty_like(dev["s"])
    bufs["ysb"] = torch.empty_like(dev["sb"])
    bufs["ywide"] = torch.empty_like(dev["wide"])
    bufs["yvoc"] = torch.empty_like(dev["voc"])
    kid = binding.softmax_select(dev["voc"].data_ptr(), bufs["yvoc"].data_ptr(), 50304, 50304, W.dtype_code("bf16"),
                                 rows=64)
    assert binding.kernel_table()[kid].name.startswith("row16_")  # 16-bit row kept as stored
    assert binding.softmax_select(dev["wide"].data_ptr(), bufs["ywide"].data_ptr(), 1 << 18, 1 << 18,
                                  W.dtype_code("bf16"), rows=8) == binding.SPLIT_KERNEL
    bufs["yw"] = torch.empty_like(dev["w"])
    bufs["o"] = torch.empty_like(dev["q"])
    nbytes = binding.split_workspace_bytes(3, 70000, W.dtype_code("f32"))
    bufs["ws"] = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    outs = ("y", "ys", "ysb", "ywide", "yvoc", "yw", "o")

    _upload(dev, host)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream, as torch asks before a capture
        _calls(bufs, side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    print("[gpu-case] graph capture of softmax, causal, batched causal, split and attention", file=sys.stderr,
          flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _calls(bufs, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()

    eager = {key: torch.empty_like(bufs[key]) for key in outs}
    for rep in range(3):
        host = _inputs(200 + rep)
        _upload(dev, host)
        for key in outs:
            bufs[key].fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"[gpu-case] graph replay {rep}", file=sys.stderr, flush=True)
        graph.replay()
        torch.cuda.synchronize()
        got = {key: bufs[key].clone() for key in outs}
        # the same calls made eagerly into the same buffers
        for key in outs:
            bufs[key].fill_(float("nan"))
        _calls(bufs, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for key in outs:
            eager[key].copy_(bufs[key])
            a, b = got[key].view(torch.int16 if got[key].element_size() == 2 else torch.int32), \
                eager[key].view(torch.int16 if got[key].element_size() == 2 else torch.int32)
            assert torch.equal(a, b), f"replay {rep}: {key} differs from the eager call"
        if rep == 0:
            y = to_host(got["y"], "f16")
            check(y, host["x"], "f16", O.softmax(host["x"], "f16"), label="graph softmax")
            ys = to_host(got["ys"], "f32")
            keep = np.arange(256)[None, :] <= np.arange(256)[:, None]
            check(ys, host["s"], "f32", O.softmax_causal(host["s"], "f32", 0.125, 0), label="graph causal", keep=keep)
            ysb = to_host(got["ysb"], "f32")
            ref = np.concatenate([O.softmax_causal(np.ascontiguousarray(host["sb"][k * 64:(k + 1) * 64]), "f32", 0.5, 2)
                                  for k in range(6)])
            keep = np.tile(np.arange(64)[None, :] <= np.arange(64)[:, None] + 2, (6, 1))
            check(ysb, host["sb"], "f32", ref, label="graph batched causal", keep=keep)
            ywide = to_host(got["ywide"], "bf16")
            check(ywide, host["wide"], "bf16", O.softmax(host["wide"], "bf16"), label="graph fwd split")
            yvoc = to_host(got["yvoc"], "bf16")
            check(yvoc, host["voc"], "bf16", O.softmax(host["voc"], "bf16"), label="graph stored-value row")
            yw = to_host(got["yw"], "f32")
            check(yw, host["w"], "f32", O.softmax(host["w"], "f32"), label="graph split")
            o = decode(to_host(got["o"], "f16"), "f16")
            want = O.attention_fwd(host["q"], host["k"], host["v"], "f16", 1.0 / np.sqrt(128), True)
            tol = 4 * 2.0 ** -11 * float(np.max(np.abs(decode(host["v"], "f16"))))
            assert float(np.max(np.abs(o - want))) <= tol
    graph.reset()

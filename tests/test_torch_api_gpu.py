"""The torch-level convenience call ``row_wise_softmax_amd.softmax(x, out=None, ...)``:
argument marshalling over the C ABI (rows over all leading dimensions, row
stride from the tensor, torch's current stream), checked against the oracle,
and its argument errors."""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import causal_mask, check, decode, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_two_dimensional(dtype):
    _say(f"torch api 2-D {dtype}")
    x = W.random_matrix(seed=111, rows=77, cols=1536, dtype=dtype, sigma=3.0)
    y = binding.softmax(to_device(x, dtype))
    check(to_host(y, dtype), x, dtype, O.softmax(x, dtype), label=f"torch api {dtype}")


def test_one_dimensional_and_rank_three():
    import torch
    _say("torch api 1-D and 3-D")
    v = W.random_matrix(seed=112, rows=1, cols=3000, dtype="f32", sigma=2.0)
    y1 = binding.softmax(torch.from_numpy(v[0].copy()).cuda())
    check(y1.cpu().numpy()[None, :], v, "f32", O.softmax(v, "f32"), label="1-D")
    x = W.random_matrix(seed=113, rows=6 * 7, cols=256, dtype="bf16", sigma=2.0)
    x3 = to_device(x, "bf16").view(6, 7, 256)
    y3 = binding.softmax(x3)
    assert y3.shape == (6, 7, 256)
    check(to_host(y3.view(42, 256), "bf16"), x, "bf16", O.softmax(x, "bf16"), label="3-D")


def test_strided_rows_view_and_in_place():
    _say("torch api strided view, in place")
    wide = W.random_matrix(seed=114, rows=40, cols=1024, dtype="f16", sigma=3.0)
    xd = to_device(wide, "f16")
    view = xd[:, :1000]  # row stride 1024, 1000 columns
    y = binding.softmax(view)
    check(to_host(y, "f16"), np.ascontiguousarray(wide[:, :1000]), "f16",
          O.softmax(np.ascontiguousarray(wide[:, :1000]), "f16"), label="strided view")
    same = binding.softmax(view, out=view)  # in place: columns 1000.. untouched
    assert same.data_ptr() == view.data_ptr()
    back = to_host(xd, "f16")
    check(np.ascontiguousarray(back[:, :1000]), np.ascontiguousarray(wide[:, :1000]), "f16",
          O.softmax(np.ascontiguousarray(wide[:, :1000]), "f16"), label="in place")
    assert np.array_equal(back[:, 1000:], wide[:, 1000:])


def test_causal_through_the_torch_call():
    _say("torch api causal")
    x = W.random_matrix(seed=115, rows=300, cols=300, dtype="f32", sigma=1.0)
    y = binding.softmax(to_device(x, "f32"), causal=True, scale=0.125, diag=2)
    check(to_host(y, "f32"), x, "f32", O.softmax_causal(x, "f32", 0.125, 2), label="causal",
          keep=causal_mask(300, 300, 2))


def test_argument_errors():
    import torch
    with pytest.raises(ValueError):
        binding.softmax(torch.zeros(4, 8))  # host tensor
    with pytest.raises(TypeError):
        binding.softmax(torch.zeros(4, 8, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError):
        binding.softmax(torch.zeros(8, 4, device="cuda").t())  # last dimension not contiguous
    with pytest.raises(ValueError):
        binding.softmax(torch.zeros(4, 8, device="cuda"), out=torch.zeros(4, 9, device="cuda"))
    with pytest.raises(ValueError):
        binding.softmax(torch.zeros(2, 4, 8, device="cuda").transpose(0, 1))  # rank 3, not contiguous


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_through_the_torch_call(dtype):
    _say(f"torch api attention {dtype}")
    rng = np.random.default_rng(116)
    q, k, v = (W.cast(rng.standard_normal((2, 3, n, 64)), dtype) for n in (150, 170, 170))
    qd, kd, vd = (to_device(t, dtype) for t in (q, k, v))
    got = binding.attention(qd, kd, vd, causal=True)  # scale defaults to 1/sqrt(64)
    want = O.attention_fwd(q, k, v, dtype, 0.125, True)
    tol = 4 * 2.0 ** -(11 if dtype == "f16" else 8) * float(np.max(np.abs(decode(v, dtype))))
    assert float(np.max(np.abs(decode(to_host(got, dtype), dtype) - want))) <= tol
    out = qd.clone()
    same = binding.attention(qd, kd, vd, scale=0.125, causal=True, out=out)
    assert same.data_ptr() == out.data_ptr()
    assert np.array_equal(to_host(out, dtype), to_host(got, dtype))


def test_attention_argument_errors():
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        binding.attention(q[0], q[0], q[0])  # rank 3
    with pytest.raises(ValueError):
        binding.attention(q, q[:, :, :8], q)  # k and v shapes differ
    with pytest.raises(ValueError):
        binding.attention(q, q, q, out=torch.zeros(1, 2, 16, 64, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        binding.attention(q, q, q.transpose(2, 3).contiguous().transpose(2, 3))  # v not contiguous

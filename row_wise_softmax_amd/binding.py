"""ctypes binding of the HIP row-softmax library (argument marshalling only).

Every step of the softmax runs in the library's HIP kernels; this module only
turns torch tensors into pointers, sizes and the current stream, and maps
status codes to exceptions.  There is no CPU or PyTorch fallback: if the
library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "librow_wise_softmax.so"


def library_path() -> str:
    return os.path.join(_HERE, "lib", LIB_NAME)


# dtype codes of the C ABI
F32, F16, BF16 = 0, 1, 2
# kernel variants of the C ABI
VARIANT_NAMES = {0: "packed", 1: "row", 2: "online", 3: "row_pf", 4: "row16"}

_lib = None


class SoftmaxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _status_string(status) if _lib is not None else f"status {status}"
        super().__init__(f"{where}: {msg} (status {status})")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    # torch ships its own HIP runtime under the same soname as ROCm's.  Load
    # it first so this library binds to that one runtime: loaded the other way
    # round, a process holds two HIP runtimes and torch's streams are invalid
    # handles to ours.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(
            f"row_wise_softmax_amd: HIP library not built ({path} missing); "
            "run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.softmax_fwd.restype = i32
    lib.softmax_fwd.argtypes = [vp, vp, i64, i64, i64, i32, vp]
    lib.softmax_fwd_kernel.restype = i32
    lib.softmax_fwd_kernel.argtypes = [i32, vp, vp, i64, i64, i64, i32, vp]
    lib.softmax_fwd_causal.restype = i32
    lib.softmax_fwd_causal.argtypes = [vp, vp, i64, i64, i64, ctypes.c_float, i64, i32, vp]
    lib.softmax_fwd_causal_batched.restype = i32
    lib.softmax_fwd_causal_batched.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_float, i64, i32, vp]
    lib.softmax_fwd_causal_kernel.restype = i32
    lib.softmax_fwd_causal_kernel.argtypes = [i32, vp, vp, i64, i64, i64, ctypes.c_float, i64, i32, vp]
    lib.softmax_fwd_variant.restype = i32
    lib.softmax_fwd_variant.argtypes = [vp, vp, i64, i64, i64, i32, i32, i32, vp]
    lib.softmax_select_variant.restype = i32
    lib.softmax_select_variant.argtypes = [i64, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.softmax_select_causal.restype = i32
    lib.softmax_select_causal.argtypes = [vp, vp, i64, i64, i64, i32, ctypes.POINTER(i32)]
    lib.softmax_select.restype = i32
    lib.softmax_select.argtypes = [vp, vp, i64, i64, i64, i32, ctypes.POINTER(i32)]
    lib.softmax_num_kernels.restype = i32
    lib.softmax_num_kernels.argtypes = []
    lib.softmax_kernel_info.restype = i32
    lib.softmax_kernel_info.argtypes = [i32] + [ctypes.POINTER(i32)] * 8 + [ctypes.POINTER(i64)]
    lib.softmax_kernel_name.restype = ctypes.c_char_p
    lib.softmax_kernel_name.argtypes = [i32]
    lib.softmax_kernel_fits.restype = i32
    lib.softmax_kernel_fits.argtypes = [i32, vp, vp, i64, i64, i32]
    lib.softmax_status_string.restype = ctypes.c_char_p
    lib.softmax_status_string.argtypes = [i32]
    lib.softmax_version.restype = ctypes.c_char_p
    lib.softmax_version.argtypes = []
    lib.softmax_bench_copy.restype = i32
    lib.softmax_bench_copy.argtypes = [vp, vp, i64, vp]
    lib.softmax_bench_chunk_copy.restype = i32
    lib.softmax_bench_chunk_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    lib.softmax_bench_stream.restype = i32
    lib.softmax_bench_stream.argtypes = [vp, vp, i64, i32, vp]
    lib.softmax_split_workspace_bytes.restype = i64
    lib.softmax_split_workspace_bytes.argtypes = [i64, i64, i32]
    lib.softmax_fwd_split.restype = i32
    lib.softmax_fwd_split.argtypes = [vp, vp, i64, i64, i64, i32, vp, i64, i32, vp]
    lib.softmax_fwd_split_noalloc.restype = i32
    lib.softmax_fwd_split_noalloc.argtypes = [vp, vp, i64, i64, i64, i32, i32, vp]
    lib.attention_fwd.restype = i32
    lib.attention_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, i32, i32, vp]
    lib.softmax_unfused_workspace_bytes.restype = i64
    lib.softmax_unfused_workspace_bytes.argtypes = [i64, i64, i32]
    lib.softmax_unfused_5op.restype = i32
    lib.softmax_unfused_5op.argtypes = [vp, vp, i64, i64, i64, i32, vp, i64, vp]
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    return _lib.softmax_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise SoftmaxError(status, where)


def softmax_fwd(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int,
                dtype: int, stream: int = 0) -> None:
    """Raw entry point: device pointers as ints, the stream as an int handle."""
    lib = _load()
    _check(lib.softmax_fwd(in_ptr, out_ptr, rows, cols, row_stride, dtype, stream), "softmax_fwd")


def softmax_fwd_kernel(kernel_id: int, in_ptr: int, out_ptr: int, rows: int, cols: int,
                       row_stride: int, dtype: int, stream: int = 0) -> None:
    """Raw entry point that forces one compiled kernel of the library's table."""
    lib = _load()
    _check(lib.softmax_fwd_kernel(kernel_id, in_ptr, out_ptr, rows, cols, row_stride, dtype, stream),
           "softmax_fwd_kernel")


def softmax_fwd_causal(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int,
                       scale: float, diag: int, dtype: int, stream: int = 0) -> None:
    """Raw entry point of the scaled, causally masked softmax (row i keeps j <= i + diag)."""
    lib = _load()
    _check(lib.softmax_fwd_causal(in_ptr, out_ptr, rows, cols, row_stride, scale, diag, dtype, stream),
           "softmax_fwd_causal")


def softmax_fwd_causal_batched(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int,
                               rows_per_matrix: int, scale: float, diag: int, dtype: int, stream: int = 0) -> None:
    """Raw entry point of the causal softmax over stacked score matrices (row i of each matrix
    keeps j <= i + diag, i counted within its matrix of rows_per_matrix rows)."""
    lib = _load()
    _check(lib.softmax_fwd_causal_batched(in_ptr, out_ptr, rows, cols, row_stride, rows_per_matrix, scale, diag,
                                          dtype, stream), "softmax_fwd_causal_batched")


def softmax_fwd_causal_kernel(kernel_id: int, in_ptr: int, out_ptr: int, rows: int, cols: int,
                              row_stride: int, scale: float, diag: int, dtype: int, stream: int = 0) -> None:
    lib = _load()
    _check(lib.softmax_fwd_causal_kernel(kernel_id, in_ptr, out_ptr, rows, cols, row_stride, scale, diag,
                                         dtype, stream), "softmax_fwd_causal_kernel")


# softmax_select's answer when softmax_fwd splits few, very wide rows over
# several workgroups (SOFTMAX_KERNEL_SPLIT): not an id of the kernel table.
SPLIT_KERNEL = -1


def softmax_select(in_ptr: int, out_ptr: int, cols: int, row_stride: int, dtype: int,
                   rows: int = 1, causal: bool = False) -> int:
    """The kernel id the library's width dispatch picks for this call, or
    SPLIT_KERNEL for softmax_fwd's split of few, very wide rows."""
    lib = _load()
    kid = ctypes.c_int(-1)
    fn = lib.softmax_select_causal if causal else lib.softmax_select
    _check(fn(in_ptr, out_ptr, rows, cols, row_stride, dtype, ctypes.byref(kid)), "softmax_select")
    return kid.value


def softmax_fwd_variant(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int, dtype: int,
                        variant: int, block: int, stream: int = 0) -> None:
    """Raw entry point through a forced variant (0 packed, 1 row, 2 online, 3 row_pf, 4 row16) and size
    (packed: lanes per row; else threads per workgroup)."""
    lib = _load()
    _check(lib.softmax_fwd_variant(in_ptr, out_ptr, rows, cols, row_stride, dtype, variant, block, stream),
           "softmax_fwd_variant")


def softmax_select_variant(cols: int, dtype: int) -> tuple[int, int]:
    """(variant, block) softmax_fwd picks for a contiguous, aligned tensor of this width."""
    lib = _load()
    v, b = ctypes.c_int(-1), ctypes.c_int(-1)
    _check(lib.softmax_select_variant(cols, dtype, ctypes.byref(v), ctypes.byref(b)), "softmax_select_variant")
    return v.value, b.value


def bench_copy(src_ptr: int, dst_ptr: int, nbytes: int, stream: int = 0) -> None:
    """Plain 16-byte-vector device copy (the achievable-bandwidth reference)."""
    lib = _load()
    _check(lib.softmax_bench_copy(src_ptr, dst_ptr, nbytes, stream), "softmax_bench_copy")


def bench_stream(src_ptr: int, dst_ptr: int, nbytes: int, mode: int, stream: int = 0) -> None:
    """The copy's directions apart: mode 0 copy, 1 read-only, 2 write-only (bandwidth references)."""
    lib = _load()
    _check(lib.softmax_bench_stream(src_ptr, dst_ptr, nbytes, mode, stream), "softmax_bench_stream")


CHUNK_COPY_SHAPES = ((4, 2), (8, 2), (4, 4), (16, 2), (4, 8), (8, 4), (4, 16), (8, 8), (16, 4))


def bench_chunk_copy(src_ptr: int, dst_ptr: int, nbytes: int, waves: int, accesses: int, stream: int = 0) -> None:
    """Copy in per-workgroup chunks shaped like the row kernels (waves x 64 x accesses x 16 bytes)."""
    lib = _load()
    _check(lib.softmax_bench_chunk_copy(src_ptr, dst_ptr, nbytes, waves, accesses, stream), "softmax_bench_chunk_copy")


def split_workspace_bytes(rows: int, cols: int, dtype: int) -> int:
    return int(_load().softmax_split_workspace_bytes(rows, cols, dtype))


def softmax_fwd_split(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int, dtype: int,
                      workspace_ptr: int, workspace_size: int, force: int = 0, stream: int = 0) -> None:
    """Softmax allowed to split few, wide rows over several workgroups (caller workspace)."""
    lib = _load()
    _check(lib.softmax_fwd_split(in_ptr, out_ptr, rows, cols, row_stride, dtype, workspace_ptr, workspace_size,
                                 force, stream), "softmax_fwd_split")


# Bytes of the library's static split-path scratch (SOFTMAX_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 1 << 20


def softmax_fwd_split_noalloc(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int, dtype: int,
                              force: int = 0, stream: int = 0) -> None:
    """softmax_fwd_split without a workspace: the split path's partials go to the
    library's static per-device scratch (calls overlapping on one GPU race)."""
    lib = _load()
    _check(lib.softmax_fwd_split_noalloc(in_ptr, out_ptr, rows, cols, row_stride, dtype, force, stream),
           "softmax_fwd_split_noalloc")


def attention_fwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, batch: int, heads: int, nq: int, nk: int,
                  head_dim: int, scale: float, causal: bool, dtype: int, stream: int = 0) -> None:
    """Raw entry point of the fused attention forward (dense [batch, heads, n, head_dim] layouts)."""
    lib = _load()
    _check(lib.attention_fwd(q_ptr, k_ptr, v_ptr, o_ptr, batch, heads, nq, nk, head_dim, scale, int(bool(causal)),
                             dtype, stream), "attention_fwd")


def attention(q, k, v, scale: float | None = None, causal: bool = False, out=None):
    """softmax(scale q k^T) v for contiguous [batch, heads, n, head_dim] fp16 / bf16 CUDA tensors."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("attention: q, k, v must be [batch, heads, n, head_dim]")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("attention: q, k, v must be contiguous GPU tensors of one dtype")
    b, h, nq, d = q.shape
    nk = k.shape[2]
    if tuple(k.shape) != (b, h, nk, d) or tuple(v.shape) != (b, h, nk, d):
        raise ValueError("attention: k and v must be [batch, heads, nk, head_dim] matching q")
    if k.device != q.device or v.device != q.device:
        raise ValueError("attention: q, k, v must be on one device")
    code = _torch_dtype_code(q)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    elif (tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous()
          or out.device != q.device):
        raise ValueError("attention: out must be a contiguous tensor of q's shape, dtype and device")
    scale = 1.0 / float(d) ** 0.5 if scale is None else float(scale)
    with torch.cuda.device(q.device):  # the library launches on the current device
        attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), b, h, nq, nk, d, scale, causal,
                      code, torch.cuda.current_stream(q.device).cuda_stream)
    return out


def unfused_workspace_bytes(rows: int, cols: int, dtype: int) -> int:
    return int(_load().softmax_unfused_workspace_bytes(rows, cols, dtype))


def unfused_5op(in_ptr: int, out_ptr: int, rows: int, cols: int, row_stride: int, dtype: int,
                workspace_ptr: int, workspace_size: int, stream: int = 0) -> None:
    """The unfused five-kernel softmax (measurement baseline); needs a caller workspace."""
    lib = _load()
    _check(lib.softmax_unfused_5op(in_ptr, out_ptr, rows, cols, row_stride, dtype, workspace_ptr,
                                   workspace_size, stream), "softmax_unfused_5op")


@dataclass(frozen=True)
class KernelInfo:
    kid: int
    name: str
    dtype: int
    variant: str
    causal: bool        # entry of the scaled, causally masked softmax
    vec_elems: int      # elements per load
    lanes: int          # lanes per row (packed) or threads per row (row/online)
    vecs_per_lane: int  # loads per lane per row (or per chunk, online)
    groups: int         # row groups per wave (packed)
    block: int          # threads per workgroup (packed: maximum)
    max_cols: int       # widest row it handles (-1: any)


def kernel_table() -> list[KernelInfo]:
    lib = _load()
    out = []
    for kid in range(lib.softmax_num_kernels()):
        ints = [ctypes.c_int() for _ in range(8)]
        mc = ctypes.c_int64()
        _check(lib.softmax_kernel_info(kid, *[ctypes.byref(v) for v in ints], ctypes.byref(mc)),
               "softmax_kernel_info")
        dt, var, causal, ve, lanes, vpl, groups, block = (v.value for v in ints)
        out.append(KernelInfo(kid, lib.softmax_kernel_name(kid).decode(), dt, VARIANT_NAMES[var],
                              bool(causal), ve, lanes, vpl, groups, block, mc.value))
    return out


def kernel_fits(kid: int, in_ptr: int, out_ptr: int, cols: int, row_stride: int, dtype: int) -> bool:
    return bool(_load().softmax_kernel_fits(kid, in_ptr, out_ptr, cols, row_stride, dtype))


def version() -> str:
    return _load().softmax_version().decode()


# ---------------------------------------------------------------- torch layer

def _torch_dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in codes:
        raise TypeError(f"softmax: unsupported dtype {t.dtype} (fp32, fp16, bf16 only)")
    return codes[t.dtype]


def _as_rows(t):
    """(rows, cols, row_stride) of the row matrix a tensor holds, or ValueError.

    The last dimension must have unit stride whatever the rank (a strided or
    expanded 1-D view is not one row of adjacent elements); a 2-D tensor may
    have gapped rows; higher ranks must be contiguous."""
    if t.dim() < 1:
        raise ValueError("softmax: input must have at least one dimension")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("softmax: the last dimension must be contiguous (unit stride)")
    cols = t.shape[-1]
    if t.dim() == 1:
        return 1, cols, cols
    if t.dim() == 2:
        return t.shape[0], cols, (t.stride(0) if t.shape[0] > 1 else cols)
    if not t.is_contiguous():
        raise ValueError("softmax: inputs of rank > 2 must be contiguous")
    return t.numel() // max(cols, 1), cols, cols


def softmax(x, out=None, kernel_id: int | None = None, causal: bool = False, scale: float = 1.0,
            diag: int = 0):
    """Row softmax over the last dimension of a CUDA (HIP) tensor.

    ``out`` (optional) must match ``x`` in shape, dtype and strides; it may be
    ``x`` itself (in place).  With ``causal=True`` row i keeps columns
    j <= i + diag and the kept entries are multiplied by ``scale`` first; for
    a tensor of rank > 2 ([..., n, m] score matrices) i counts within each
    matrix.  The call is asynchronous on torch's current stream.
    """
    import torch
    if causal and x.dim() > 2 and kernel_id is not None:
        raise ValueError("softmax: a forced causal kernel takes one score matrix (1-D or 2-D input)")
    if not x.is_cuda:
        raise ValueError("softmax: input must be a GPU tensor")
    code = _torch_dtype_code(x)
    rows, cols, stride = _as_rows(x)
    if out is None:  # same strides as x (empty_like would make a gapped row view contiguous)
        out = torch.empty_strided(x.shape, x.stride(), dtype=x.dtype, device=x.device)
    if out.shape != x.shape or out.dtype != x.dtype or out.stride() != x.stride() or out.device != x.device:
        raise ValueError("softmax: out must match the input's shape, dtype, strides and device")
    with torch.cuda.device(x.device):  # the library launches on the current device
        stream = torch.cuda.current_stream(x.device).cuda_stream
        if causal:
            if x.dim() > 2:  # contiguous (checked by _as_rows): matrices of x.shape[-2] rows each
                softmax_fwd_causal_batched(x.data_ptr(), out.data_ptr(), rows, cols, stride, x.shape[-2], scale,
                                           diag, code, stream)
            elif kernel_id is None:
                softmax_fwd_causal(x.data_ptr(), out.data_ptr(), rows, cols, stride, scale, diag, code, stream)
            else:
                softmax_fwd_causal_kernel(kernel_id, x.data_ptr(), out.data_ptr(), rows, cols, stride, scale,
                                          diag, code, stream)
        elif kernel_id is None:
            softmax_fwd(x.data_ptr(), out.data_ptr(), rows, cols, stride, code, stream)
        else:
            softmax_fwd_kernel(kernel_id, x.data_ptr(), out.data_ptr(), rows, cols, stride, code, stream)
    return out

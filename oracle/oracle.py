"""CPU oracle for the row softmax -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around ``softmax_oracle.c``: a plain, single-threaded,
double-precision implementation of the definition

    y[i, j] = exp(x[i, j] - max_k x[i, k]) / sum_k exp(x[i, k] - max_k x[i, k])

(the row softmax with max subtraction described on the pages "I Wrote My First
GPU Kernel", section "What Fusion Actually Does", and "GPU Kernels -
Implementing and optimizing Softmax", section "Baseline & Triton Softmax
kernel"), plus ``softmax_mt``, the same function run unchanged over
contiguous row ranges on several threads for the CPU baseline's timing.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It never imports the GPU package, and the GPU
package never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "softmax_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at a deliberately broken build of the oracle
# (mutation testing of the pins); nothing else sets this.
_LIB_OVERRIDE = os.environ.get("ROW_SOFTMAX_ORACLE_LIB")

# Element-type codes of the oracle's C interface (fp32, fp16, bf16).
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile softmax_oracle.c with gcc (no fast-math) into liboracle.so."""
    if _LIB_OVERRIDE is not None:
        return _LIB_OVERRIDE
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-shared", "-fPIC", "-pthread",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if _LIB_OVERRIDE is None and not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(path)
        lib.oracle_softmax.restype = ctypes.c_int
        lib.oracle_softmax.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p,
        ]
        lib.oracle_softmax_mt.restype = ctypes.c_int
        lib.oracle_softmax_mt.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.oracle_softmax_causal.restype = ctypes.c_int
        lib.oracle_softmax_causal.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int64, ctypes.c_void_p,
        ]
        lib.oracle_attention_fwd.restype = ctypes.c_int
        lib.oracle_attention_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
        ]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        _lib = lib
    return _lib


def softmax(x: np.ndarray, dtype: str, cols: int | None = None) -> np.ndarray:
    """Row softmax of ``x`` in float64.

    ``x`` is a 2-D C-contiguous array holding the raw input: ``float32`` for
    ``dtype == "f32"``, ``uint16`` bit patterns for ``"f16"`` and ``"bf16"``.
    Its second dimension is the row stride; ``cols`` (default: all of it) is
    the number of leading columns each row actually has.  Returns a dense
    ``(rows, cols)`` float64 array.
    """
    lib = _load()
    code = DTYPE_CODES[dtype]
    want = np.float32 if dtype == "f32" else np.uint16
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} input must be held as {want.__name__}, got {x.dtype}")
    if x.ndim != 2 or not x.flags.c_contiguous:
        raise ValueError("oracle: input must be a 2-D C-contiguous array")
    rows, stride = x.shape
    cols = stride if cols is None else int(cols)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib.oracle_softmax(x.ctypes.data, code, rows, cols, stride, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_softmax rejected its arguments (rc={rc})")
    return out


def softmax_mt(x: np.ndarray, dtype: str, threads: int, cols: int | None = None) -> np.ndarray:
    """:func:`softmax` over ``threads`` contiguous row ranges on POSIX threads
    (the CPU baseline's all-cores timing); bit-identical to :func:`softmax`."""
    lib = _load()
    code = DTYPE_CODES[dtype]
    want = np.float32 if dtype == "f32" else np.uint16
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} input must be held as {want.__name__}, got {x.dtype}")
    if x.ndim != 2 or not x.flags.c_contiguous:
        raise ValueError("oracle: input must be a 2-D C-contiguous array")
    rows, stride = x.shape
    cols = stride if cols is None else int(cols)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib.oracle_softmax_mt(x.ctypes.data, code, rows, cols, stride, out.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_softmax_mt rejected its arguments (rc={rc})")
    return out


def softmax_causal(x: np.ndarray, dtype: str, scale: float, diag: int = 0,
                   cols: int | None = None) -> np.ndarray:
    """Scaled, causally masked row softmax in float64.

    Row i keeps columns j <= i + diag; kept entries are multiplied by
    ``scale`` (> 0) before the softmax, masked ones give +0.  ``x`` is held
    as in :func:`softmax`.
    """
    lib = _load()
    code = DTYPE_CODES[dtype]
    want = np.float32 if dtype == "f32" else np.uint16
    if x.dtype != want:
        raise TypeError(f"oracle: {dtype} input must be held as {want.__name__}, got {x.dtype}")
    if x.ndim != 2 or not x.flags.c_contiguous:
        raise ValueError("oracle: input must be a 2-D C-contiguous array")
    rows, stride = x.shape
    cols = stride if cols is None else int(cols)
    out = np.empty((rows, cols), dtype=np.float64)
    rc = lib.oracle_softmax_causal(x.ctypes.data, code, rows, cols, stride, float(scale), int(diag),
                                   out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_softmax_causal rejected its arguments (rc={rc})")
    return out


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dtype: str, scale: float,
                  causal: bool) -> np.ndarray:
    """O = softmax(scale * Q K^T, causal mask) V in float64.

    q is [batch, heads, nq, d], k and v are [batch, heads, nk, d], held as in
    :func:`softmax` (float32, or uint16 bits for f16 / bf16).  With ``causal``
    query i keeps keys j <= i + (nk - nq); a query with no kept key gives 0.
    """
    lib = _load()
    code = DTYPE_CODES[dtype]
    want = np.float32 if dtype == "f32" else np.uint16
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != want or t.ndim != 4 or not t.flags.c_contiguous:
            raise ValueError(f"oracle: {name} must be a C-contiguous 4-D {want.__name__} array")
    b, h, nq, d = q.shape
    nk = k.shape[2]
    if k.shape != (b, h, nk, d) or v.shape != (b, h, nk, d):
        raise ValueError("oracle: k and v must be [batch, heads, nk, d] matching q")
    out = np.empty((b, h, nq, d), dtype=np.float64)
    rc = lib.oracle_attention_fwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, code, b, h, nq, nk, d,
                                  float(scale), int(bool(causal)), out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attention_fwd rejected its arguments (rc={rc})")
    return out


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode fp16 / bf16 bit patterns to float64 with the oracle's own decoders."""
    lib = _load()
    fn = lib.oracle_decode_f16 if dtype == "f16" else lib.oracle_decode_bf16
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.fromiter((fn(int(b)) for b in flat), dtype=np.float64, count=flat.size).reshape(np.shape(bits))

"""Seeded synthetic inputs for the row softmax, shared by tests and the benchmark.

This module only *generates inputs*: it holds none of the softmax arithmetic.
Each workload stands in for one of the shapes the pages measure (their input
distributions are never stated, so the distributions here are a stated recipe):

* ``c1``  128 x 1000 fp32, x ~ N(0, 3^2); row 0 all 0.5, row 1 has 100.0 in its
  last column, row 2 has its last 200 columns at -inf (the stability and
  masking cases of "I Wrote My First GPU Kernel", sections "What Fusion
  Actually Does" and "The Kernel");
* ``c2``  causal attention scores 2048 x 2048 fp32: x = q k^T / sqrt(64) with
  q, k ~ N(0, 1) of head dim 64, and x[i, j] = -inf for j > i (the causal mask
  and 1/sqrt(d) scale of "Dissecting Memory Bandwidth & SRAM Tiling in
  Triton", section "Writing the Kernel in OpenAI Triton");
* ``c3``  8192 x 4096 fp16, x ~ N(0, 1) (the shape of "fused-softmax-roofline");
* ``c4``  4096 x 4096 fp32, x ~ U(-10, 10) (the shape of "Kernel Fusion",
  section "Where the time goes in an elementwise chain");
* ``c5``  the width sweep of "GPU Kernels - Implementing and optimizing
  Softmax" (widths 32 ... 16384, about 200 MB per tensor), bf16 and fp32,
  x ~ N(0, 2^2), rows = floor(200e6 / (cols * element size));
* ``wide_*`` few, wide rows for the split-row path (8 x 2^20 fp32 and
  32 x 2^18 bf16, x ~ N(0, 2^2)); not a configuration of the pages.

Recipe: numpy ``default_rng`` (PCG64) draws in float64, in slices of about
2^20 elements whose streams are the children of ``SeedSequence(seed)``, then a
cast to the element type: fp32 and fp16 by numpy's round-to-nearest-even casts, bf16 by
rounding the fp32 value to nearest-even on its upper 16 bits.  fp16 and bf16
inputs are returned as ``uint16`` bit patterns, fp32 as ``float32``.
Seeds: c1 = 1, c2 = 2, c3 = 3, c4 = 4, c5 = [5, cols, dtype code].
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# dtype name -> (C-ABI code, element size in bytes)
DTYPES = {"f32": (0, 4), "f16": (1, 2), "bf16": (2, 2)}

SWEEP_WIDTHS = (32, 64, 128, 256, 512, 1000, 1024, 2048, 3000, 4096, 8192, 16384)
# Rows past the sweep's widest, as wide as a vocabulary's logits (about 200 MB per tensor too).
VOCAB_WIDTHS = {"bf16": (24576, 32000, 32768, 50304, 65536, 128256, 151936),
                "f32": (24576, 32000, 32768, 50304, 65536, 128256)}
SWEEP_BYTES = 200_000_000  # decimal bytes of input per sweep tensor

_CHUNK_ELEMS = 1 << 20  # rows are drawn in slices of about this many elements


def dtype_code(dtype: str) -> int:
    return DTYPES[dtype][0]


def elem_size(dtype: str) -> int:
    return DTYPES[dtype][1]


def algorithmic_bytes(rows: int, cols: int, dtype: str) -> int:
    """Bytes a single-pass row softmax must move: every element read once and written once."""
    return 2 * rows * cols * elem_size(dtype)


def cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Cast float64 draws to the storage of ``dtype`` (float32, or uint16 bits)."""
    if dtype == "f32":
        return x64.astype(np.float32)
    if dtype == "f16":
        return x64.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        b = x64.astype(np.float32).view(np.uint32)
        b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return b.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def neg_inf(dtype: str):
    """The storage value of -inf for ``dtype``."""
    return {"f32": np.float32(-np.inf), "f16": np.uint16(0xFC00), "bf16": np.uint16(0xFF80)}[dtype]


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


@dataclass(frozen=True)
class Workload:
    """One seeded input matrix.  ``kind`` selects the recipe, ``params`` its constants."""

    name: str
    rows: int
    cols: int
    dtype: str
    kind: str
    seed: tuple
    params: dict = field(default_factory=dict, hash=False, compare=False)

    @property
    def bytes(self) -> int:
        return algorithmic_bytes(self.rows, self.cols, self.dtype)

    def generate(self, rows: int | None = None) -> np.ndarray:
        """The input as a (rows, cols) array; ``rows`` truncates to the leading rows.

        The leading rows of a truncated draw equal those of the full draw.
        """
        n = self.rows if rows is None else min(int(rows), self.rows)
        if self.kind == "normal":
            return _normal(self.seed, n, self.cols, self.params["sigma"], self.dtype)
        if self.kind == "uniform":
            return _uniform(self.seed, n, self.cols, self.params["lo"], self.params["hi"], self.dtype)
        if self.kind == "c1":
            return _c1(self.seed, n, self.cols, self.dtype)
        if self.kind == "causal":
            return _causal(self.seed, n, self.cols, self.params["head_dim"], self.dtype)
        raise ValueError(self.kind)


def _draw_rows(seed, n: int, cols: int, dtype: str, draw) -> np.ndarray:
    """Rows are drawn in fixed slices; slice k uses child k of SeedSequence(seed).

    Slices are independent streams, so they are drawn on a thread pool; the
    slicing depends only on ``cols``, so a truncated draw equals the leading
    rows of the full draw.
    """
    out = np.empty((n, cols), dtype=storage_dtype(dtype))
    if n == 0 or cols == 0:
        return out
    step = max(1, _CHUNK_ELEMS // cols)
    starts = list(range(0, n, step))
    children = np.random.SeedSequence(list(seed)).spawn(len(starts))

    def fill(k: int) -> None:
        r0 = starts[k]
        r1 = min(n, r0 + step)
        rng = np.random.default_rng(children[k])
        out[r0:r1] = cast(draw(rng, (r1 - r0, cols)), dtype)

    if len(starts) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def _normal(seed, n, cols, sigma, dtype):
    return _draw_rows(seed, n, cols, dtype, lambda g, s: g.standard_normal(s) * sigma)


def _uniform(seed, n, cols, lo, hi, dtype):
    return _draw_rows(seed, n, cols, dtype, lambda g, s: g.uniform(lo, hi, s))


def _c1(seed, n, cols, dtype):
    x = _normal(seed, n, cols, 3.0, dtype)
    if n > 0:
        x[0, :] = cast(np.full(cols, 0.5), dtype)
    if n > 1:
        x[1, cols - 1] = cast(np.array([100.0]), dtype)[0]
    if n > 2:
        x[2, max(0, cols - 200):] = neg_inf(dtype)
    return x


def _causal(seed, n, cols, head_dim, dtype):
    rng = np.random.default_rng(list(seed))
    q = rng.standard_normal((cols, head_dim))  # one query per row of the full square
    k = rng.standard_normal((cols, head_dim))
    s = (q[:n] @ k.T) / np.sqrt(head_dim)
    x = cast(s, dtype)
    i = np.arange(n)[:, None]
    j = np.arange(cols)[None, :]
    x[j > i] = neg_inf(dtype)
    return x


def sweep_rows(cols: int, dtype: str) -> int:
    return SWEEP_BYTES // (cols * elem_size(dtype))


def _build_registry() -> dict:
    reg = {
        "c1": Workload("c1_128x1000_f32", 128, 1000, "f32", "c1", (1,)),
        "c2": Workload("c2_causal_2048x2048_f32", 2048, 2048, "f32", "causal", (2,), {"head_dim": 64}),
        "c3": Workload("c3_8192x4096_f16", 8192, 4096, "f16", "normal", (3,), {"sigma": 1.0}),
        "c4": Workload("c4_4096x4096_f32", 4096, 4096, "f32", "uniform", (4,), {"lo": -10.0, "hi": 10.0}),
    }
    # few, wide rows (the split-row path): vocabulary-sized logits rows
    reg["wide_f32"] = Workload("few_wide_8x1048576_f32", 8, 1 << 20, "f32", "normal", (6, 1), {"sigma": 2.0})
    reg["wide_bf16"] = Workload("few_wide_32x262144_bf16", 32, 1 << 18, "bf16", "normal", (6, 2), {"sigma": 2.0})
    for dt in ("bf16", "f32"):
        for w in SWEEP_WIDTHS:
            key = f"c5_{dt}_{w}"
            reg[key] = Workload(f"c5_sweep_{sweep_rows(w, dt)}x{w}_{dt}", sweep_rows(w, dt), w, dt,
                                "normal", (5, w, dtype_code(dt)), {"sigma": 2.0})
    for dt, widths in VOCAB_WIDTHS.items():
        for w in widths:
            reg[f"vocab_{dt}_{w}"] = Workload(f"vocab_{sweep_rows(w, dt)}x{w}_{dt}", sweep_rows(w, dt), w, dt,
                                              "normal", (7, w, dtype_code(dt)), {"sigma": 2.0})
    return reg


WORKLOADS = _build_registry()


def random_matrix(seed: int, rows: int, cols: int, dtype: str, sigma: float = 1.0,
                  row_stride: int | None = None, pad_value=None) -> np.ndarray:
    """A (rows, row_stride) N(0, sigma^2) matrix whose columns past ``cols`` hold ``pad_value``.

    Used for edge-case shapes (odd widths, padded strides).  Padding defaults
    to NaN (fp32) or an fp16/bf16 NaN pattern so any read of it shows up.
    """
    stride = cols if row_stride is None else int(row_stride)
    rng = np.random.default_rng([seed, rows, cols, stride, dtype_code(dtype)])
    x = np.empty((rows, stride), dtype=storage_dtype(dtype))
    x[:, :cols] = cast(rng.standard_normal((rows, cols)) * sigma, dtype)
    if stride > cols:
        if pad_value is None:
            pad_value = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}[dtype]
        x[:, cols:] = pad_value
    return x

"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every case prints what it runs before touching the GPU, so a failing run
names its case.  Inputs are the seeded workloads and seeded edge shapes; the
oracle computes every expected value.
"""
import os
import sys

import numpy as np
import pytest

from oracle import oracle as O
from row_wise_softmax_amd import binding
from row_wise_softmax_amd import workloads as W

from gpu_util import (TOL, causal_mask, check, check_every_row, check_padding_untouched, decode, run, sentinel,
                      to_device, to_host)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    binding._load()  # fails loudly if the HIP library is missing


# --------------------------------------------------------- the five configs

@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c4"])
def test_config_full_parity(key):
    wl = W.WORKLOADS[key]
    _say(f"{key} {wl.name}")
    x = wl.generate()
    y = run(x, wl.dtype)
    ref = O.softmax(x, wl.dtype)
    err = check(y, x, wl.dtype, ref, label=wl.name)
    _say(f"{key} max abs err {err:.3e}")


def test_c1_special_rows():
    wl = W.WORKLOADS["c1"]
    x = wl.generate()
    y = decode(run(x, "f32"), "f32")
    assert np.all(np.abs(y[0] - 1e-3) <= 2e-6)          # constant row -> 1/n
    assert np.isfinite(y[1]).all() and y[1, -1] > 0.999  # the 100.0 entry dominates
    assert np.all(y[2, 800:] == 0.0)                     # -inf tail -> exact zeros
    assert abs(y[2, :800].sum() - 1.0) <= 1e-5


def test_c2_causal_first_rows():
    x = W.WORKLOADS["c2"].generate()
    y = decode(run(x, "f32"), "f32")
    assert y[0, 0] == 1.0 and np.all(y[0, 1:] == 0.0)
    for i in (1, 7, 2047):
        assert np.all(y[i, i + 1:] == 0.0)


_FULL_KEYS = [f"c5_{dt}_{w}" for w in W.SWEEP_WIDTHS for dt in ("bf16", "f32")] + \
             [f"vocab_{dt}_{w}" for dt, ws in W.VOCAB_WIDTHS.items() for w in ws]


@pytest.mark.parametrize("key", _FULL_KEYS)
def test_sweep_full_size_every_row(key):
    """Full-size sweep and vocabulary-width inputs (about 200 MB each) in the
    benchmark's launch shape, compared with the oracle element by element over
    every row, plus the value range and the row sums."""
    wl = W.WORKLOADS[key]
    dtype = wl.dtype
    _say(f"sweep {wl.name}")
    x = wl.generate()
    y = run(x, dtype, prefill_out=False)
    err = check_every_row(y, x, dtype, label=wl.name)
    yd = decode(y, dtype)
    assert np.all(yd >= 0.0) and np.all(yd <= 1.0)
    # fp32 row sums are held to 1e-5 inside check_every_row.  bf16: each output
    # carries a relative rounding error of at most its unit roundoff 2^-8 (8
    # significant bits, round to nearest), so the sum is within 2^-8 of 1.
    if dtype == "bf16":
        assert np.max(np.abs(yd.sum(axis=1) - 1.0)) <= 2.0 ** -8
    _say(f"sweep {wl.name} rows {wl.rows} max abs err {err:.3e}")


# Rows just past a power of two of 16-byte accesses, in job sizes that take
# three accesses per lane on half the waves (and one that stays past the fill
# line), rows of 2049..3072 accesses on sixteen waves of three, and 16-bit rows
# of 1537..2000 accesses in jobs of 1281..3072 rows on eight waves of four,
# jobs just past the persistent twin's two rounds (a quarter of the waves with
# eight accesses each; fp32 sixteen-wave rows on the twin up to 1280 rows);
# softmax_fwd picks the kernel, every row is compared.
_V3_CASES = [("bf16", 2100, 8800, "row_bf16_w8_v3"), ("f16", 2100, 8 * 1536, "row_f16_w8_v3"),
             ("bf16", 4200, 4160, "row_bf16_w4_v3"), ("bf16", 8300, 2400, "row_bf16_w2_v3"),
             ("f32", 2100, 4400, "row_f32_w8_v3"), ("f32", 4200, 2080, "row_f32_w4_v3"),
             ("bf16", 4200, 6000, "row_bf16_w8_v2"), ("bf16", 2100, 20000, "row_bf16_w16_v3"),
             ("f16", 1500, 24576, "row_f16_w16_v3"), ("f32", 1100, 10000, "row_f32_w16_v3"),
             ("bf16", 1700, 14400, "row_bf16_w8_v4"), ("f16", 3072, 8 * 1537, "row_f16_w8_v4"),
             ("bf16", 1100, 16384, "row_bf16_w4_v8"), ("f16", 2200, 8192, "row_f16_w2_v8"),
             ("f32", 1200, 8192, "rowpf_f32_w16_v2")]


@pytest.mark.parametrize("dtype,rows,cols,kernel", _V3_CASES)
def test_three_access_dispatch_every_row(dtype, rows, cols, kernel):
    import torch
    _say(f"three-access dispatch {dtype} {rows}x{cols} -> {kernel}")
    x = W.random_matrix(seed=cols, rows=rows, cols=cols, dtype=dtype, sigma=3.0)
    x[3, : cols // 2] = W.neg_inf(dtype)
    xd = to_device(x, dtype)
    yd = torch.empty_like(xd)
    kid = binding.softmax_select(xd.data_ptr(), yd.data_ptr(), cols, cols, W.dtype_code(dtype), rows=rows)
    assert binding.kernel_table()[kid].name == kernel
    y = run(x, dtype, prefill_out=False)
    check_every_row(y, x, dtype, label=f"{dtype} {rows}x{cols}")


# ------------------------------------------------------------ edge shapes

EDGE_WIDTHS = [1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 64, 65, 127, 129, 255, 257, 511, 513,
               999, 1000, 1001, 2047, 2048, 2049, 3000, 4095, 4096, 4097, 8191, 8192, 8193]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", EDGE_WIDTHS)
def test_edge_widths(dtype, cols):
    _say(f"edge {dtype} cols={cols}")
    x = W.random_matrix(seed=21, rows=37, cols=cols, dtype=dtype, sigma=3.0)
    y = run(x, dtype)
    check(y, x, dtype, O.softmax(x, dtype), label=f"{dtype} cols={cols}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [16384, 32768, 65536, 65537, 131072, 1 << 18])
def test_wide_rows(dtype, cols):
    _say(f"wide {dtype} cols={cols}")
    x = W.random_matrix(seed=22, rows=6, cols=cols, dtype=dtype, sigma=2.0)
    y = run(x, dtype)
    check(y, x, dtype, O.softmax(x, dtype), label=f"{dtype} cols={cols}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols,stride", [(1000, 1024), (1000, 1003), (96, 128), (4096, 4104), (7, 8)])
def test_row_stride_and_untouched_padding(dtype, cols, stride):
    _say(f"stride {dtype} cols={cols} stride={stride}")
    x = W.random_matrix(seed=23, rows=29, cols=cols, dtype=dtype, row_stride=stride)
    y = run(x, dtype, cols=cols)
    check(y, x, dtype, O.softmax(x, dtype, cols=cols), cols=cols, label=f"{dtype} {cols}/{stride}")
    check_padding_untouched(y, cols, dtype, label=f"{dtype} {cols}/{stride}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [64, 1000, 4096, 70000])
def test_in_place(dtype, cols):
    _say(f"in-place {dtype} cols={cols}")
    x = W.random_matrix(seed=24, rows=33, cols=cols, dtype=dtype)
    y = run(x, dtype, inplace=True)
    check(y, x, dtype, O.softmax(x, dtype), label=f"in-place {dtype} {cols}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("out_shift", [1, 2])
def test_misaligned_pointers(dtype, out_shift):
    """Rows one element past a 16-byte boundary.  With the output at the same
    offset (out_shift 1) the any-alignment kernels run; at another offset
    (out_shift 2) the scalar path does."""
    import torch
    _say(f"misaligned {dtype} out_shift={out_shift}")
    cols = 1000
    x = W.random_matrix(seed=25, rows=11, cols=cols + 1, dtype=dtype)
    xd = to_device(x, dtype)[:, 1:]            # starts one element past a 16-byte boundary
    out_full = torch.full((11 * (cols + 1) + 2,), float("nan"), dtype=xd.dtype, device="cuda")
    out = out_full[out_shift:out_shift + 11 * (cols + 1)].view(11, cols + 1)[:, :cols]
    code = W.dtype_code(dtype)
    kid = binding.softmax_select(xd.data_ptr(), out.data_ptr(), cols, cols + 1, code, rows=11)
    k = binding.kernel_table()[kid]
    assert ("any_" in k.name) if out_shift == 1 else (k.vec_elems == 1)
    binding.softmax_fwd(xd.data_ptr(), out.data_ptr(), 11, cols, cols + 1, code,
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    y = to_host(out, dtype)
    xs = np.ascontiguousarray(x[:, 1:])
    check(np.ascontiguousarray(y), xs, dtype, O.softmax(xs, dtype), label="misaligned")
    # the gaps between rows, and the elements around the output, stay untouched
    full = to_host(out_full, dtype).reshape(-1)
    wrote = np.zeros(full.size, dtype=bool)
    for r in range(11):
        wrote[out_shift + r * (cols + 1): out_shift + r * (cols + 1) + cols] = True
    rest = full[~wrote]
    assert np.isnan(decode(rest, dtype)).all(), "an element outside the rows was written"


def test_empty_inputs_launch_nothing():
    import torch
    x = torch.empty((0, 128), device="cuda")
    binding.softmax_fwd(x.data_ptr(), x.data_ptr(), 0, 128, 128, 0, 0)
    binding.softmax_fwd(0, 0, 5, 0, 0, 1, 0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("cols", [8, 256, 4096, 40000])
def test_all_neg_inf_rows_give_zeros(dtype, cols):
    _say(f"all -inf {dtype} cols={cols}")
    x = W.random_matrix(seed=26, rows=9, cols=cols, dtype=dtype)
    x[3, :] = W.neg_inf(dtype)
    x[5, ::2] = W.neg_inf(dtype)
    y = run(x, dtype)
    check(y, x, dtype, O.softmax(x, dtype), label=f"-inf {dtype} {cols}")
    yd = decode(y, dtype)
    assert np.all(yd[3] == 0.0) and not np.signbit(yd[3]).any()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_extreme_values(dtype):
    _say(f"extremes {dtype}")
    big = {"f32": 3.0e38, "f16": 65504.0, "bf16": 3.0e38}[dtype]
    x64 = np.random.default_rng(27).standard_normal((6, 300))
    x64[0, 17] = big
    x64[1, :] = -big
    x64[2, 5] = 100.0
    x64[3, :] = big
    x = W.cast(x64, dtype)
    y = run(x, dtype)
    check(y, x, dtype, O.softmax(x, dtype), label=f"extremes {dtype}")


@pytest.mark.parametrize("key", ["c3", "c4", "c5_bf16_32"])
def test_deterministic(key):
    wl = W.WORKLOADS[key]
    x = wl.generate(rows=min(wl.rows, 50000))
    a = run(x, wl.dtype)
    b = run(x, wl.dtype)
    assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_many_rows_past_the_grid_cap():
    """More workgroups than one launch holds: the kernels' grid-stride loop."""
    table = binding.kernel_table()
    kid = next(k.kid for k in table if k.name == "row_f32_w2_v1")
    rows = (1 << 20) + 3
    _say(f"grid cap rows={rows}")
    x = W.random_matrix(seed=28, rows=rows, cols=8, dtype="f32")
    y = run(x, "f32", kernel_id=kid, prefill_out=False)
    check(y, x, "f32", O.softmax(x, "f32"), label="grid cap")


# ---------------------------------------------------- every table entry

def _table():
    try:
        return binding.kernel_table()
    except Exception:  # library missing: the fixture above fails each test loudly
        return []


_TABLE = _table()
_DT = {0: "f32", 1: "f16", 2: "bf16"}


def _widths_for(k):
    n = k.vec_elems
    if "any_" in k.name:  # odd widths: consecutive rows start at every offset within a chunk
        if k.max_cols > 0:
            m = k.max_cols
            return sorted({w for w in (m, m - 2, (m // 2) | 1, 1, 3) if 1 <= w <= m})
        chunk = k.lanes * k.vecs_per_lane * n
        return sorted({1, chunk + 1, 2 * chunk + 3 * n + 1})
    if k.max_cols > 0:
        m = k.max_cols
        ws = {m, max(n, m - n), max(n, (m // 2 // n) * n + n), n}
    else:
        chunk = k.lanes * k.vecs_per_lane * n
        ws = {n, 2 * chunk + 3 * n, chunk + n} if n > 1 else {1, 2 * chunk + 3, 777}
    return sorted(ws)


def _rows_for(k, cols):
    if k.variant == "packed":
        per_block = 4 * (64 // k.lanes) * k.groups
        return 2 * per_block + 7
    if k.variant == "row_pf":
        # more rows than the chip holds workgroups, so every workgroup runs
        # its prefetch loop (at most 32 resident workgroups per CU x 256 CUs)
        return max(45, min(16389, 20_000_000 // max(cols, 1)))
    return 45


@pytest.mark.parametrize("kid", [k.kid for k in _TABLE], ids=[k.name for k in _TABLE])
def test_every_kernel_in_the_table(kid):
    k = _TABLE[kid]
    dtype = _DT[k.dtype]
    for cols in _widths_for(k):
        rows = _rows_for(k, cols)
        _say(f"{k.name} rows={rows} cols={cols}")
        x = W.random_matrix(seed=kid, rows=rows, cols=cols, dtype=dtype, sigma=3.0)
        x[1, : max(1, cols // 3)] = W.neg_inf(dtype)  # a partly masked row
        if k.causal:
            # a diagonal that leaves some rows empty, some partial, some full
            diag = cols // 2 - rows // 2
            y = run(x, dtype, kernel_id=kid, causal=True, scale=0.375, diag=diag)
            check(y, x, dtype, O.softmax_causal(x, dtype, 0.375, diag), label=f"{k.name} cols={cols}",
                  keep=causal_mask(rows, cols, diag))
        else:
            y = run(x, dtype, kernel_id=kid)
            check(y, x, dtype, O.softmax(x, dtype), label=f"{k.name} cols={cols}")


# ------------------------------------------- magnitudes x kernel families

_MAGNITUDES = [1e3, 1e5, 3e6, 1e7, 1e9, 3e9, 1e12, 1e20, 1e30, 1e37, 3e38]
_FAMILIES = ["packed_{d}_l64_v2_g1", "row_{d}_w4_v2", "rowpf_{d}_w4_v2", "online_{d}_vec_w4_v2",
             "online_{d}_scalar_w4_v8"]
_CAUSAL_FAMILIES = ["causal_packed_{d}_l64_v2_g1", "causal_row_{d}_w4_v2", "causal_online_{d}_vec_w16_v4",
                    "causal_online_{d}_scalar_w4_v8"]


def _magnitude_rows(dtype, cols=512, seed=51):
    """Rows whose max spans 1e3 .. 3e38 (clipped to the type), both signs,
    entries a few units in the last place apart, some mixed with ordinary values."""
    top = {"f32": 3.3e38, "bf16": 3.3e38, "f16": 6.0e4}[dtype]
    rng = np.random.default_rng(seed)
    rows = []
    for mag in _MAGNITUDES:
        mag = min(mag, top)
        for sign in (1.0, -1.0):
            base = np.float64(np.float32(sign * mag))
            ulp = float(np.spacing(np.float32(abs(base)))) * (2 ** 16 if dtype != "f32" else 1)
            rows.append(base + rng.integers(-40, 1, size=cols) * ulp)   # a cluster just below the max
            mixed = rng.standard_normal(cols) * 3.0
            mixed[rng.integers(0, cols, size=3)] = base
            rows.append(mixed)                                          # ordinary values and a few huge ones
    x = W.cast(np.clip(np.array(rows), -top, top), dtype)
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("family", _FAMILIES + _CAUSAL_FAMILIES + ["row16_{d}_w8_v12"])
def test_magnitudes_every_family(dtype, family):
    if family.startswith("row16_") and dtype == "f32":
        pytest.skip("the stored-value row kernel is 16-bit only")
    name = family.format(d=dtype)
    k = next((k for k in _TABLE if k.name == name), None)
    assert k is not None, f"no table entry {name}"
    x = _magnitude_rows(dtype)
    rows, cols = x.shape
    _say(f"magnitudes {name} rows={rows}")
    if k.causal:
        y = run(x, dtype, kernel_id=k.kid, causal=True, scale=0.75, diag=cols)
        check(y, x, dtype, O.softmax_causal(x, dtype, 0.75, cols), label=name)
    else:
        y = run(x, dtype, kernel_id=k.kid)
        check(y, x, dtype, O.softmax(x, dtype), label=name)


# ------------------------------------------- the pages' worked examples

# "GPU Kernels - Implementing and optimizing Softmax", section "Per-thread
# accumulation": 10 columns over 4 threads, threads 0-1 taking three columns
# and threads 2-3 two; section "The tree reduction": those four partial maxes
# are 3.1, 7.2, 1.0, 9.5 and the row max is 9.5.  This row has exactly those
# partial maxes under that partition (the max sits in column 3, a runner-up
# 9.0 in column 7); the second row is the four partial maxes themselves.
_WORKED_ROW = [3.1, 7.2, 1.0, 9.5, 2.0, 5.0, 0.5, 9.0, 1.5, 6.0]


@pytest.mark.parametrize("stride", [10, 12])
def test_pages_worked_partition_and_tree(stride):
    row = np.array(_WORKED_ROW)
    parts = [row[t::4].max() for t in range(4)]
    assert parts == [3.1, 7.2, 1.0, 9.5]  # the fixture is the pages' partition
    x = np.full((2, stride), np.nan)
    x[0, :10] = row
    x[1, :4] = parts
    x[1, 4:10] = -np.inf
    x = W.cast(x, "f32")
    want = O.softmax(x, "f32", cols=10)
    assert np.argmax(want[0]) == 3 and abs(want[0, 3] / want[0, 7] - np.exp(0.5)) < 1e-12
    for k in _TABLE:
        if k.causal or k.dtype != W.dtype_code("f32"):
            continue
        xd = to_device(x, "f32")
        if not binding.kernel_fits(k.kid, xd.data_ptr(), xd.data_ptr(), 10, stride, W.dtype_code("f32")):
            continue
        _say(f"worked example {k.name} stride={stride}")
        y = run(x, "f32", cols=10, kernel_id=k.kid)
        check(y, x, "f32", want, cols=10, label=f"{k.name} stride={stride}")
        check_padding_untouched(y, 10, "f32", label=k.name)


# "Dissecting Memory Bandwidth & SRAM Tiling in Triton", section "Writing the
# Kernel in OpenAI Triton": a row of 6 columns read by a block of 8 lanes
# takes the mask [T, T, T, T, T, T, F, F]; the two masked lanes must add
# nothing.  Here the two columns past the row hold a huge finite value, so a
# kernel that read them would get another max and another sum.  The same
# shape is run at the level of elements (6 of 8 columns, scalar accesses) and
# of 16-byte accesses (6 of 8 accesses), through every table kernel that fits.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("unit", ["element", "access"])
def test_pages_mask_example(dtype, unit):
    mask = np.arange(8) < 6
    assert mask.tolist() == [True] * 6 + [False] * 2  # the pages' mask for n_cols 6, BLOCK 8
    vec = 16 // (4 if dtype == "f32" else 2)
    per = 1 if unit == "element" else vec
    cols, stride = 6 * per, 8 * per
    rng = np.random.default_rng([31, per])
    x = np.full((5, stride), 3.0e4)
    x[:, :cols] = 2.0 * rng.standard_normal((5, cols))
    x[1, : cols // 2] = -np.inf
    x = W.cast(x, dtype)
    want = O.softmax(x, dtype, cols=cols)
    ran = 0
    for k in _TABLE:
        if k.causal or k.dtype != W.dtype_code(dtype):
            continue
        xd = to_device(x, dtype)
        if not binding.kernel_fits(k.kid, xd.data_ptr(), xd.data_ptr(), cols, stride, W.dtype_code(dtype)):
            continue
        _say(f"mask example {k.name} cols={cols} stride={stride}")
        y = run(x, dtype, cols=cols, kernel_id=k.kid)
        check(y, x, dtype, want, cols=cols, label=f"{k.name} {unit}")
        check_padding_untouched(y, cols, dtype, label=k.name)
        ran += 1
    assert ran > 0


# ------------------------------------------------ extents beyond 4 GiB

def test_extent_beyond_4gib():
    """1,200,000 rows x 1024 fp32 (4.9 GB each way): rows past the 4 GiB mark
    must come out right, so every byte offset is 64-bit.  The input is made on
    the device by seeded torch ops (too large to stage from the host), and 64
    sampled rows, the last ones included, go back to the oracle."""
    import torch
    rows, cols = 1_200_000, 1024
    _say(f"extent beyond 4 GiB: {rows} x {cols} fp32")
    g = torch.Generator(device="cuda").manual_seed(97)
    x = torch.randn((rows, cols), generator=g, device="cuda", dtype=torch.float32) * 3.0
    y = torch.empty_like(x)
    binding.softmax_fwd(x.data_ptr(), y.data_ptr(), rows, cols, cols, W.dtype_code("f32"),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([[0, rows // 2, rows - 2, rows - 1],
                                     np.random.default_rng(98).integers(1_050_000, rows, 60)]))
    idx = torch.from_numpy(pick).to("cuda")
    xs = x.index_select(0, idx).cpu().numpy()
    ys = y.index_select(0, idx).cpu().numpy()
    assert int(pick.max()) * cols * 4 > (1 << 32)  # the check reaches past 4 GiB
    check(ys, xs, "f32", O.softmax(xs, "f32"), label="beyond 4 GiB")
    del x, y
    torch.cuda.empty_cache()


# ------------------------------------------------- line-shifted row kernels

_ROW_KERNELS = [k for k in _TABLE if k.variant in ("row", "row_pf") and k.vec_elems * (4 if k.dtype == 0 else 2) == 16]


def _at_offset(host: np.ndarray, dtype: str, off: int, fill: int):
    """A device copy of host starting `off` bytes into a buffer whose other bytes hold `fill`."""
    import torch
    esz = 4 if dtype == "f32" else 2
    n = host.size * esz
    raw = torch.full((n + 512,), fill, dtype=torch.uint8, device="cuda")
    view = raw[off:off + n].view(torch.float32 if dtype == "f32" else torch.int16).view(host.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(host).view(np.float32 if dtype == "f32" else np.int16)))
    return raw, view


@pytest.mark.parametrize("kid", [k.kid for k in _ROW_KERNELS], ids=[k.name for k in _ROW_KERNELS])
def test_line_shifted_rows(kid):
    """Row kernels move each row's accesses onto 128-byte lines when the
    workgroup has spare slots.  Here the width leaves exactly 7 spare slots,
    the pitch is an odd number of 16-byte accesses (so the rows' shifts take
    all 8 values) and input and output start at different offsets within a
    line; the output's padding and the bytes around it must stay untouched."""
    import torch
    k = _TABLE[kid]
    dtype = _DT[k.dtype]
    esz = 4 if dtype == "f32" else 2
    slots = k.lanes * k.vecs_per_lane
    nacc = slots - 7
    cols = nacc * k.vec_elems
    pitch = nacc if nacc % 2 else nacc + 1
    stride = pitch * k.vec_elems
    rows = _rows_for(k, cols)
    _say(f"line-shifted {k.name} rows={rows} cols={cols} stride={stride}")
    x = W.random_matrix(seed=300 + kid, rows=rows, cols=cols, dtype=dtype, sigma=3.0, row_stride=stride)
    x[2, : cols // 2] = W.neg_inf(dtype)
    in_raw, xd = _at_offset(x, dtype, 80, 0)
    pad = np.full_like(x, sentinel(dtype))
    out_raw, yd = _at_offset(pad, dtype, 48, 0xA5)
    out_addr = yd.data_ptr()
    shifts = {((out_addr >> 4) + r * pitch) & 7 for r in range(8)}
    assert max(shifts) == 7 and slots >= nacc + 7  # every shift value occurs and fits
    stream = torch.cuda.current_stream().cuda_stream
    code = W.dtype_code(dtype)
    if k.causal:
        diag = cols // 2 - rows // 2
        binding.softmax_fwd_causal_kernel(kid, xd.data_ptr(), out_addr, rows, cols, stride, 0.5, diag, code, stream)
    else:
        binding.softmax_fwd_kernel(kid, xd.data_ptr(), out_addr, rows, cols, stride, code, stream)
    torch.cuda.synchronize()
    y = to_host(yd, dtype)
    if k.causal:
        check(y, x, dtype, O.softmax_causal(x, dtype, 0.5, diag, cols=cols), cols=cols, label=k.name,
              keep=causal_mask(rows, cols, diag))
    else:
        check(y, x, dtype, O.softmax(x, dtype, cols=cols), cols=cols, label=k.name)
    check_padding_untouched(y, cols, dtype, label=k.name)
    around = out_raw.cpu().numpy()
    assert (around[:48] == 0xA5).all() and (around[48 + y.nbytes:] == 0xA5).all(), "bytes outside the output written"


# ------------------------------------------------- forced variant and size

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant,block,cols", [(0, 8, 32), (0, 64, 512), (0, 64, 1000), (1, 256, 2048),
                                                 (1, 512, 3000), (1, 1024, 8192), (2, 256, 70001),
                                                 (2, 1024, 4096), (3, 256, 4096), (3, 128, 1000)])
def test_forced_variant_and_size(dtype, variant, block, cols):
    """softmax_fwd_variant (a variant and a lane / workgroup size, as a width sweep
    forces them) against the oracle."""
    import torch
    _say(f"variant {variant} block {block} {dtype} cols={cols}")
    x = W.random_matrix(seed=51, rows=67, cols=cols, dtype=dtype, sigma=2.0)
    xd = to_device(x, dtype)
    out = torch.empty_like(xd)
    binding.softmax_fwd_variant(xd.data_ptr(), out.data_ptr(), 67, cols, cols, W.dtype_code(dtype), variant, block,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check(to_host(out, dtype), x, dtype, O.softmax(x, dtype), label=f"variant {variant}/{block} {dtype} {cols}")


# ------------------------- 16-bit rows kept as stored values, against widened

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kind", ["plain", "causal", "any", "causal_any"])
@pytest.mark.parametrize("cols,stride,offset", [(65536, 65536, 0), (65536 - 8, 65536, 0), (40000, 40008, 0),
                                                (8, 8, 0), (65529, 65529, 3), (40001, 40003, 1)])
def test_row16_bits_equal_the_widened_row_kernel(dtype, kind, cols, stride, offset):
    """row16 (stored 16-bit values, exponentials taken twice) gives the bits of
    the row kernel of the same shape (values widened once) on the same rows:
    ordinary, partly and wholly -inf, huge maxima (the rebase), rows starting
    inside a 128-byte line (the line-shifted launch); causal (scaled, kept
    columns only) and at any element offset (odd widths and pitches, pointers
    inside a chunk)."""
    import torch
    from gpu_util import to_device, to_host
    aligned = offset == 0 and (cols * 2) % 16 == 0 and (stride * 2) % 16 == 0
    if (kind in ("any", "causal_any")) == aligned:
        pytest.skip("alignment decides between the aligned and any-offset kernels")
    pre = {"plain": "", "causal": "causal_", "any": "any_", "causal_any": "causal_any_"}[kind]
    table = {k.name: k for k in _TABLE}
    a = table[f"{pre}row_{dtype}_w16_v8"]
    b = table[f"{pre}row16_{dtype}_w16_v8"]
    rows = 37
    causal = kind.startswith("causal")
    diag = cols - rows - 5
    _say(f"row16 vs row {kind} {dtype} rows={rows} cols={cols} stride={stride} offset={offset}")
    x = W.random_matrix(seed=cols + stride, rows=rows, cols=cols, dtype=dtype, sigma=3.0, row_stride=stride)
    x[1, : cols // 2] = W.neg_inf(dtype)
    x[2, :cols] = W.neg_inf(dtype)
    top = W.cast(np.array([6.0e4 if dtype == "f16" else 3.0e38]), dtype)[0]
    x[3, : max(1, cols // 7)] = top
    x[4, :cols] = W.cast(np.linspace(-3.0e4, -2.9e4, cols), dtype)
    code = W.dtype_code(dtype)
    flat = np.zeros(offset + x.size, dtype=x.dtype)
    flat[offset:] = x.ravel()
    xd = to_device(flat, dtype)
    outs = []
    for k in (a, b):
        yd = torch.zeros_like(xd)
        pi, po = xd.data_ptr() + 2 * offset, yd.data_ptr() + 2 * offset
        stream = torch.cuda.current_stream().cuda_stream
        if causal:
            binding.softmax_fwd_causal_kernel(k.kid, pi, po, rows, cols, stride, 0.5, diag, code, stream)
        else:
            binding.softmax_fwd_kernel(k.kid, pi, po, rows, cols, stride, code, stream)
        torch.cuda.synchronize()
        outs.append(to_host(yd, dtype)[offset:].reshape(rows, stride))
    assert np.array_equal(outs[0], outs[1]), "bits differ"
    if causal:
        ref = O.softmax_causal(x, dtype, 0.5, diag, cols=cols)
        check(outs[1], x, dtype, ref, cols=cols, label=f"row16 {kind} {dtype} {cols}",
              keep=causal_mask(rows, cols, diag))
    else:
        check(outs[1], x, dtype, O.softmax(x, dtype, cols=cols), cols=cols, label=f"row16 {kind} {dtype} {cols}")

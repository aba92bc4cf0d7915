"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments before any HIP call.  Nothing here launches work."""
import ctypes
import os
import re

import pytest

from row_wise_softmax_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "row_wise_softmax.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


@pytest.fixture(scope="module")
def lib():
    path = binding.library_path()
    if not os.path.exists(path):
        pytest.fail(f"HIP library not built: {path}")
    return binding._load()


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for want in ("softmax_fwd", "softmax_fwd_kernel", "softmax_select", "softmax_num_kernels",
                 "softmax_fwd_causal", "softmax_fwd_causal_kernel", "softmax_select_causal",
                 "softmax_kernel_info", "softmax_kernel_name", "softmax_kernel_fits",
                 "softmax_status_string", "softmax_version", "softmax_bench_copy"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(binding.library_path())
    for name in _declared_functions():
        assert hasattr(raw, name), f"{name} declared in the header but not exported"


def test_library_is_built_for_gfx950():
    blob = open(binding.library_path(), "rb").read()
    assert b"gfx950" in blob


def test_version_and_status_strings(lib):
    assert "gfx950" in binding.version()
    for st in range(9):
        assert lib.softmax_status_string(st) != b"unknown status"
    assert lib.softmax_status_string(99) == b"unknown status"


def _fwd(lib, in_ptr, out_ptr, rows, cols, stride, dtype):
    return lib.softmax_fwd(in_ptr, out_ptr, rows, cols, stride, dtype, None)


# Host addresses only: every case in this file is rejected (or is empty)
# before the library touches the device, so no address is ever dereferenced
# and no kernel is launched.
A, B = 0x100000, 0x900000


@pytest.mark.parametrize("args,status", [
    ((A, B, 4, 8, 8, 7), 3),            # bad dtype
    ((A, B, 4, 8, 8, -1), 3),
    ((A, B, -1, 8, 8, 0), 2),           # negative rows
    ((A, B, 4, -8, 8, 0), 2),           # negative cols
    ((A, B, 4, 8, 7, 0), 2),            # row_stride < cols
    ((A, B, 4, 2**30 + 1, 2**31, 0), 2),  # cols > 2^30
    ((A, B, 2**40, 2**30, 2**30, 0), 2),  # byte extent past INT64_MAX
    ((0, B, 4, 8, 8, 0), 1),            # null input
    ((A, 0, 4, 8, 8, 0), 1),            # null output
    ((A, A + 16, 4, 8, 8, 0), 4),       # partial overlap
    ((A + 16, A, 4, 8, 8, 1), 4),
    ((A, B, 0, 8, 8, 0), 0),            # empty: nothing to do
    ((A, B, 4, 0, 8, 0), 0),
    ((0, 0, 0, 0, 0, 2), 0),
])
def test_argument_errors_before_any_launch(lib, args, status):
    assert _fwd(lib, *args) == status


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan"), 3e38])
def test_causal_bad_scale(lib, scale):
    assert lib.softmax_fwd_causal(A, B, 4, 8, 8, scale, 0, 0, None) == 7


def test_causal_argument_errors(lib):
    assert lib.softmax_fwd_causal(A, B, 4, 8, 7, 1.0, 0, 0, None) == 2      # row_stride < cols
    assert lib.softmax_fwd_causal(0, B, 4, 8, 8, 1.0, 0, 0, None) == 1      # null
    assert lib.softmax_fwd_causal(A, B, 4, 8, 8, 1.0, 0, 9, None) == 3      # dtype
    assert lib.softmax_fwd_causal(A, A + 4, 4, 8, 8, 1.0, 0, 0, None) == 4  # overlap
    assert lib.softmax_fwd_causal(A, B, 0, 8, 8, 1.0, 0, 0, None) == 0      # empty: nothing launched


def test_plain_and_causal_entries_are_not_interchangeable(lib):
    table = binding.kernel_table()
    plain = next(k for k in table if k.dtype == 0 and not k.causal and k.variant == "online")
    causal = next(k for k in table if k.dtype == 0 and k.causal and k.variant == "online")
    assert lib.softmax_fwd_kernel(causal.kid, A, B, 4, 8, 8, 0, None) == 5
    assert lib.softmax_fwd_causal_kernel(plain.kid, A, B, 4, 8, 8, 1.0, 0, 0, None) == 5


def test_forced_kernel_errors(lib):
    n = lib.softmax_num_kernels()
    assert n > 100
    assert lib.softmax_fwd_kernel(-1, A, B, 4, 8, 8, 0, None) == 5
    assert lib.softmax_fwd_kernel(n, A, B, 4, 8, 8, 0, None) == 5
    table = binding.kernel_table()
    f16 = next(k for k in table if k.dtype == 1 and not k.causal)
    assert lib.softmax_fwd_kernel(f16.kid, A, B, 4, 8, 8, 0, None) == 5  # wrong dtype
    narrow = next(k for k in table if k.dtype == 0 and k.max_cols == 4 and not k.causal)
    assert lib.softmax_fwd_kernel(narrow.kid, A, B, 4, 8, 8, 0, None) == 5  # too wide
    vec = next(k for k in table if k.dtype == 0 and k.vec_elems == 4 and not k.causal)
    assert lib.softmax_fwd_kernel(vec.kid, A + 4, B, 4, 8, 8, 0, None) == 5  # misaligned


def test_kernel_table_is_consistent(lib):
    table = binding.kernel_table()
    names = [k.name for k in table]
    assert len(set(names)) == len(names)
    for k in table:
        assert k.variant in ("packed", "row", "row_pf", "online", "row16")
        if k.variant == "row16":  # 16-bit rows kept as stored: 16-bit types only
            assert k.dtype in (1, 2) and k.vec_elems == 8
        assert k.name.startswith("causal_") == k.causal
        assert k.dtype in (0, 1, 2)
        if k.variant == "online":
            assert k.max_cols == -1
        elif "any_" in k.name:  # rows at any element offset give vec - 1 slots to the offset
            assert k.max_cols == k.lanes * k.vecs_per_lane * k.vec_elems - (k.vec_elems - 1)
        else:
            assert k.max_cols == k.lanes * k.vecs_per_lane * k.vec_elems
        if k.vec_elems > 1:
            assert k.vec_elems * (4 if k.dtype == 0 else 2) == 16
    # every dtype has the scalar (any-alignment) path, plain and causal
    for dt in (0, 1, 2):
        for c in (False, True):
            assert any(k.dtype == dt and k.vec_elems == 1 and k.causal == c for k in table)


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("cols", [1, 3, 8, 32, 64, 100, 256, 1000, 1001, 2048, 3000, 4096, 8192,
                                  16384, 32768, 65536, 131072, 1 << 18])
@pytest.mark.parametrize("causal", [False, True])
def test_dispatch_always_picks_a_fitting_kernel(lib, dtype, cols, causal):
    kid = binding.softmax_select(A, B, cols, cols, dtype, rows=4, causal=causal)
    esz = 4 if dtype == 0 else 2
    if kid == binding.SPLIT_KERNEL:  # few, very wide rows out of place: softmax_fwd's own split
        assert not causal and cols * esz >= 128 << 10
        kid = binding.softmax_select(A, A, cols, cols, dtype, rows=4)  # in place takes the table
    assert binding.kernel_fits(kid, A, B, cols, cols, dtype)
    info = binding.kernel_table()[kid]
    assert info.causal == causal
    # 16-byte accesses whatever the width: aligned rows on the aligned kernels,
    # other widths on the any-alignment ones
    assert info.vec_elems * esz == 16
    assert ("any_" in info.name) == ((cols * esz) % 16 != 0)
    # pointers one 16-bit element past a chunk boundary, at the same offset:
    # element-aligned for 16-bit types (any-alignment kernels), not for fp32 (scalar)
    kid2 = binding.softmax_select(A + 2, B + 2, cols, cols, dtype, rows=4, causal=causal)
    k2 = binding.kernel_table()[kid2]
    assert k2.causal == causal
    assert (k2.vec_elems == 1) if esz == 4 else ("any_" in k2.name and k2.vec_elems == 8)
    # input and output at different offsets in their chunks: the scalar path
    kid3 = binding.softmax_select(A + 4, B + 8, cols, cols, dtype, rows=4, causal=causal)
    assert binding.kernel_table()[kid3].vec_elems == 1


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_causal_dispatch_takes_the_plain_shapes(lib, dtype):
    """Across the sweep's widths the scaled, masked softmax runs the same
    kernel shape as the plain one: the causal table holds every such pick."""
    table = binding.kernel_table()
    esz = 4 if dtype == 0 else 2
    for cols in (8, 32, 64, 128, 256, 512, 1000, 1024, 2048, 3000, 4096, 8192, 16384):
        if (cols * esz) % 16:
            continue
        plain = table[binding.softmax_select(A, B, cols, cols, dtype, rows=4)].name
        masked = table[binding.softmax_select(A, B, cols, cols, dtype, rows=4, causal=True)].name
        assert masked == "causal_" + plain, (cols, plain, masked)


def test_bench_copy_argument_errors(lib):
    assert lib.softmax_bench_copy(A, B, 15, None) == 2
    assert lib.softmax_bench_copy(A + 4, B, 16, None) == 2
    assert lib.softmax_bench_copy(0, B, 16, None) == 1
    assert lib.softmax_bench_copy(A, A + 16, 64, None) == 4
    assert lib.softmax_bench_copy(A, B, 0, None) == 0


def test_bench_stream_argument_errors(lib):
    st = lib.softmax_bench_stream
    assert st(A, B, 64, 3, None) == 5       # unknown mode
    assert st(A, B, 15, 1, None) == 2
    assert st(A + 4, B, 16, 1, None) == 2   # misaligned source of the read stream
    assert st(0, B, 16, 1, None) == 1
    assert st(A, 0, 16, 2, None) == 1
    assert st(A, A + 16, 64, 0, None) == 4  # mode 0 is the copy, with its overlap check
    assert st(A, B, 0, 2, None) == 0


def test_unfused_baseline_argument_errors(lib):
    ws = binding.unfused_workspace_bytes(4, 8, 0)
    assert ws > 2 * 4 * 8 * 4
    assert binding.unfused_workspace_bytes(-1, 8, 0) == -1
    assert binding.unfused_workspace_bytes(4, 8, 9) == -1
    W = 0x4000000  # host address, 256-byte aligned, never dereferenced
    assert lib.softmax_unfused_5op(A, B, 4, 8, 8, 0, W, ws - 1, None) == 2      # short workspace
    assert lib.softmax_unfused_5op(A + 4, B, 4, 8, 8, 0, W, ws, None) == 2      # misaligned input
    assert lib.softmax_unfused_5op(A, B, 4, 7, 7, 0, W, ws, None) == 2          # not whole 16-byte accesses
    assert lib.softmax_unfused_5op(A, B, 4, 8, 8, 0, W + 16, ws, None) == 2     # workspace not 256-aligned
    assert lib.softmax_unfused_5op(A, B, 4, 8, 8, 0, 0, ws, None) == 1          # null workspace
    assert lib.softmax_unfused_5op(A, A + 16, 4, 8, 8, 0, W, ws, None) == 4     # in/out overlap
    assert lib.softmax_unfused_5op(A, B, 4, 8, 8, 0, A, ws, None) == 4          # workspace overlaps input
    assert lib.softmax_unfused_5op(A, B, 4, 8, 8, 5, W, ws, None) == 3          # dtype
    assert lib.softmax_unfused_5op(A, B, 0, 8, 8, 0, W, ws, None) == 0          # empty


def test_split_argument_errors(lib):
    ws = binding.split_workspace_bytes(4, 1 << 16, 0)
    assert ws >= 4 * ((1 << 16) // 2048) * 8 and ws % 256 == 0
    assert binding.split_workspace_bytes(-1, 8, 0) == -1
    assert binding.split_workspace_bytes(4, 8, 7) == -1
    Wk = 0x40000000  # host address, 256-byte aligned, never dereferenced
    n = 1 << 16
    # force = 1 (split): every case below is rejected before any launch
    assert lib.softmax_fwd_split(A, A + 4 * n * 4 + 256, 4, n, n, 0, 0, ws, 1, None) == 1        # null workspace
    assert lib.softmax_fwd_split(A, A + 4 * n * 4 + 256, 4, n, n, 0, Wk, ws - 256, 1, None) == 2  # short
    assert lib.softmax_fwd_split(A, A + 4 * n * 4 + 256, 4, n, n, 0, Wk + 8, ws, 1, None) == 2   # misaligned
    assert lib.softmax_fwd_split(A, A + 4 * n * 4 + 256, 4, n, n, 0, A, ws, 1, None) == 4        # overlaps input
    assert lib.softmax_fwd_split(A, A + 4 * n * 4 + 256, 4, n, n, 0, Wk, ws, 2, None) == 5       # bad force
    assert lib.softmax_fwd_split(A, A + 16, 4, n, n, 0, Wk, ws, 1, None) == 4                    # in/out overlap
    assert lib.softmax_fwd_split(A, B, 0, n, n, 0, 0, 0, 1, None) == 0                           # empty


def test_attention_argument_errors(lib):
    a = lambda *args: lib.attention_fwd(*args, None)  # noqa: E731
    Q, K, V, O = 0x100000, 0x200000, 0x300000, 0x400000
    assert a(Q, K, V, O, 1, 1, 64, 64, 64, 0.125, 1, 0) == 3       # fp32 not supported
    assert a(Q, K, V, O, 1, 1, 64, 64, 96, 0.125, 1, 1) == 2       # head_dim
    assert a(Q, K, V, O, 1, 1, 64, 64, 64, 0.0, 1, 1) == 7         # scale
    assert a(Q, K, V, O, 1, 1, 64, 64, 64, 0.125, 2, 1) == 2       # causal flag
    assert a(0, K, V, O, 1, 1, 64, 64, 64, 0.125, 1, 1) == 1       # null
    assert a(Q + 2, K, V, O, 1, 1, 64, 64, 64, 0.125, 1, 1) == 2   # misaligned
    assert a(Q, K, V, Q + 64, 1, 1, 64, 64, 64, 0.125, 1, 1) == 4  # o overlaps q
    assert a(Q, K, V, O, 300, 300, 64, 64, 64, 0.125, 1, 1) == 2   # batch * heads > 65535
    assert a(Q, K, V, O, 1, 1, 64, 1 << 23, 128, 0.125, 1, 1) == 2  # K of one head >= 2 GiB
    assert a(Q, K, V, O, 1, 1, 64, 1 << 24, 64, 0.125, 1, 1) == 2   # (same bytes at head_dim 64)
    assert a(Q, K, V, O, 0, 1, 64, 64, 64, 0.125, 1, 1) == 0       # empty


# The width dispatch's picks at the BASELINE configs and the sweep widths, at
# those workloads' row counts (the "pick" column of the measured sweep); a
# change to the rule must change this table knowingly.
_PICKS = {
    "c1": "rowpf_f32_w2_v2", "c2": "rowpf_f32_w4_v2", "c3": "row_f16_w4_v2", "c4": "row_f32_w8_v2",
    "c5_bf16_32": "packed_bf16_l4_v1_g2", "c5_bf16_64": "packed_bf16_l8_v1_g2", "c5_bf16_128": "packed_bf16_l16_v1_g2",
    "c5_bf16_256": "packed_bf16_l32_v1_g2", "c5_bf16_512": "packed_bf16_l64_v1_g2",
    "c5_bf16_1000": "packed_bf16_l64_v2_g1", "c5_bf16_1024": "packed_bf16_l64_v2_g1", "c5_bf16_2048": "row_bf16_w2_v2",
    "c5_bf16_3000": "row_bf16_w4_v2", "c5_bf16_4096": "row_bf16_w4_v2", "c5_bf16_8192": "row_bf16_w8_v2",
    "c5_bf16_16384": "row_bf16_w16_v2",
    "c5_f32_32": "packed_f32_l8_v1_g2", "c5_f32_64": "packed_f32_l16_v1_g2", "c5_f32_128": "packed_f32_l32_v1_g2",
    "c5_f32_256": "packed_f32_l64_v1_g2", "c5_f32_512": "packed_f32_l64_v2_g1", "c5_f32_1000": "row_f32_w4_v2",
    "c5_f32_1024": "row_f32_w4_v2", "c5_f32_2048": "row_f32_w8_v2", "c5_f32_3000": "row_f32_w8_v2",
    "c5_f32_4096": "row_f32_w8_v2", "c5_f32_8192": "row_f32_w16_v2", "c5_f32_16384": "row_f32_w4_v16",
}


@pytest.mark.parametrize("key", sorted(_PICKS))
def test_dispatch_picks_the_measured_shapes(lib, key):
    from row_wise_softmax_amd import workloads as W
    wl = W.WORKLOADS[key]
    code = W.dtype_code(wl.dtype)
    a, b = 1 << 40, 1 << 41  # far apart: no overlap at any of these sizes (never dereferenced)
    kid = binding.softmax_select(a, b, wl.cols, wl.cols, code, rows=wl.rows)
    assert binding.kernel_table()[kid].name == _PICKS[key]


def test_few_rows_take_the_persistent_twin(lib):
    """Row shapes whose rows x waves fill the chip's 8192 wave slots at most twice
    run the persistent twin of the same shape, plain and causal."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, rows, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=rows,
                                                                               causal=causal)].name
    assert pick(4096, 2, 4096) == "rowpf_bf16_w4_v2" and pick(4096, 2, 4097) == "row_bf16_w4_v2"
    assert pick(8192, 2, 2048) == "rowpf_bf16_w8_v2" and pick(8192, 2, 2561) == "row_bf16_w8_v2"
    assert pick(2048, 0, 2048, causal=True) == "causal_rowpf_f32_w4_v2"
    assert pick(16384, 0, 16) == "row_f32_w4_v16"  # rows past the register-resident two-access shapes keep theirs


def test_few_16bit_rows_take_one_access_on_twice_the_waves(lib):
    """16-bit jobs whose rows, on twice the twin's waves, fit one round of the
    8192 wave slots take the persistent shape of one access per lane, plain and
    causal; fp32 keeps the twin."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, rows, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=rows,
                                                                               causal=causal)].name
    assert pick(2048, 2, 2048) == "rowpf_bf16_w4_v1" and pick(2048, 2, 2049) == "rowpf_bf16_w2_v2"
    assert pick(4096, 1, 1024) == "rowpf_f16_w8_v1" and pick(4096, 1, 1025) == "rowpf_f16_w4_v2"
    assert pick(8192, 2, 512) == "rowpf_bf16_w16_v1" and pick(8192, 2, 513) == "rowpf_bf16_w8_v2"
    assert pick(16384, 2, 256) == "rowpf_bf16_w16_v2"      # no thirty-two-wave shape
    assert pick(2048, 0, 512) == "rowpf_f32_w4_v2"         # fp32 keeps the twin
    assert pick(2048, 2, 2048, causal=True) == "causal_rowpf_bf16_w4_v1"
    assert pick(4096, 2, 1024, causal=True) == "causal_rowpf_bf16_w8_v1"
    assert pick(4097, 2, 64) == "any_rowpf_bf16_w4_v3"    # three accesses: the twin as it is


def test_rows_just_past_a_power_of_two_take_three_accesses(lib):
    """Aligned rows that fill little of the two-access shape's slots take three
    accesses on half the waves, by the measured fill lines (16-bit: 75% on
    sixteen waves, 70% on eight, 62% on four; fp32: 62% on sixteen, 53% on
    eight); fuller rows, jobs of few rows and causal rows keep two accesses."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, rows, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=rows,
                                                                               causal=causal)].name
    assert pick(8800, 2, 11363) == "row_bf16_w8_v3"          # 1100 chunks of 2048 slots
    assert pick(12000, 2, 8333) == "row_bf16_w8_v3"          # 1500 chunks of 2048
    assert pick(8 * 1536, 2, 8000) == "row_bf16_w8_v3"       # 1536: the last inside 75%
    assert pick(8 * 1537, 2, 8000) == "row_bf16_w16_v2"
    assert pick(4160, 2, 24038) == "row_bf16_w4_v3"          # 520 chunks of 1024
    assert pick(8 * 716, 1, 20000) == "row_f16_w4_v3" and pick(8 * 717, 1, 20000) == "row_f16_w8_v2"
    assert pick(2400, 2, 41666) == "row_bf16_w2_v3"          # 300 chunks of 512
    assert pick(8 * 317, 2, 40000) == "row_bf16_w2_v3" and pick(8 * 318, 2, 40000) == "row_bf16_w4_v2"
    assert pick(6000, 2, 16666) == "row_bf16_w8_v2"          # 750 chunks: full enough
    assert pick(4400, 0, 11363) == "row_f32_w8_v3"           # 1100 chunks of 2048
    assert pick(4 * 1269, 0, 8000) == "row_f32_w8_v3" and pick(4 * 1270, 0, 8000) == "row_f32_w16_v2"
    assert pick(2080, 0, 24038) == "row_f32_w4_v3"           # 520 chunks of 1024
    assert pick(4 * 542, 0, 24000) == "row_f32_w4_v3" and pick(4 * 543, 0, 24000) == "row_f32_w8_v2"
    assert pick(1200, 0, 41666) == "row_f32_w4_v2"           # fp32 on four waves keeps two
    # few rows: the two-access shape's persistent twin, as before
    assert pick(8800, 2, 1024) == "rowpf_bf16_w16_v2" and pick(8800, 2, 2048) == "row_bf16_w16_v2"
    assert pick(8800, 2, 2049) == "row_bf16_w8_v3"
    assert pick(8800, 2, 11363, causal=True) == "causal_row_bf16_w16_v2"  # no causal three-access entry


def test_full_fp32_rows_of_many_rows_take_twice_the_waves(lib):
    """fp32 rows of exactly 256 or 512 16-byte accesses in jobs of 16384 rows
    or more take twice the waves of two accesses; fewer rows, other widths,
    16-bit rows and causal rows keep the general shape."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, rows, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=rows,
                                                                               causal=causal)].name
    assert pick(1024, 0, 16384) == "row_f32_w4_v2" and pick(1024, 0, 16383) == "row_f32_w2_v2"
    assert pick(2048, 0, 16384) == "row_f32_w8_v2" and pick(2048, 0, 16383) == "row_f32_w4_v2"
    assert pick(2048, 0, 4096) == "rowpf_f32_w4_v2"          # c2's shape: the persistent twin
    assert pick(4096, 0, 16384) == "row_f32_w8_v2"           # 1024 accesses keep eight waves
    assert pick(2044, 0, 16384) == "row_f32_w4_v2"           # 511 accesses: not full
    assert pick(4096, 2, 24414) == "row_bf16_w4_v2"          # 16-bit keeps its shape
    assert pick(2048, 0, 16384, causal=True) == "causal_row_f32_w4_v2"


def test_jobs_just_past_two_rounds(lib):
    """16-bit jobs just past the persistent twin's two rounds take a quarter of
    the waves with eight accesses each, plain, while the job fits one round of
    that shape (1280 rows of 1537..2048 accesses, 2560 rows of 769..1024);
    fp32 rows on sixteen waves keep the twin up to 1280 rows."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, rows, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=rows,
                                                                               causal=causal)].name
    assert pick(16384, 2, 1024) == "rowpf_bf16_w16_v2"
    assert pick(16384, 2, 1025) == "row_bf16_w4_v8" and pick(16384, 1, 1280) == "row_f16_w4_v8"
    assert pick(16384, 2, 1281) == "row_bf16_w16_v2"
    assert pick(8 * 1537, 2, 1100) == "row_bf16_w4_v8" and pick(8 * 1536, 2, 1100) == "row_bf16_w16_v2"
    assert pick(8192, 2, 2048) == "rowpf_bf16_w8_v2"
    assert pick(8192, 2, 2049) == "row_bf16_w2_v8" and pick(8192, 2, 2560) == "row_bf16_w2_v8"
    assert pick(8192, 2, 2561) == "row_bf16_w8_v2" and pick(8 * 768, 2, 2200) == "row_bf16_w8_v2"
    assert pick(16384, 2, 1100, causal=True) == "causal_row_bf16_w16_v2"
    assert pick(8192, 0, 1024) == "rowpf_f32_w16_v2" and pick(8192, 0, 1280) == "rowpf_f32_w16_v2"
    assert pick(8192, 0, 1281) == "row_f32_w16_v2" and pick(8192, 0, 1100, causal=True) == "causal_row_f32_w16_v2"
    assert pick(4096, 0, 2049) == "row_f32_w8_v2"             # eight waves: the twin up to two rounds


def test_quarter_wave_shapes_keep_five_waves_per_simd():
    """The one-round limits of the rule above assume the 16-bit row kernels of
    four and two waves with eight accesses each run five waves per SIMD; the
    committed resource table (from the compiler's remarks) must agree."""
    text = open(os.path.join(os.path.dirname(__file__), "..", "profiles", "kernel_resources.md")).read()
    for dt in ("F16", "BF16"):
        for w in (4, 2):
            line = next(l for l in text.splitlines()
                        if f"`rws::softmax_row<rws::{dt}, 8, {w}, 8, false, false, false>`" in l)
            assert line.rstrip(" |").split("|")[-1].strip() == "5", line


def test_rows_past_2048_chunks_take_sixteen_waves_of_three(lib):
    """Aligned rows of 2049..3072 16-byte accesses take sixteen waves of three,
    plain, both element sizes; wider rows keep their shapes, and so do causal
    rows (no such causal entry).  16-bit rows past 75% of sixteen waves of two
    and at most 2000 accesses, in jobs of 1281..3072 rows, take eight waves of
    four, not their persistent twin."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, rows, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=rows,
                                                                               causal=causal)].name
    assert pick(20000, 2, 5000) == "row_bf16_w16_v3" and pick(8 * 3072, 1, 4000) == "row_f16_w16_v3"
    assert pick(8 * 3073, 2, 4000) == "row_bf16_w16_v4"
    assert pick(10000, 0, 5000) == "row_f32_w16_v3" and pick(4 * 3072, 0, 5000) == "row_f32_w16_v3"
    assert pick(4 * 3073, 0, 5000) == "row_f32_w4_v16" and pick(16384, 0, 3051) == "row_f32_w4_v16"
    assert pick(20000, 2, 5000, causal=True) == "causal_row_bf16_w16_v4"
    assert pick(10000, 0, 5000, causal=True) == "causal_row_f32_w4_v16"
    assert pick(15600, 2, 1602) == "row_bf16_w8_v4" and pick(8 * 1537, 1, 3072) == "row_f16_w8_v4"
    assert pick(8 * 2000, 2, 1281) == "row_bf16_w8_v4" and pick(8 * 2000, 2, 1280) == "row_bf16_w4_v8"
    assert pick(15600, 2, 3073) == "row_bf16_w16_v2" and pick(15600, 2, 1024) == "rowpf_bf16_w16_v2"
    assert pick(8 * 2001, 2, 2000) == "row_bf16_w16_v2" and pick(16384, 2, 2000) == "row_bf16_w16_v2"
    assert pick(8 * 1536, 2, 1500) == "row_bf16_w16_v2"   # inside 75%: sixteen waves of two
    assert pick(15600, 2, 1602, causal=True) == "causal_row_bf16_w16_v2"
    assert pick(7800, 0, 1602) == "row_f32_w16_v2"        # fp32 keeps sixteen waves of two


def test_few_very_wide_rows_split_through_the_output(lib):
    """softmax_fwd splits few, very wide rows out of place on the 16-byte path,
    by the measured (row bytes, most rows) lines; anything else takes the
    kernel table."""
    a, b = 1 << 40, 1 << 41
    S = binding.SPLIT_KERNEL

    def sel(cols, code, rows, x=a, y=b, stride=None, causal=False):
        return binding.softmax_select(x, y, cols, stride or cols, code, rows=rows, causal=causal)

    # fp32: >= 2 MiB rows up to 192 rows, >= 1 MiB up to 128, past 256 KiB (the two-pass kernel's
    # widths) up to 64, >= 224 KiB up to 32, >= 192 KiB up to 16
    assert sel(1 << 20, 0, 192) == S and sel(1 << 20, 0, 193) != S
    assert sel(1 << 18, 0, 128) == S and sel(1 << 18, 0, 129) != S
    assert sel(1 << 17, 0, 1) == S and sel(1 << 17, 0, 64) == S and sel(1 << 17, 0, 65) != S
    assert sel((1 << 16) + 4, 0, 64) == S and sel((1 << 16) + 4, 0, 65) != S and sel(128256, 0, 64) == S
    assert sel(1 << 16, 0, 32) == S and sel(1 << 16, 0, 33) != S
    assert sel(57344, 0, 32) == S and sel(57344, 0, 33) != S
    assert sel(49152, 0, 16) == S and sel(49152, 0, 17) != S and sel(49152 - 4, 0, 8) != S
    # fp16 / bf16: >= 2 MiB up to 256, >= 1 MiB up to 192, >= 512 KiB up to 128, >= 192 KiB up to 64,
    # >= 128 KiB up to 16
    for code in (1, 2):
        assert sel(1 << 20, code, 256) == S and sel(1 << 20, code, 257) != S
        assert sel(1 << 19, code, 192) == S and sel(1 << 19, code, 193) != S
        assert sel(1 << 18, code, 128) == S and sel(1 << 18, code, 129) != S
        assert sel(1 << 17, code, 64) == S and sel(1 << 17, code, 65) != S
        assert sel(98304, code, 64) == S and sel(98304, code, 65) != S
        assert sel(65536, code, 16) == S and sel(65536, code, 17) != S
        assert sel(65536 - 8, code, 8) != S  # below 128 KiB: one workgroup per row
    assert sel((1 << 17) + 4, 0, 3, stride=(1 << 17) + 8) == S          # ragged last tile, padded stride
    assert sel(1 << 17, 0, 8, y=a) != S                                 # in place
    assert sel(1 << 17, 0, 8, x=a + 4, y=b + 4) != S                    # not on the 16-byte path
    assert sel(1 << 17, 0, 8, stride=(1 << 17) + 1) != S                # row pitch not a 16-byte multiple
    assert sel(1 << 17, 0, 8, causal=True) != S                         # the causal form never splits


def test_any_alignment_dispatch(lib):
    """Rows at any element offset take the any-alignment entries of the width rule
    on the chunks a row can touch, ceil((cols + vec - 1) / vec); just past a power of
    two, half the waves with three accesses each, and sixteen waves for wide rows
    that would leave a quarter of the slots idle."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()

    def pick(cols, code, rows=50000, x=a, y=b, causal=False):
        return table[binding.softmax_select(x, y, cols, cols, code, rows=rows, causal=causal)].name

    assert pick(1001, 2) == "any_packed_bf16_l64_v2_g1" and pick(33, 2) == "any_packed_bf16_l8_v1_g2"
    assert pick(1001, 0) == "any_row_f32_w4_v2"
    assert pick(4089, 2) == "any_row_bf16_w4_v2"      # 512 chunks: the aligned shape
    assert pick(4097, 2) == "any_row_bf16_w4_v3"      # 513 chunks
    assert pick(2049, 0) == "any_row_f32_w4_v3" and pick(4097, 0) == "any_row_f32_w8_v3"
    assert pick(16385, 2) == "any_row_bf16_w16_v3" and pick(32001, 2) == "any_row_bf16_w8_v8"
    assert pick(50257, 2) == "any_row16_bf16_w8_v16"
    assert pick(4097, 2, rows=64) == "any_rowpf_bf16_w4_v3"  # few rows: the persistent twin
    assert pick(4097, 2, causal=True) == "causal_any_row_bf16_w4_v3"
    assert pick(4096, 2, x=a + 2, y=b + 2) == "any_row_bf16_w4_v3"  # aligned width, pointers inside a chunk
    assert pick(4096, 2) == "row_bf16_w4_v2"


def test_wide_16bit_rows_take_sixteen_waves(lib):
    """16-bit rows past 16384 columns: sixteen waves of three up to 3072
    chunks, of four up to 4096 (past that the stored-value kernel, tested on
    its own); causal rows sixteen waves of four; fp32 keeps four or eight waves
    of sixteen past 3072 chunks."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    pick = lambda cols, code, causal=False: table[binding.softmax_select(a, b, cols, cols, code, rows=2000,
                                                                        causal=causal)].name
    assert pick(24576, 2) == "row_bf16_w16_v3" and pick(32000, 1) == "row_f16_w16_v4"
    assert pick(32000, 2, causal=True) == "causal_row_bf16_w16_v4"
    assert pick(65536, 2, causal=True) == "causal_row16_bf16_w8_v16"
    assert pick(50304, 2, causal=True) == "causal_row16_bf16_w8_v16"
    assert pick(16384, 2) == "row_bf16_w16_v2"  # 2048 chunks: the two-access rule
    assert pick(32000, 0) == "row_f32_w8_v16" and pick(16384, 0) == "row_f32_w4_v16"


def test_wide_16bit_rows_keep_stored_values(lib):
    """16-bit rows of 4097..24576 chunks keep their stored values in registers
    (row16): eight waves of 12, 16, 20 accesses up to 6144, 8192, 10240 chunks,
    sixteen waves of 12, 16, 20, 24 up to 24576 (causal and any-offset rows up
    to 16384); wider rows take the online kernel."""
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()

    def pick(cols, code, rows=2000, x=a, y=b, causal=False):
        return table[binding.softmax_select(x, y, cols, cols, code, rows=rows, causal=causal)].name

    assert pick(32768, 2) == "row_bf16_w16_v4" and pick(32776, 2) == "row16_bf16_w8_v12"
    assert pick(49152, 1) == "row16_f16_w8_v12" and pick(49160, 1) == "row16_f16_w8_v16"
    assert pick(50304, 2) == "row16_bf16_w8_v16" and pick(65536, 2) == "row16_bf16_w8_v16"
    assert pick(81920, 2) == "row16_bf16_w8_v20" and pick(81928, 2) == "row16_bf16_w16_v12"
    assert pick(128256, 2) == "row16_bf16_w16_v16" and pick(151936, 2) == "row16_bf16_w16_v20"
    assert pick(196608, 1) == "row16_f16_w16_v24" and pick(196616, 1) == "online_f16_vec_w16_v2"
    assert pick(128256, 2, causal=True) == "causal_row16_bf16_w16_v16"
    assert pick(128256, 2, x=a + 2, y=b + 2) == "any_row16_bf16_w16_v16"
    assert pick(50257, 2) == "any_row16_bf16_w8_v16" and pick(65535, 1) == "any_row16_f16_w8_v20"
    # masked forms stop at 16384 chunks (131072 columns); plain rows go on to 24576
    assert pick(151936, 2, causal=True) == "causal_online_bf16_vec_w16_v2"
    assert pick(151937, 2) == "any_online_bf16_w16_v4"
    assert pick(50000, 0) == "row_f32_w16_v16"  # fp32 keeps its rule


def test_ragged_rule_follows_the_row_count(lib):
    """Ragged rows of 129..255 accesses: two waves of two accesses, except fp32
    rows of 240 accesses or more from 8192 rows on (four waves of two), and
    16-bit rows of more than 250 accesses past 8192 rows (four waves of one);
    up to 8192 rows the two-wave shape runs as its persistent twin, and 16-bit
    jobs of at most 2048 rows take four waves of one (the one-round rule)."""
    a, b = 1 << 40, 1 << 41
    names = lambda cols, code, rows: binding.kernel_table()[binding.softmax_select(a, b, cols, cols, code,
                                                                                      rows=rows)].name
    assert names(1000, 0, 8191) == "rowpf_f32_w2_v2" and names(1000, 0, 8192) == "row_f32_w4_v2"
    assert names(956, 0, 100000) == "row_f32_w2_v2"  # 239 accesses
    assert names(1000, 0, 4096) == "rowpf_f32_w2_v2" and names(600, 0, 100000) == "row_f32_w2_v2"
    assert names(2000, 2, 2048) == "rowpf_bf16_w4_v1" and names(2000, 2, 2049) == "rowpf_bf16_w2_v2"
    assert names(2000, 2, 100000) == "row_bf16_w2_v2" and names(2008, 2, 100000) == "row_bf16_w4_v1"
    assert names(2008, 2, 8192) == "rowpf_bf16_w2_v2" and names(2008, 1, 8193) == "row_f16_w4_v1"
    assert names(2048, 2, 100000) == "row_bf16_w2_v2"  # 256 accesses: the general rule


# ----------------------------------------------- torch-level argument checks
# _as_rows only reads shapes and strides, so CPU tensors exercise it; nothing
# here reaches the library.

def test_strided_or_expanded_last_dim_is_rejected():
    import torch
    base = torch.arange(10, dtype=torch.float32)
    for bad in (base[::2],                                       # 1-D, stride 2
                torch.tensor([1.0]).expand(5),                    # 1-D, stride 0
                base.view(2, 5)[:, ::2],                          # 2-D, last stride 2
                torch.tensor([[1.0]]).expand(3, 4)):              # 2-D, last stride 0
        with pytest.raises(ValueError, match="unit stride"):
            binding._as_rows(bad)


def test_row_shapes_of_accepted_views():
    import torch
    assert binding._as_rows(torch.zeros(7)) == (1, 7, 7)
    assert binding._as_rows(torch.zeros(1).expand(1)) == (1, 1, 1)
    assert binding._as_rows(torch.zeros(6, 10)[:, :7]) == (6, 7, 10)   # gapped rows keep their pitch
    assert binding._as_rows(torch.zeros(1, 10)[:, :7]) == (1, 7, 7)
    assert binding._as_rows(torch.zeros(2, 3, 5)) == (6, 5, 5)
    with pytest.raises(ValueError, match="contiguous"):
        binding._as_rows(torch.zeros(2, 3, 6)[:, :, :5])


def test_forced_causal_kernel_on_a_batch_of_matrices_is_rejected():
    import torch
    with pytest.raises(ValueError, match="forced causal kernel takes one score matrix"):
        binding.softmax(torch.zeros(2, 4, 4), causal=True, kernel_id=0)


def test_batched_causal_rejects_before_any_launch(lib):
    far = A + (1 << 40)
    fb = lib.softmax_fwd_causal_batched
    c = ctypes.c_float
    assert fb(A, far, 12, 64, 64, 0, c(0.5), 0, 0, None) == 2    # no matrix height
    assert fb(A, far, 12, 64, 64, 5, c(0.5), 0, 0, None) == 2    # 12 rows are not whole matrices of 5
    assert fb(A, far, 12, 64, 64, 4, c(-1.0), 0, 0, None) == 7   # bad scale
    assert fb(A, far, 0, 64, 64, 4, c(0.5), 0, 0, None) == 0     # empty
    assert fb(A, far, 0, 64, 64, 0, c(0.5), 0, 0, None) == 0     # empty, from a [..., 0, m] batch
    assert fb(A, far, 0, 64, 64, 0, c(-1.0), 0, 0, None) == 7    # the scale is checked even then
    assert fb(A, A + 8, 12, 64, 64, 4, c(0.5), 0, 0, None) == 4  # overlap


def test_noalloc_split_rejects_before_any_launch(lib):
    """Host addresses: every case is refused by validation or the scratch limit."""
    nal = lib.softmax_fwd_split_noalloc
    far = A + (1 << 46)  # an output address past every input extent below
    assert nal(A, far, 4, 1 << 20, 1 << 20, 0, 2, None) == 5          # force not 0 or 1
    assert nal(A, far, 512, 1 << 20, 1 << 20, 0, 1, None) == 8        # 2 MiB of pairs > 1 MiB scratch
    assert nal(A, far, 1 << 40, 8, 8, 1, 1, None) == 8                # one tile per row, far too many rows
    assert nal(A, B, -1, 8, 8, 0, 1, None) == 2
    assert nal(A, A + 8, 4, 64, 64, 0, 1, None) == 4                  # partial overlap
    assert nal(A, B, 0, 64, 64, 0, 1, None) == 0                      # empty: nothing launched
    assert binding.NOALLOC_SCRATCH_BYTES == 1 << 20
    text = open(HEADER).read()
    assert "#define SOFTMAX_NOALLOC_SCRATCH_BYTES (1 << 20)" in text


def test_bench_chunk_copy_argument_errors(lib):
    cc = lib.softmax_bench_chunk_copy
    far = A + (1 << 40)
    assert cc(A, far, 64 << 10, 3, 16, None) == 5     # no such shape
    assert cc(A, far, (64 << 10) + 16, 4, 16, None) == 2  # not a whole number of 64 KiB chunks
    assert cc(A + 4, far, 64 << 10, 4, 16, None) == 2
    assert cc(0, far, 64 << 10, 4, 16, None) == 1
    assert cc(A, A + 1024, 64 << 10, 4, 16, None) == 4
    assert cc(A, far, 0, 4, 16, None) == 0
    assert binding.CHUNK_COPY_SHAPES[-1] == (16, 4)


def test_select_variant_reports_the_dispatch_pick(lib):
    """softmax_select_variant gives the (variant, size) of softmax_fwd's pick for
    a contiguous, aligned tensor with many rows (variant 0 packed, 1 row)."""
    from row_wise_softmax_amd import workloads as W
    a, b = 1 << 40, 1 << 41
    table = binding.kernel_table()
    for key in ("c3", "c4", "c5_bf16_32", "c5_bf16_1000", "c5_f32_3000", "c5_f32_16384", "c5_bf16_16384"):
        wl = W.WORKLOADS[key]
        code = W.dtype_code(wl.dtype)
        k = table[binding.softmax_select(a, b, wl.cols, wl.cols, code, rows=1 << 20)]
        want = ({"packed": 0, "row": 1, "online": 2, "row_pf": 3}[k.variant],
                k.lanes if k.variant == "packed" else k.block)
        assert binding.softmax_select_variant(wl.cols, code) == want, key
    v, blk = ctypes.c_int(), ctypes.c_int()
    assert lib.softmax_select_variant(0, 0, ctypes.byref(v), ctypes.byref(blk)) == 2
    assert lib.softmax_select_variant(8, 9, ctypes.byref(v), ctypes.byref(blk)) == 3
    assert lib.softmax_select_variant(8, 0, None, ctypes.byref(blk)) == 1


def test_fwd_variant_rejects_before_any_launch(lib):
    far = A + (1 << 40)
    fv = lib.softmax_fwd_variant
    assert fv(A, far, 4, 64, 64, 0, 7, 64, None) == 5       # unknown variant
    assert fv(A, far, 4, 64, 64, 0, 0, 3, None) == 5        # no packed entry with 3 lanes per row
    assert fv(A, far, 4, 1 << 20, 1 << 20, 0, 1, 256, None) == 5  # no row entry holds 2^20 columns
    assert fv(A, far, 0, 64, 64, 0, 0, 16, None) == 0       # empty: nothing launched
    assert fv(A, far, -1, 64, 64, 0, 0, 16, None) == 2

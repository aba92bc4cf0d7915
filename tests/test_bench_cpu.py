"""Host logic of bench.py, on the CPU: the one-GPU refusal, the counter
calibration and its source-digest guard, and the profile summaries.  Every
summary is written into a temporary directory, never over the committed
profiles."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.fixture
def profile_dir(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    return tmp_path


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_calibration_and_digest_guard(profile_dir, tmp_path):
    """The copy kernel moves exactly C3_BYTES each way, so its counter reading
    fixes the scale; the softmax's bytes are its reading times that scale."""
    kib = bench.C3_BYTES / 1024
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    sm, cp = "void rws::softmax_row<rws::F16, 8, 4, 2, false, false>(rws::Args)", "void rws::copy16<4>(...)"
    # FETCH reads half the true bytes, WRITE reads them exactly; the softmax re-reads 1% of its input
    _counter_csv(fetch, "FETCH_SIZE", [(cp, kib / 2), (cp, kib / 2), (sm, 1.01 * kib / 2)])
    _counter_csv(write, "WRITE_SIZE", [(cp, kib), (sm, kib), (sm, kib)])
    bench.summarize_counters(str(fetch), str(write))
    got = bench.stored_traffic("c3_8192x4096_f16")
    assert got is not None
    assert got["bytes"] == pytest.approx(2.01 * bench.C3_BYTES, rel=1e-6)
    text = (profile_dir / "counters_c3_8192x4096_f16.txt").read_text()
    assert f"source_digest: {bench.source_digest()}" in text
    assert "traffic_over_algorithmic: 1.00500" in text
    # counters of another kernel than the dispatch picks now are not reported
    from row_wise_softmax_amd import binding
    table = {k.name: k for k in binding.kernel_table()}
    assert bench.stored_traffic("c3_8192x4096_f16", table["row_f16_w4_v2"]) is not None
    assert bench.stored_traffic("c3_8192x4096_f16", table["row_f16_w2_v4"]) is None
    assert bench.stored_traffic("c3_8192x4096_f16", table["rowpf_f16_w4_v2"]) is None
    # counters taken on other kernel sources are not reported
    (profile_dir / "counters_c3_8192x4096_f16.txt").write_text(
        text.replace(bench.source_digest(), "0000000000000000"))
    assert bench.stored_traffic("c3_8192x4096_f16") is None


def test_digest_ignores_comments_only(tmp_path):
    code = "int f(int x) {  // add one\n    return x + 1;  /* done */\n}\n"
    assert bench._code_only(code) == bench._code_only(code.replace("add one", "increment"))
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))


def test_sweep_summary(profile_dir, tmp_path):
    rows = [
        {"workload": "w", "dtype": "bf16", "cols": 64, "rows": 10, "dispatch": "packed_a", "dispatch_gbps": 6400.0,
         "best": "packed_a", "best_gbps": 6400.0, "top5": [["packed_a", 6400.0], ["row_b", 6000.0]]},
        {"workload": "w", "dtype": "bf16", "cols": 4096, "rows": 10, "dispatch": "row_c", "dispatch_gbps": 6300.0,
         "best": "row_d", "best_gbps": 6350.0, "top5": [["row_d", 6350.0], ["row_c", 6300.0]]},
        {"crossover": "bf16", "packed_wins_up_to_cols": 64, "row_wins_from_cols": 4096},
    ]
    src = tmp_path / "sweep.json"
    src.write_text(json.dumps(rows))
    bench.summarize_sweep(str(src))
    text = (profile_dir / "sweep_c5_widths.md").read_text()
    assert "| bf16 | 64 | 10 | packed_a | 6400 | packed_a | 6400 | row_b 6000 |" in text
    assert "| bf16 | 4096 | 10 | row_c | 6300 | row_d | 6350 | row_c 6300 |" in text
    assert "wins up to 64 columns; one workgroup per row wins from 4096 columns" in text


def test_trace_summary_groups_attention_by_grid(profile_dir, tmp_path):
    stats = tmp_path / "bench_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "void rws::softmax_row<rws::F16, 8, 4, 2, false, false>(rws::Args)", "Calls": 3,
                    "AverageNs": 22306.4, "MinNs": 20478, "MaxNs": 32076})
    trace = tmp_path / "attn_trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp",
                                          "End_Timestamp"])
        w.writeheader()
        for start, end in ((0, 1000), (5000, 7000)):
            w.writerow({"Kernel_Name": "attention_fwd_kernel<rws::F16, 128, true>", "Grid_Size_X": 1024 * 256,
                        "Workgroup_Size_X": 256, "Start_Timestamp": start, "End_Timestamp": end})
    bench.summarize_trace(str(stats))
    text = (profile_dir / "kernel_trace_bench.md").read_text()
    assert "| 3 | 22306 | 20478 | 32076 |" in text
    assert "| f16 | 1024 | 1024 | 2 | 1500 | 1000 |" in text


def test_wide_counter_summary(profile_dir, tmp_path):
    """Each kernel's bytes are its counter reading times the copy's calibration,
    reported against its own tensor's bytes."""
    kib = (64 << 20) / 1024
    f32_kib = 8 * (1 << 20) * 4 / 1024
    online = "void rws::softmax_online<rws::F32, 4, 16, 4, false>(rws::Args)"
    cp = "void rws::copy16<4>(...)"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(cp, kib / 2), (online, 1.5 * f32_kib / 2)])
    _counter_csv(write, "WRITE_SIZE", [(cp, kib), (online, f32_kib)])
    bench.summarize_wide_counters(str(fetch), str(write))
    text = (profile_dir / "counters_wide_rows.txt").read_text()
    assert "[wide_f32 8x1048576]" in text
    assert "(1.500 x input)" in text and "(1.000 x input)" in text


def test_result_line_contract():
    """The JSON line's fields, from a stand-in measurement of the headline shape."""
    head = {"workload": "c3_8192x4096_f16", "rows": 8192, "cols": 4096, "dtype": "f16", "kernel": "row_f16_w4_v2",
            "buffers": 8, "us": 23.0, "gbps": 5835.6, "copy_kernel_gbps": 5900.0, "memcpy_gbps": 5100.0,
            "_res": object()}
    cpu = {"value": 0.4, "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": "s"}
    line = bench.result_line(head, {"c3": head}, 200, 50, cpu, {"bytes": 134223438.2})
    json.dumps(line)  # serialisable: the resources handle is dropped
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line
    assert line["value"] == 5835.6 and line["unit"] == "GB/s" and line["n_gpus"] == 1
    assert line["ms_per_step"] == 0.023 and line["higher_is_better"] is True and line["scaling"] == "weak"
    assert line["config"]["workload"] == "c3_8192x4096_f16" and "model" not in line["config"]
    assert line["vs_baseline"] == round(5835.6 / 2800.0, 3)
    r = line["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["frac"] == round(5835.6 / 8000.0, 4) and r["traffic"] == 134223438
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] == 1
    assert "_res" not in line["shapes"]["c3"]
    assert bench.result_line(head, {}, 1, 1, None, None)["roofline"]["traffic"] is None


def test_fixed_shape_sweep_summary_goes_to_its_own_file(profile_dir, tmp_path):
    rows = [{"workload": "c3_8192x4096_f16", "key": "c3", "dtype": "f16", "cols": 4096, "rows": 8192,
             "dispatch": "row_f16_w4_v2", "dispatch_gbps": 5800.0, "best": "row_f16_w4_v2", "best_gbps": 5800.0,
             "top5": [["row_f16_w4_v2", 5800.0], ["row_f16_w8_v1", 5700.0]]}]
    src = tmp_path / "fixed.json"
    src.write_text(json.dumps(rows))
    bench.summarize_sweep(str(src))
    text = (profile_dir / "sweep_fixed_shapes.md").read_text()
    assert "--sweep-keys c3" in text
    assert "| f16 | 4096 | 8192 | row_f16_w4_v2 | 5800 | row_f16_w4_v2 | 5800 | row_f16_w8_v1 5700 |" in text
    assert not (profile_dir / "sweep_c5_widths.md").exists()


def test_copy_size_summary(profile_dir, tmp_path):
    table = [{"mib": 64, "bytes": 64 << 20, "buffers": 8, "copy_us": 22.5, "copy_gbps": 5965.2, "read_us": 11.0,
              "read_gbps": 6100.5, "write_us": 11.2, "write_gbps": 5991.8}]
    src = tmp_path / "copy.json"
    src.write_text(json.dumps({"value": 1.0, "copy_ceiling": table}))  # a bench line carries the same table
    bench.summarize_copy_sizes(str(src))
    text = (profile_dir / "copy_ceiling_sizes.md").read_text()
    assert "| 64 MiB | 22.50 | 5965 | 74.6 | 6100 | 5992 |" in text


def test_shape_counter_summary(profile_dir, tmp_path):
    """Dispatch groups are found by element type and grid (one workgroup per row),
    and scaled by the 64 MiB copy's calibration."""
    kib = (64 << 20) / 1024
    rows, cols = 3051, 16384
    size = rows * cols * 4
    row = "void rws::softmax_row<rws::F32, 4, 4, 16, false, false>(rws::Args)"
    cp = "void rws::copy16<4>(unsigned int __vector(4) const*, unsigned int __vector(4)*, long)"
    fields = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    for path, counter, vals in ((fetch, "FETCH_SIZE", (kib / 2, 1.02 * size / 1024 / 2)),
                                (write, "WRITE_SIZE", (kib, size / 1024))):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=fields)
            w.writeheader()
            w.writerow({"Kernel_Name": cp, "Grid_Size": 4096 * 256, "Workgroup_Size": 256, "Counter_Name": counter,
                        "Counter_Value": vals[0]})
            w.writerow({"Kernel_Name": row, "Grid_Size": rows * 256, "Workgroup_Size": 256, "Counter_Name": counter,
                        "Counter_Value": vals[1]})
    manifest = tmp_path / "m.json"
    manifest.write_text(json.dumps([{"key": "c5_f32_16384", "workload": "c5_sweep_3051x16384_f32", "rows": rows,
                                     "cols": cols, "dtype": "f32", "kernel": "row_f32_w4_v16", "input_bytes": size}]))
    bench.summarize_shape_counters(str(fetch), str(write), str(manifest))
    text = (profile_dir / "counters_c5_wide_widths.txt").read_text()
    assert "c5_f32_16384  [c5_sweep_3051x16384_f32, row_f32_w4_v16]" in text
    assert "(1.0200 x input)" in text and "(1.0000 x input)" in text
    assert "traffic_over_algorithmic: 1.0100" in text


def test_chunk_copy_summary_lists_the_row_kernels_of_each_shape(profile_dir, tmp_path):
    rows = [{"kernel": "copy16", "waves": None, "accesses": None, "chunk_kib": None, "gbps": 6400.0,
             "runs": [6400.0, 6390.0, 6410.0]},
            {"kernel": "w4_v16", "waves": 4, "accesses": 16, "chunk_kib": 64, "gbps": 6050.0,
             "runs": [6050.0, 6040.0, 6060.0]}]
    src = tmp_path / "cc.json"
    src.write_text(json.dumps(rows))
    line = {"value": 1.0, "shapes": {"c5_f32_16384": {"kernel": "row_f32_w4_v16", "cols": 16384, "gbps": 6143.1},
                                     "c3": {"kernel": "row_f16_w4_v2", "cols": 4096, "gbps": 5800.0}}}
    bj = tmp_path / "bench.json"
    bj.write_text(json.dumps(line) + "\n")
    bench.summarize_chunk_copy(str(src), str(bj))
    text = (profile_dir / "chunk_copy_shapes.md").read_text()
    assert "| w4_v16 | 4 | 16 | 64 | 6050 | 6050, 6040, 6060 | f32 16384: 6143 |" in text
    assert "| copy16 |  |  |  | 6400 |" in text


def test_trace_reduction_and_per_grid_softmax_rows(profile_dir, tmp_path):
    """group_trace keeps one line per (kernel, grid); the summary names a row kernel's
    workload by its grid (one workgroup per row) and reads attention grids from it."""
    trace = tmp_path / "bench_kernel_trace.csv"
    fields = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    c3 = "void rws::softmax_row<rws::F16, 8, 4, 2, false, false>(rws::Args)"
    att = "void (anonymous namespace)::attention_fwd_kernel<rws::F16, 128, true>((anonymous namespace)::AttnArgs)"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for s0, s1 in ((0, 22000), (50000, 73000)):
            w.writerow({"Kernel_Name": c3, "Grid_Size_X": 8192 * 256, "Workgroup_Size_X": 256,
                        "Start_Timestamp": s0, "End_Timestamp": s1})
        w.writerow({"Kernel_Name": att, "Grid_Size_X": 1024 * 256, "Workgroup_Size_X": 256,
                    "Start_Timestamp": 0, "End_Timestamp": 48000})
    groups = tmp_path / "bench_dispatch_groups.csv"
    bench.group_trace(str(trace), str(groups))
    rows = list(csv.DictReader(open(groups)))
    assert len(rows) == 2 and {r["Calls"] for r in rows} == {"2", "1"}
    trace.unlink()  # the summary must work from the reduced file alone
    stats = tmp_path / "bench_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": c3, "Calls": 2, "AverageNs": 22500, "MinNs": 22000, "MaxNs": 23000})
    bench.summarize_trace(str(stats))
    text = (profile_dir / "kernel_trace_bench.md").read_text()
    assert "| `softmax_row<F16, 8, 4, 2, false, false>` | 8192 | 256 | c3 | 2 | 22500 | 22000 |" in text
    assert "| f16 | 1024 | 1024 | 1 | 48000 | 48000 |" in text


def test_split_crossover_summary(profile_dir, tmp_path):
    """The gain column is the one-workgroup-per-row time over softmax_fwd's, and
    each line names the path softmax_fwd took."""
    rows = [{"dtype": "f32", "row_kib": 4096, "rows": 8, "cols": 1 << 20, "softmax_fwd_path": "split via out",
             "one_wg_per_row": 180.0, "split_workspace": 15.0, "softmax_fwd": 18.0},
            {"dtype": "bf16", "row_kib": 64, "rows": 256, "cols": 32768, "softmax_fwd_path": "table",
             "one_wg_per_row": 12.0, "split_workspace": 15.0, "softmax_fwd": 12.0}]
    src = tmp_path / "cross.json"
    src.write_text(json.dumps(rows))
    bench.summarize_split_crossover(str(src))
    text = (profile_dir / "split_crossover.md").read_text()
    assert "| f32 | 4096 | 8 | 180.0 | 15.0 | 18.0 | split via out | 10.00 |" in text
    assert "| bf16 | 64 | 256 | 12.0 | 15.0 | 12.0 | table | 1.00 |" in text
    assert "--split-crossover --split-out" in text


def test_odd_width_summary(profile_dir, tmp_path):
    """Gains are softmax_fwd over the scalar path and over the aligned width below."""
    rows = [{"dtype": "bf16", "rows": 24408, "cols": 4097, "aligned_cols": 4096, "kernel": "any_row_bf16_w4_v3",
             "softmax_fwd": 5800.0, "scalar": 1700.0, "aligned_below": 5900.0}]
    src = tmp_path / "odd.json"
    src.write_text(json.dumps(rows))
    bench.summarize_odd_widths(str(src))
    text = (profile_dir / "odd_widths.md").read_text()
    assert "| bf16 | 24408 | 4097 | any_row_bf16_w4_v3 | 5800 | 1700 | 3.41x | 5900 (4096) | 0.983 |" in text


def test_ragged_rows_summary(profile_dir, tmp_path):
    """One line per (width, rows): the pick, every forced shape, and the pick
    against the fastest of them."""
    r = {"dtype": "bf16", "rows": 65536, "cols": 2040, "accesses": 255, "kernel": "row_bf16_w4_v1",
         "softmax_fwd": 5900.0, "row_bf16_w4_v1": 5910.0, "rowpf_bf16_w4_v1": 4960.0, "row_bf16_w2_v2": 5466.0,
         "rowpf_bf16_w2_v2": 4793.0, "row_bf16_w4_v2": 5166.0}
    src = tmp_path / "ragged.json"
    src.write_text(json.dumps([r]))
    bench.summarize_ragged_rows(str(src))
    text = (profile_dir / "ragged_widths_rows.md").read_text()
    assert "| row w4v1 | rowpf w4v1 | row w2v2 | rowpf w2v2 | row w4v2 | pick / best |" in text
    assert "| bf16 | 2040 | 255 | 65536 | row_bf16_w4_v1 | 5900 | 5910 | 4960 | 5466 | 4793 | 5166 | 0.998 |" in text


def test_few_rows_summary(profile_dir, tmp_path):
    """The best forced persistent shape, softmax_fwd against it, and the next three."""
    r = {"dtype": "bf16", "rows": 512, "cols": 2048, "kernel": "rowpf_bf16_w4_v1",
         "gbps": {"softmax_fwd": 1180.0, "rowpf_bf16_w4_v1": 1188.0, "rowpf_bf16_w2_v2": 1048.0,
                  "rowpf_bf16_w8_v1": 1148.0, "rowpf_bf16_w4_v2": 1031.0, "rowpf_bf16_w1_v4": 878.0}}
    src = tmp_path / "few.json"
    src.write_text(json.dumps([r]))
    bench.summarize_few_rows(str(src))
    text = (profile_dir / "few_rows_shapes.md").read_text()
    assert ("| bf16 | 2048 | 512 | rowpf_bf16_w4_v1 | 1180 | rowpf_bf16_w4_v1 | 1188 | 0.993 | "
            "w8_v1 1148, w2_v2 1048, w4_v2 1031 |") in text


def test_past_pow2_summary(profile_dir, tmp_path):
    """One line per (width, rows): the pick, the fastest forced row shape, the
    next three, and the pick against the fastest of all."""
    r = {"dtype": "bf16", "rows": 11363, "cols": 8800, "accesses": 1100, "kernel": "row_bf16_w8_v3",
         "gbps": {"softmax_fwd": 5950.0, "row_bf16_w8_v3": 5962.0, "row_bf16_w16_v2": 4774.0,
                  "row_bf16_w8_v4": 5800.0, "row_bf16_w16_v3": 5100.0}}
    src = tmp_path / "past.json"
    src.write_text(json.dumps([r]))
    bench.summarize_past_pow2(str(src))
    text = (profile_dir / "past_pow2_widths.md").read_text()
    assert ("| bf16 | 8800 | 1100 | 11363 | row_bf16_w8_v3 | 5950 | w8v3 | 5962 | w8v4 5800, w16v3 5100, "
            "w16v2 4774 | 0.998 |") in text

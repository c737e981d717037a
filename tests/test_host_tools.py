"""Host logic of the measurement tools (no GPU): the bench's byte accounting
and its refusal of more than one GPU, and the rocprofv3 summarizers on small
synthetic CSV files of the profiler's format."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from w8a8_quantized_speculative_amd import profiling, synth  # noqa: E402

KERN = ("void quasar::(anonymous namespace)::w8a8_linear_fused_kernel<6, 4, 2>"
        "(unsigned short const*, float const*)")
COPY = "quasar::(anonymous namespace)::stream_copy_kernel(int __vector(4) const*, int __vector(4)*, unsigned long)"
READ = "quasar::(anonymous namespace)::stream_read_kernel(int __vector(4) const*, unsigned long, unsigned int*)"


def test_short_kernel_names():
    assert profiling._short(KERN) == "w8a8_linear_fused_kernel<6, 4, 2>"
    assert profiling._short(COPY) == "stream_copy_kernel"
    assert profiling._short("Cijk_Alik_Bljk_BBS_BH_MT32x16x256") == "Cijk_Alik_Bljk_BBS_BH_MT32x16x256"


def test_algorithmic_bytes_of_a_layer_and_a_step():
    # one Qwen3-8B layer at 6 tokens: 192,937,984 weight bytes, 193,953,792 in all
    lin = synth.QWEN3_8B_LINEARS
    assert sum(N * K for _, K, N in lin) == 192_937_984
    assert sum(bench.algorithmic_bytes(6, N, K) for _, K, N in lin) == 193_953_792
    # the 36-layer stack with the LM head
    step = 36 * 193_953_792 + bench.algorithmic_bytes(6, synth.QWEN3_8B_VOCAB, 4096)
    assert step == 7_607_162_880
    # plus the drafts read (4 B x B x k) and the accept lengths and next tokens written
    assert step + 4 * 1 * 5 + 8 * 1 == 7_607_162_908
    assert bench.algorithmic_bytes_w4(6, 4096, 4096) == 4096 * 4096 // 2 + 4 * 4096 + 4 * 4096 \
        + 2 * 6 * 4096 + 2 * 6 * 4096


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_kernel_source_hash_follows_the_kernel_family():
    a = profiling.kernel_source_hash("w8a8_linear_fused_kernel<6, 4, 2>")
    assert a == profiling.kernel_source_hash("w4a8_linear_fused_kernel<6, 4, 1>")  # same file
    assert a != profiling.kernel_source_hash("w8a8_linear_wide_kernel<3, 1>")
    assert profiling.kernel_source_hash("w4a8_linear_wide_kernel<3, 1>") == \
        profiling.kernel_source_hash("w8a8_linear_wide_kernel<6, 4>")  # same file
    assert len(a) == 16


def test_kernel_source_hash_ignores_comments_and_layout():
    a = 'int f(int x) {  // twice\n  return 2 * x; /* doubled */ }\nconst char* s = "a // b";'
    b = 'int f(int x) {\n    return 2 * x;   }\n// a note\nconst char* s = "a // b";'
    c = 'int f(int x) { return 3 * x; } const char* s = "a // b";'
    assert profiling.code_only(a) == profiling.code_only(b)
    assert profiling.code_only(a) != profiling.code_only(c)
    assert profiling.code_only('char q = \'"\'; // x') == "char q = '\"';"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def _bench_line(path, extra=None):
    line = {
        "value": 4700.0, "unit": "GB/s", "ms_per_step": 1.6,
        "config": {"workload": "test workload", "M": 6},
        "roofline": {"kernel": "w8a8_linear_fused_kernel<6, 4, 2>", "launch_avg_us": 11.0,
                     "algorithmic_bytes_per_launch": 53_080_608, "achieved": 4825.5},
        "kernels": [{"kernel": "w8a8_linear_fused_kernel<6, 4, 2>",
                     "algorithmic_bytes_per_launch": 53_080_608, "launch_avg_us": 11.0}],
        "copy_calibration": {"bytes": 512 << 20},
        "read_calibration": {"bytes": 1 << 30, "dispatches": 11},
        "read_twin": {"bytes": 7_568_097_280, "passes": 6, "launches_per_pass": 145},
    }
    line.update(extra or {})
    with open(path, "w") as f:
        f.write("[bench] progress line\n" + json.dumps(line) + "\n")


def test_pmc_summary_scales_by_the_copy_and_cross_checks_on_the_read(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy_units = (512 << 20) / 2048.0          # FETCH counts 2048 B per unit here
    n_read = 11 + 6 * 145
    read_mean = (11 * (1 << 30) + 6 * 7_568_097_280) / n_read
    fetch = [[1, COPY, "FETCH_SIZE", copy_units], [2, COPY, "FETCH_SIZE", copy_units],
             [3, KERN, "FETCH_SIZE", 53_600_000 / 2048.0], [4, KERN, "FETCH_SIZE", 53_600_000 / 2048.0]]
    fetch += [[10 + i, READ, "FETCH_SIZE", read_mean / 2048.0] for i in range(n_read)]
    write = [[1, COPY, "WRITE_SIZE", (512 << 20) / 1024.0], [3, KERN, "WRITE_SIZE", 150_000 / 1024.0]]
    _write(tmp_path / "f.csv", hdr, fetch)
    _write(tmp_path / "w.csv", hdr, write)
    _bench_line(tmp_path / "b.json")
    res = profiling.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                  str(tmp_path / "b.json"), str(tmp_path / "o.json"),
                                  str(tmp_path / "o.md"), "cmd-f", "cmd-w")
    k = res["kernels"]["w8a8_linear_fused_kernel<6, 4, 2>"]
    assert k["fetch_bytes_per_launch"] == 53_600_000 and k["write_bytes_per_launch"] == 150_000
    assert k["traffic_over_algorithmic"] == pytest.approx(53_750_000 / 53_080_608, abs=1e-4)
    assert k["kernel_source_hash"] == profiling.kernel_source_hash("w8a8_linear_fused_kernel<6, 4, 2>")
    x = res["fetch_cross_check"]
    assert x["dispatches"] == x["expected_dispatches"] == n_read and x["ratio"] == pytest.approx(1.0)
    assert json.load(open(tmp_path / "o.json"))["kernels"].keys() == res["kernels"].keys()
    assert "ratio 1.0" in open(tmp_path / "o.md").read()


def test_stats_summary_takes_the_step_grid_from_the_trace(tmp_path):
    _write(tmp_path / "s.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage",
                                "MinNs", "MaxNs", "StdDev"],
           [[KERN, 13, 13 * 10_000, 10_000, 50, 4_700, 11_000, 1]])
    hdr = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
           "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    rows = [["KERNEL_DISPATCH", KERN, 1000 * i, 1000 * i + 11_000, 0, 131072, 1, 1] for i in range(10)]
    rows += [["KERNEL_DISPATCH", KERN, 1000 * i, 1000 * i + 4_700, 0, 32768, 1, 1] for i in range(3)]
    _write(tmp_path / "t.csv", hdr, rows)
    _bench_line(tmp_path / "b.json")
    res = profiling.summarize_stats(str(tmp_path / "s.csv"), str(tmp_path / "b.json"),
                                    str(tmp_path / "o.md"), "cmd", str(tmp_path / "t.csv"))
    assert res["rocprof_avg_us"] == pytest.approx(10.0)
    assert res["rocprof_step_config_avg_us"] == pytest.approx(11.0)
    md = open(tmp_path / "o.md").read()
    assert "the 10 of its 13 dispatches" in md and "11.00 us" in md


def test_kernel_launch_times_cover_every_section():
    line = {"kernels": [{"kernel": "a<6>", "launch_avg_us": 10.0}],
            "window_m48": {"kernels": [{"kernel": "b<3>", "launch_avg_us": 20.0}],
                           "w4a8_variant": {"kernels": [{"kernel": "c<3>", "launch_avg_us": 15.0}]}},
            "w4a8_variant": {"kernels": [{"kernel": "d<6>", "launch_avg_us": 8.0}]},
            "roofline": {"kernel": "a<6>"}}
    t = profiling.kernel_launch_times(line)
    assert {k: v["launch_avg_us"] for k, v in t.items()} == {"a<6>": 10.0, "b<3>": 20.0,
                                                               "c<3>": 15.0, "d<6>": 8.0}

"""The rocprofv3 summariser (host logic, no GPU): counter scaling against the calibration copy,
per-dispatch medians, and the trace table, on small synthetic CSV files laid out as rocprofv3
writes them."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DECODE = "void pa::(anonymous namespace)::decode_partition_kernel<128, 16, 4, false, true>(pa::DecodeParams)"
COUNTER_HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id",'
                  '"Grid_Size","Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size",'
                  '"Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count","Counter_Name",'
                  '"Counter_Value","Start_Timestamp","End_Timestamp"')


def counter_csv(path, counter, rows):
    lines = [COUNTER_HEADER]
    for i, (name, grid, value) in enumerate(rows):
        lines.append(f'{i},{i},"Agent 1",1,1,1,{grid},1,"{name}",256,0,0,8,0,32,"{counter}",'
                     f'{value},0,1')
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(lines) + "\n")


def bench_log(path, nbytes):
    line = {"value": 6500.0, "unit": "GB/s", "ms_per_step": 0.165,
            "config": {"workload": "paged decode 8b: synthetic"},
            "roofline": {"algorithmic_bytes_per_call": nbytes, "avg_call_us": 164.0}}
    open(path, "w").write("[bench] progress\n" + json.dumps(line) + "\n")


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "rocprof_summary.py"), *args],
                          capture_output=True, text=True, check=True, cwd=ROOT).stdout


def test_traffic_scales_counters_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    # the copy of 256 MiB reads as half its size in FETCH_SIZE and exactly in WRITE_SIZE
    counter_csv(str(tmp_path / "fetch" / "x" / "f_counter_collection.csv"), "FETCH_SIZE",
                [(copy, 131072, 131072.0)] * 3 + [(copy, 512, 2.0)] +
                [(DECODE, 131072, 500.0), (DECODE, 131072, 524800.0), (DECODE, 131072, 524900.0)])
    counter_csv(str(tmp_path / "write" / "w_counter_collection.csv"), "WRITE_SIZE",
                [(copy, 131072, 262144.0)] * 3 +
                [(DECODE, 131072, 768.0), (DECODE, 131072, 768.0), (DECODE, 131072, 768.0)])
    bench_log(str(tmp_path / "b.log"), 1_000_000_000)
    md, js = str(tmp_path / "t.md"), str(tmp_path / "t.json")
    run("traffic", str(tmp_path / "fetch"), str(tmp_path / "write"), "--bench-log",
        str(tmp_path / "b.log"), "--command", "cmd1", "--command", "cmd2", "--out", md, "--json", js)
    rec = json.load(open(js))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    # median of the three dispatches, each counter scaled, in bytes
    assert rec["hbm_bytes_per_call"] == (524800.0 * 2.0 + 768.0) * 1024
    assert rec["fetch_kib"] == 524800.0 and rec["write_kib"] == 768.0
    sys.path.insert(0, ROOT)
    import bench

    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    text = open(md).read()
    assert "cmd1" in text and "cmd2" in text and "ratio 1.0756" in text


def test_trace_reports_the_dominant_kernel(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    (d / "trace_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        f'"{DECODE}",10,1650000,165000.0,90.0,160000,170000,1.0\n'
        '"other",2,20000,10000.0,10.0,9000,11000,1.0\n')
    bench_log(str(tmp_path / "b.log"), 1_073_741_824)
    out = str(tmp_path / "t.md")
    run("trace", str(d), "--bench-log", str(tmp_path / "b.log"), "--command", "cmd", "--out", out)
    text = open(out).read()
    assert "| `decode_partition_kernel<128, 16, 4, false, true>` | 10 | 165.0 | 160.0 | 170.0 |" in text
    # 1 GiB per call / 165 us
    assert "6508 GB/s (81.3 % of 8 TB/s)" in text
    # a second kernel of the same call adds its average to the call time: 1 GiB / 175 us
    run("trace", str(d), "--bench-log", str(tmp_path / "b.log"), "--command", "cmd", "--also",
        "other", "--out", out)
    assert "6136 GB/s (76.7 % of 8 TB/s)" in open(out).read()

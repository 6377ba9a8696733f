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


def sq_csv(path, kernel, values, start=0, end=100_000):
    """One dispatch of `kernel` with the given {counter: value}, plus an unrelated kernel."""
    lines = [COUNTER_HEADER]
    for i, (name, v) in enumerate(values.items()):
        lines.append(f'{i},1,"Agent 1",1,1,1,131072,1,"{kernel}",256,0,0,8,0,32,"{name}",'
                     f'{v},{start},{end}')
    lines.append(f'99,2,"Agent 1",1,1,1,512,2,"other",256,0,0,8,0,32,"SQ_WAVES",5,0,1')
    os.makedirs(os.path.dirname(path), exist_ok=True)
    open(path, "w").write("\n".join(lines) + "\n")


def test_sq_ratios_from_two_counter_passes(tmp_path):
    # 100 us at 2.0 GHz: GRBM_GUI_ACTIVE counts 200,000 cycles in each of the 8 XCDs
    cyc = 200_000
    sq_csv(str(tmp_path / "a" / "a_counter_collection.csv"), DECODE,
           {"SQ_WAVES": 2048, "SQ_INSTS_VALU": 1024 * cyc // 8, "SQ_INSTS_MFMA": 0,
            "SQ_VALU_MFMA_BUSY_CYCLES": 0, "GRBM_GUI_ACTIVE": 8 * cyc})
    sq_csv(str(tmp_path / "b" / "b_counter_collection.csv"), DECODE,
           {"SQ_WAVE_CYCLES": 1000, "SQ_ACTIVE_INST_ANY": 250, "SQ_WAIT_INST_ANY": 500,
            "SQ_WAIT_ANY": 250, "SQ_LDS_IDX_ACTIVE": 256 * cyc // 4, "SQ_LDS_BANK_CONFLICT": 16_000_000 // 4,
            "GRBM_GUI_ACTIVE": 8 * cyc})
    bench_log(str(tmp_path / "b.log"), 1 << 30)
    out = str(tmp_path / "sq.md")
    run("sq", str(tmp_path / "a"), str(tmp_path / "b"), "--bench-log", str(tmp_path / "b.log"),
        "--kernel", "decode_partition_kernel", "--command", "ca", "--command", "cb", "--out", out)
    text = open(out).read()
    assert "ca" in text and "cb" in text
    assert "| busy cycles per ns | 2.00 |" in text
    # 1024 * cyc / 8 VALU instructions, 4 cycles each, over 1024 SIMDs x cyc cycles
    assert "| vector-ALU issue share | 0.500 |" in text
    assert f"| VALU per wave | {1024 * cyc // 8 // 2048} |" in text
    # 1 GiB per call = 1,048,576 KiB
    assert f"| VALU per KiB | {1024 * cyc / 8 / 1048576:.1f} |" in text
    assert "| LDS active | 0.250 |" in text
    assert "| LDS bank-conflict share | 0.312 |" in text
    assert "| wave time waiting to issue (dependencies, busy units) | 0.500 |" in text


def test_sq_vector_alu_rows_leave_out_the_mfma_instructions(tmp_path):
    # SQ_INSTS_VALU counts the matrix-core instructions as well: the vector-ALU rows subtract
    # SQ_INSTS_MFMA, the raw VALU row keeps the counter as read
    cyc = 200_000
    valu, mfma = 1024 * cyc // 8, 3_000_000
    sq_csv(str(tmp_path / "a" / "a_counter_collection.csv"), DECODE,
           {"SQ_WAVES": 2048, "SQ_INSTS_VALU": valu + mfma, "SQ_INSTS_MFMA": mfma,
            "SQ_VALU_MFMA_BUSY_CYCLES": 0, "GRBM_GUI_ACTIVE": 8 * cyc})
    bench_log(str(tmp_path / "b.log"), 1 << 30)
    out = str(tmp_path / "sq.md")
    run("sq", str(tmp_path / "a"), "--bench-log", str(tmp_path / "b.log"),
        "--kernel", "decode_partition_kernel", "--command", "ca", "--out", out)
    text = open(out).read()
    assert "| vector-ALU issue share | 0.500 |" in text
    assert f"| VALU excl. MFMA per wave | {valu / 2048:.0f} |" in text
    assert f"| VALU per wave | {(valu + mfma) / 2048:.0f} |" in text
    assert f"| MFMA per wave | {mfma / 2048:.0f} |" in text

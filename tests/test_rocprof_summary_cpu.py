"""The measurement pipeline's host logic (rocprof_summary.py) on synthetic
rocprofv3 CSVs whose answers are known: the timed-region selection (last N
dispatches before the final `skip`), the duration statistics, and the HBM
traffic scaling by the plain copy probe."""
import argparse
import csv
import json

from greedy_block_verification_amd import rocprof_summary as R

K = "void sv::k_gemm_bf16<1, 2, 8, false>(sv::GemmArgs)"


def _trace(path):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for i in range(1, 11):                      # durations 1..10 us
            w.writerow({"Kernel_Name": K, "Start_Timestamp": t, "End_Timestamp": t + 1000 * i})
            t += 100_000
            w.writerow({"Kernel_Name": "void sv::k_attn_mfma<128, true>(sv::AttnArgs)",
                        "Start_Timestamp": t, "End_Timestamp": t + 500})
            t += 100_000


def _counters(path, name, copy_kib, kib):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerow({"Dispatch_Id": 0, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": name,
                    "Counter_Value": copy_kib})
        for d, v in enumerate(kib, start=1):
            w.writerow({"Dispatch_Id": d, "Kernel_Name": K, "Counter_Name": name, "Counter_Value": v})


def test_stats_takes_the_timed_region(tmp_path):
    _trace(tmp_path / "t.csv")
    a = argparse.Namespace(trace=str(tmp_path / "t.csv"), kernel="sv::k_gemm_bf16<1, 2, 8, false>", last=4, skip=2,
                           top=5, title="synthetic", command="cmd", out=str(tmp_path / "o.md"))
    R.stats(a)
    text = open(tmp_path / "o.md").read()
    # dispatches 5..8 (1-based) of the kernel: 5, 6, 7, 8 us
    assert "last 4 dispatches (before the final 2)" in text
    assert "mean 6.50 us, median 7.00 us, min 5.00 us, max 8.00 us" in text
    assert "| `void sv::k_gemm_bf16<1, 2, 8, false>` | 10 | 5.50 | 0.06 |" in text


def test_traffic_scales_counters_by_the_copy_probe(tmp_path):
    # a 1 GiB copy reads as 512 MiB of FETCH_SIZE (x 2) and 1 GiB of WRITE_SIZE (x 1)
    _counters(tmp_path / "f.csv", "FETCH_SIZE", 524288.0, [999.0, 100.0, 100.0, 100.0, 7.0])
    _counters(tmp_path / "w.csv", "WRITE_SIZE", 1048576.0, [999.0, 10.0, 10.0, 10.0, 7.0])
    a = argparse.Namespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"),
                           kernel="sv::k_gemm_bf16<1, 2, 8, false>", last=3, skip=1, copy_bytes=1 << 30,
                           algorithmic_bytes=204800 + 10240, command="cmd", out=str(tmp_path / "t.json"),
                           table_out=None, table_last=200, title="synthetic")
    R.traffic(a)
    rec = json.load(open(tmp_path / "t.json"))
    assert rec["dispatches"] == {"fetch": 3, "write": 3}
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 204800 and rec["write_bytes_per_launch"] == 10240
    assert rec["traffic_over_algorithmic"] == 1.0
    assert rec["kernel_source_sha256"] == R.kernel_source_sha256()


def test_counters_means_and_wait_shares(tmp_path):
    path = tmp_path / "c.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d in range(1, 4):                     # three dispatches of 2, 4, 6 us
            vals = {"SQ_WAVES": 100.0, "SQ_INSTS_VALU": 1000.0 * d, "SQ_WAVE_CYCLES": 4000.0,
                    "SQ_WAIT_ANY": 1000.0 * d, "SQ_WAIT_INST_ANY": 400.0}
            for n, v in vals.items():
                w.writerow({"Dispatch_Id": d, "Kernel_Name": K, "Counter_Name": n, "Counter_Value": v,
                            "Start_Timestamp": 0, "End_Timestamp": 2000 * d})
    a = argparse.Namespace(counters=str(path), kernel=["sv::k_gemm_bf16"], last=2, xcc=8, simds=1024,
                           title="synthetic", command="cmd", out=str(tmp_path / "c.md"))
    R.counters(a)
    text = open(tmp_path / "c.md").read()
    # last two dispatches: 4 and 6 us, VALU 2500 per dispatch = 25 per wave, wait any 62.5 %, wait issue 10 %
    row = [l for l in text.splitlines() if l.startswith("| `void sv::k_gemm_bf16")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1:3] == ["2", "5.00"]
    assert cells[-3:] == ["25", "62.5", "10"]

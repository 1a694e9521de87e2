"""Host logic of bench.py, on the CPU: the one-GPU guard of every mode, the
parsing of rocprofv3 output, and the copy-calibrated traffic that the bench
line reports (written to, and read back from, a traffic file)."""

import csv
import json
import os

import pytest

import bench


@pytest.mark.parametrize("mode", [[], ["--mx"], ["--calib"], ["--chain"], ["--probe"]])
def test_more_than_one_gpu_is_refused_before_any_device_work(mode, capsys):
    assert bench.main(["--gpus", "2", *mode]) == 2
    assert "one GPU" in capsys.readouterr().err


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


_CC_HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
              "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
              "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
              "End_Timestamp"]
_GEMM = "void hsq::(anonymous namespace)::k_gemm_tiled<false, 4, 0, 1, 1, false>(hsq::GemmArgs, int, int)"


def _counter_dir(root, counter, gemm_values, copy_kib):
    """A counter-collection directory: launches of the contraction (the first
    two are warm-up), then three reference copies; a counter may be split
    over several rows of one dispatch (they add up)."""
    rows, did = [], 0
    for v in gemm_values:
        did += 1
        rows.append([did, did, "Agent 1", 1, 1, 1, 1, 3, _GEMM, 512, 0, 0, 116, 0, 64, counter, v / 2, 0, 1])
        rows.append([did, did, "Agent 1", 1, 1, 1, 1, 3, _GEMM, 512, 0, 0, 116, 0, 64, counter, v / 2, 0, 1])
    for _ in range(3):
        did += 1
        rows.append([did, did, "Agent 1", 1, 1, 1, 1, 9, "__amd_rocclr_copyBuffer", 256, 0, 0, 8, 0, 16,
                     counter, copy_kib, 0, 1])
    _write_csv(os.path.join(root, "run_counter_collection.csv"), _CC_HEADER, rows)


def test_summarize_scales_counters_by_the_reference_copy(tmp_path, monkeypatch, capsys):
    # FETCH_SIZE reads half of the copy's true KiB (factor 2), WRITE_SIZE all
    # of it; the contraction's launches after the two warm-up ones average
    # 1000 KiB fetched and 300 KiB written
    copy_mb = 8.0
    true_kib = (int(copy_mb * 1e6) // 16 * 16) / 1024
    fetch_dir, write_dir = tmp_path / "fetch", tmp_path / "write"
    _counter_dir(str(fetch_dir), "FETCH_SIZE", [5000.0, 5000.0, 900.0, 1100.0, 1000.0], true_kib / 2)
    _counter_dir(str(write_dir), "WRITE_SIZE", [9000.0, 9000.0, 300.0, 300.0, 300.0], true_kib)
    traffic = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    rc = bench.main(["--summarize", str(fetch_dir), str(write_dir), "--copy-mb", str(copy_mb),
                     "--layer", "pixart_up", "--write-traffic"])
    assert rc == 0
    out = capsys.readouterr().out
    assert "FETCH_SIZE factor 2.0000" in out and "WRITE_SIZE factor 1.0000" in out
    rec = json.loads(traffic.read_text())["pixart_up"]["tiled"]
    assert rec["fetch_bytes"] == int(1000.0 * 1024 * 2.0)
    assert rec["write_bytes"] == int(300.0 * 1024 * 1.0)
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["source_sha256_16"] == bench.source_hash(bench.KERNEL_SOURCES["tiled"])
    # read back while the kernel source is unchanged; a stale hash reads as none
    assert bench.read_traffic("tiled", "pixart_up") == rec["bytes_per_launch"]
    rec_all = json.loads(traffic.read_text())
    rec_all["pixart_up"]["tiled"]["source_sha256_16"] = "0" * 16
    traffic.write_text(json.dumps(rec_all))
    assert bench.read_traffic("tiled", "pixart_up") is None


def test_summarize_lists_kernel_stats_by_total_time(tmp_path, capsys):
    d = tmp_path / "trace"
    _write_csv(str(d / "run_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
               [["small_kernel", 10, 1000, 100.0, 1.0, 90, 110, 5.0],
                [_GEMM, 4, 1200000, 300000.0, 99.0, 290000, 310000, 100.0]])
    assert bench.main(["--summarize", str(d)]) == 0
    lines = capsys.readouterr().out.splitlines()
    body = [l for l in lines if l.startswith("  ") and "calls" not in l]
    assert body[0].split()[-4:] == ["4", "300.00", "290.00", "310.00"]
    assert body[1].split()[-4:] == ["10", "0.10", "0.09", "0.11"]


def test_traffic_keys_name_layer_tokens_and_group():
    assert bench.traffic_key("flux_mlp", None, 4608, 64) == "flux_mlp"
    assert bench.traffic_key("qwen3_up", 16, 16, 64) == "qwen3_up_M16"
    assert bench.traffic_key("qwen3_up", 256, 256, 128) == "qwen3_up_M256_g128"


def test_sample_rows_spread_over_the_layer():
    rows = bench._sample_rows(4608, 192)
    assert rows[0] == 0 and rows[-1] == 4607 and len(rows) == 192
    assert list(bench._sample_rows(3, 192)) == [0, 1, 2]

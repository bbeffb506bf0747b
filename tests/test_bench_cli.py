"""The benchmark's command line on the CPU: more than one GPU is refused with a message
(the hot path is single-GPU), and the profile summaries parse rocprofv3's CSV layout."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_summaries_from_rocprof_csv(tmp_path):
    sys.path.insert(0, ROOT)
    import bench
    stats = tmp_path / "kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow(["zc::(anonymous namespace)::compress_single_kernel(zc::CArgs)", 3, 150000, 50000, 50, 48000,
                    52000, 1])
        w.writerow(["zc::(anonymous namespace)::decompress_kernel(zc::DArgs)", 3, 120000, 40000, 40, 39000,
                    41000, 1])
        w.writerow(["__amd_rocclr_copyBuffer", 1, 1000, 1000, 10, 1000, 1000, 0])
    out = tmp_path / "k.txt"
    bench.summarize_stats(str(stats), str(out))
    text = out.read_text()
    assert "| compress_single_kernel | 3 | 50.00 | 48.00 | 52.00 |" in text
    assert "| decompress_kernel | 3 | 40.00 | 39.00 | 41.00 |" in text
    assert "copyBuffer" not in text

    def counters(path, counter, vals):
        with open(path, "w", newline="") as f:
            w = csv.writer(f, quoting=csv.QUOTE_ALL)
            w.writerow(["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
            for name, grid, v in vals:
                w.writerow([name, grid, counter, v])

    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    units = 4096
    cgrid, dgrid = (units + units // 8) * 512, units * 512
    counters(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 1, 524288.0),
                                   ("compress_single_kernel(zc::CArgs)", cgrid, 1000.0),
                                   ("decompress_kernel(zc::DArgs)", dgrid, 500.0)])
    counters(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1, 1048576.0),
                                   ("compress_single_kernel(zc::CArgs)", cgrid, 300.0),
                                   ("decompress_kernel(zc::DArgs)", dgrid, 700.0)])
    out2 = tmp_path / "p.txt"
    bench.summarize_pmc(str(fetch), str(write), str(out2), n_units=units)
    kv = dict(line.split("=", 1) for line in out2.read_text().splitlines() if "=" in line and " " not in line)
    # FETCH_SIZE scaled x2 (the copy read 1 GiB and counted half), WRITE_SIZE x1; KiB -> bytes
    assert int(kv["compress_traffic_bytes"]) == (2 * 1000 + 300) * 1024
    assert int(kv["decompress_traffic_bytes"]) == (2 * 500 + 700) * 1024

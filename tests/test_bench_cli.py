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
    bench.summarize_stats_any(str(stats), str(out), "bucket_64m", bench.only_cmd_stats("bucket_64m"))
    text = out.read_text()
    assert "| compress_single_kernel | 3 | 50.00 | 48.00 | 52.00 |" in text
    assert "| decompress_kernel | 3 | 40.00 | 39.00 | 41.00 |" in text
    assert "copyBuffer" not in text
    assert "python3 bench.py --only bucket_64m" in text

    def counters(path, vals):
        with open(path, "w", newline="") as f:
            w = csv.writer(f, quoting=csv.QUOTE_ALL)
            w.writerow(["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
            for name, grid, counter, v in vals:
                w.writerow([name, grid, counter, v])

    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cgrid, dgrid = 4608 * 512, 16384 * 128
    counters(fetch, [("__amd_rocclr_copyBuffer", 1, "FETCH_SIZE", 524288.0),
                     ("compress_single_kernel(zc::CArgs)", cgrid, "FETCH_SIZE", 1000.0),
                     ("compress_single_kernel(zc::CArgs)", cgrid, "FETCH_SIZE", 1200.0),
                     ("decompress_kernel(zc::DArgs)", dgrid, "FETCH_SIZE", 500.0)])
    counters(write, [("__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", 1048576.0),
                     ("compress_single_kernel(zc::CArgs)", cgrid, "WRITE_SIZE", 300.0),
                     ("compress_single_kernel(zc::CArgs)", cgrid, "WRITE_SIZE", 300.0),
                     ("decompress_kernel(zc::DArgs)", dgrid, "WRITE_SIZE", 700.0)])
    launches = tmp_path / "l.json"
    launches.write_text('[{"kernel": "compress_single_kernel", "grid": %d, "per_step": 1, "bytes": 3000000, '
                        '"values": 1}, {"kernel": "decompress_kernel", "grid": %d, "per_step": 1, "bytes": 2000000, '
                        '"values": 1}]' % (cgrid, dgrid))
    out2 = tmp_path / "p.txt"
    bench.summarize_pmc_any("bucket_64m", str(launches), str(fetch), str(write), str(out2))
    kv = dict(line.split("=", 1) for line in out2.read_text().splitlines() if "=" in line and " " not in line)
    # FETCH_SIZE scaled x2 (the copy read 1 GiB and counted half), WRITE_SIZE x1; mean over
    # dispatches; KiB -> bytes
    assert int(kv[f"compress_single_kernel_{cgrid}_traffic_bytes"]) == (2 * 1100 + 300) * 1024
    assert int(kv[f"decompress_kernel_{dgrid}_traffic_bytes"]) == (2 * 500 + 700) * 1024

    # the raw TCC cross-check: every route agrees on a plain 1 GiB read
    c0, c1 = tmp_path / "t0.csv", tmp_path / "t1.csv"
    q = GIB = 1 << 30
    counters(c0, [("__amd_rocclr_copyBuffer", 1, "TCC_EA0_RDREQ_sum", q / 128),
                  ("__amd_rocclr_copyBuffer", 1, "TCC_EA0_RDREQ_32B_sum", 0),
                  ("__amd_rocclr_copyBuffer", 1, "TCC_BUBBLE_sum", q / 128),
                  ("__amd_rocclr_copyBuffer", 1, "TCC_EA0_RDREQ_128B_sum", q / 128)])
    counters(c1, [("__amd_rocclr_copyBuffer", 1, "TCC_EA0_RDREQ_DRAM_32B_sum", q / 32),
                  ("__amd_rocclr_copyBuffer", 1, "TCC_EA0_RDREQ_64B_sum", 0),
                  ("__amd_rocclr_copyBuffer", 1, "TCC_EA0_WRREQ_sum", q / 64),
                  ("__amd_rocclr_copyBuffer", 1, "TCC_EA0_WRREQ_64B_sum", q / 64)])
    bench.summarize_tcc(str(c0), str(c1), str(out2))
    assert f"| __amd_rocclr_copyBuffer | 1 | {GIB / 1e6:.2f} | {GIB / 1e6:.2f} | {GIB / 1e6:.2f} | {GIB / 1e6:.2f} |" \
        in out2.read_text()


def test_profiles_follow_the_kernel_code_not_its_comments():
    sys.path.insert(0, ROOT)
    import bench
    code = "// header\nint f(int x)  \n{\n\n    return x + 1;   // one more\n}\n"
    assert bench.kernel_code_text(code) == "int f(int x)\n{\n    return x + 1;\n}\n"
    assert bench.kernel_code_text(code.replace("one more", "plus one")) == bench.kernel_code_text(code)
    assert bench.kernel_code_text(code.replace("x + 1", "x + 2")) != bench.kernel_code_text(code)

"""Host-side logic of bench.py: the one-GPU contract and the arithmetic that turns
rocprofv3 counter readings into HBM bytes per launch (on synthetic counter files)."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for (d, name, v) in rows:
            # two rows per dispatch (the counter is reported per hardware instance)
            w.writerow(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter,
                            Counter_Value=v / 2))
            w.writerow(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name=counter,
                            Counter_Value=v / 2))


def test_counter_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """FETCH_SIZE reading half the known 256 MiB copy gives a factor of 2; the GEMM
    dispatches' mean reading is scaled by it; smaller copies (not the calibration) are
    ignored; the summary is stamped with the kernel-source hash."""
    sys.path.insert(0, ROOT)
    import bench
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(out))
    copy_kib = (256 << 20) / 1024.0
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    gemm = "void w4a16::skinny_kernel<4, 1, 8, 4, 0>(...)"
    copy = "copyBuffer"
    _write(fetch, "FETCH_SIZE", [(1, copy, 10.0), (2, copy, copy_kib / 2), (3, copy, copy_kib / 2),
                                 (4, copy, copy_kib / 2), (5, gemm, 1000.0), (6, gemm, 3000.0)])
    _write(write, "WRITE_SIZE", [(1, copy, copy_kib), (2, copy, copy_kib), (3, copy, copy_kib),
                                 (4, gemm, 10.0), (5, gemm, 30.0)])
    bench.pmc_summary(str(fetch), str(write))
    d = json.loads(out.read_text())
    assert abs(d["fetch_factor"] - 2.0) < 1e-9 and abs(d["write_factor"] - 1.0) < 1e-9
    assert d["fetch_kib_per_launch"] == 2000.0 and d["write_kib_per_launch"] == 20.0
    assert d["hbm_bytes_per_launch"] == int((2000.0 * 2.0 + 20.0) * 1024)
    assert d["kernel_sha"] == bench.kernel_sha() and d["launches"] == 2
    assert str(fetch) in d["commands"][-1]

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
    monkeypatch.setitem(bench.TRAFFIC_JSON, "skinny", str(out))
    copy_kib = (256 << 20) / 1024.0
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    gemm = "void w4a16::skinny_kernel<4, 1, 8, 4, 0>(...)"
    copy = "copyBuffer"
    _write(fetch, "FETCH_SIZE", [(1, copy, 10.0), (2, copy, copy_kib / 2), (3, copy, copy_kib / 2),
                                 (4, copy, copy_kib / 2), (5, gemm, 1000.0), (6, gemm, 3000.0)])
    _write(write, "WRITE_SIZE", [(1, copy, copy_kib), (2, copy, copy_kib), (3, copy, copy_kib),
                                 (4, gemm, 10.0), (5, gemm, 30.0)])
    bench.pmc_summary(str(fetch), str(write), kind="skinny")
    d = json.loads(out.read_text())
    assert abs(d["fetch_factor"] - 2.0) < 1e-9 and abs(d["write_factor"] - 1.0) < 1e-9
    assert d["fetch_kib_per_launch"] == 2000.0 and d["write_kib_per_launch"] == 20.0
    assert d["hbm_bytes_per_launch"] == int((2000.0 * 2.0 + 20.0) * 1024)
    assert d["kernel_sha"] == bench.kernel_sha("skinny") and d["launches"] == 2
    assert str(fetch) in d["commands"][-1]


def test_tiled_counter_summary_counts_the_fixup_into_its_call(tmp_path, monkeypatch):
    """kind "tiled": a call is a tiled_kernel dispatch plus, where tiles are cut, a
    tiled_fixup_kernel dispatch; bytes per call = (all of them) / (tiled_kernel
    dispatches)."""
    sys.path.insert(0, ROOT)
    import bench
    out = tmp_path / "traffic.json"
    monkeypatch.setitem(bench.TRAFFIC_JSON, "tiled", str(out))
    copy_kib = (256 << 20) / 1024.0
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    k = "void w4a16::tiled_kernel<8, 4, 3, 0>(...)"
    fx = "void w4a16::tiled_fixup_kernel<8, 4>(...)"
    _write(fetch, "FETCH_SIZE", [(1, "copyBuffer", copy_kib), (2, "copyBuffer", copy_kib),
                                 (3, "copyBuffer", copy_kib), (4, k, 1000.0), (5, fx, 200.0),
                                 (6, k, 3000.0)])
    _write(write, "WRITE_SIZE", [(1, "copyBuffer", copy_kib), (2, k, 10.0), (3, k, 30.0)])
    bench.pmc_summary(str(fetch), str(write), kind="tiled")
    d = json.loads(out.read_text())
    assert d["launches"] == 2 and d["fixup_dispatches"] == 1
    assert d["fetch_kib_per_launch"] == 2100.0 and d["write_kib_per_launch"] == 20.0
    assert d["kernel_sha"] == bench.kernel_sha("tiled")


def test_the_bench_line_is_compact_and_complete():
    """The driver keeps only the tail of stdout: the one JSON line must stay well under
    4 KB with every field the contract names (built here from synthetic timings)."""
    sys.path.insert(0, ROOT)
    import bench
    launches = [(M, K, N) for M in (16, 64, 256, 1024, 4096)
                for (K, N) in ((8192, 28672), (28672, 8192), (8192, 10240))]
    table = [dict(M=M, K=K, N=N, us=100.0, TFLOPs=1.0, roofline_frac=0.5, plan="tiled_bm128_bn256_s3")
             for (M, K, N) in launches]
    per_m = {str(M): dict(us=300.0, TFLOPs=1000.0, weight_GBps=4000.0, roofline_frac=0.5)
             for M in (16, 64, 256, 1024, 4096)}
    h = dict(t_step=5e-3, step_flops=6.05e12, step_wbytes=8.1e8, per_m=per_m, table=table,
             roof=dict(n=9, t=4.8e-3, flops=6.0e12, alg_bytes=3e9), frac_all=0.45)
    cpu = dict(value=0.05, unit="TFLOP/s", cores=16, kind="oracle", sample="x" * 120, seconds=12.0)
    base = dict(kind="y" * 80, ms_per_step=12.0, TFLOPs=500.0, w4_speedup=2.0,
                per_m_TFLOPs={str(M): 500.0 for M in (16, 64, 256, 1024, 4096)},
                torch_matmul_ms_per_step=6.0, w4_speedup_vs_torch_matmul=1.2)
    dec = dict(workload="z" * 160, ms_per_step=0.2, weight_GBps=2400.0, avg_launch_us=8.5,
               hbm_frac=0.3, read_ceiling_us_per_launch=4.7, gemm_over_read_time=1.8,
               launch="hip_graph")
    line = bench.build_line(h, 20, 3, 123456789, cpu, base, dec)
    text = json.dumps(line)
    assert len(text) < 4000, len(text)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in line, key
    r = line["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == bench.FP16_PEAK_TFLOPS
    assert abs(r["achieved"] - 6.0e12 / 4.8e-3 / 1e12) < 0.1
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert line["value"] == round(6.05e12 / 5e-3 / 1e12, 2) and line["unit"] == "TFLOP/s"
    assert "workload" in line["config"] and line["dtype"] == "fp16"


def test_small_summary_splits_the_dispatches_into_the_cases(tmp_path, monkeypatch):
    """--small-summary: GEMM dispatches go to the cases in order, `launches` each; a
    second-pass dispatch belongs to the call before it; other kernels (repack, copies) are
    skipped; durations come from the trace, bytes are scaled by the copy calibration."""
    sys.path.insert(0, ROOT)
    import bench
    md = tmp_path / "small.md"
    monkeypatch.setattr(bench, "SMALL_MD", str(md))
    cases = tmp_path / "cases.json"
    cases.write_text("noise\n" + json.dumps(dict(
        profile_small=[dict(cfg=3, K=1024, N=512, M=1, kind="dense", zero_points=True),
                       dict(cfg=4, K=2048, N=1024, M=64, kind="2:4", zero_points=False)],
        launches=2)) + "\n")
    sk = "void w4a16::(anonymous namespace)::skinny_kernel<4, 1, 8, 2, 1>(...)"
    tk = "void w4a16::(anonymous namespace)::tiled_kernel<4, 4, 3, 3, 4>(...)"
    fx = "void w4a16::(anonymous namespace)::tiled_fixup_kernel<4, 4, 4>(...)"
    rp = "void w4a16::(anonymous namespace)::repack_all_kernel(...)"
    trace = tmp_path / "t.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                          "End_Timestamp"])
        w.writeheader()
        for d, name, ns in [(1, rp, 5000), (2, sk, 3000), (3, sk, 5000), (4, rp, 9000),
                            (5, tk, 10000), (6, fx, 2000), (7, tk, 12000), (8, fx, 4000)]:
            w.writerow(dict(Dispatch_Id=d, Kernel_Name=name, Start_Timestamp=100, End_Timestamp=100 + ns))
    copy_kib = (256 << 20) / 1024.0
    seq = [(1, rp), (2, sk), (3, sk), (4, rp), (5, tk), (6, fx), (7, tk), (8, fx)]
    fetch, write, sq = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "s.csv"
    _write(fetch, "FETCH_SIZE", [(10, "copyBuffer", copy_kib / 2)] * 1 +
           [(11, "copyBuffer", copy_kib / 2), (12, "copyBuffer", copy_kib / 2)] +
           [(d, n, 100.0 if n != fx else 50.0) for d, n in seq])
    _write(write, "WRITE_SIZE", [(10, "copyBuffer", copy_kib), (11, "copyBuffer", copy_kib),
                                 (12, "copyBuffer", copy_kib)] + [(d, n, 10.0) for d, n in seq])
    rows = []
    for d, n in seq:
        rows += [(d, n, "SQ_WAVES", 64.0), (d, n, "GRBM_GUI_ACTIVE", 8000.0),
                 (d, n, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0), (d, n, "SQ_INSTS_VALU", 2000.0),
                 (d, n, "SQ_LDS_BANK_CONFLICT", 0.0)]
    with open(sq, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, n, c, v in rows:
            w.writerow(dict(Dispatch_Id=d, Kernel_Name=n, Counter_Name=c, Counter_Value=v))
    bench.small_summary(str(cases), str(trace), str(sq), str(fetch), str(write))
    text = md.read_text()
    assert "`skinny_kernel<4, 1, 8, 2, 1>` | 4.0 | 0.0 |" in text      # (3 + 5) / 2 us
    assert "`tiled_kernel<4, 4, 3, 3, 4>` | 14.0 | 0.214 |" in text    # (10 + 2 + 12 + 4) / 2 us
    # traffic: fetch x2 (half the copy read), write x1; tiled call = kernel + second pass
    wb, ab, _ = bench.algorithmic(64, 2048, 1024)
    ab += 2048 * 1024 // 4 + 2048 * 1024 // 8 - 2048 * 1024 // 2
    assert f"| {round(((150.0 * 2 + 20.0) * 1024) / ab, 3)} |" in text
    assert "| 0.5 |" in text  # MFMA busy: 512000 / 1024 / (8000 / 8)

#!/usr/bin/env python3
"""Benchmark of the fused W4A16 GEMM on one MI355X.

Workload (one "step"): the 70B-class large-layer sweep -- every (K, N) in
{(8192,28672), (28672,8192), (8192,10240)} times every M in {16, 64, 256, 1024, 4096},
group 128 along K, symmetric INT4, fp16 activations ~N(0,1), scales uniform in
[0.001, 0.01]: 15 launches of w4a16_gemm (automatic plans) through the C ABI, spanning
the memory-bound (M = 16, 64) and the matrix-bound (M >= 256) regimes.  Inputs are
seeded, synthetic, repacked once and resident in HBM before timing; every launch of a
step reads its own copy of the weights (1.36 GiB in all), so none finds them in L2 or
the 256 MiB Infinity Cache.

Prints ONE JSON line (the last line of stdout).  `value` is the step's algorithmic
TFLOP/s (2MNK summed over the 15 GEMMs / step time); the line also carries the weight
GB/s, per-M figures with their roofline fractions, the roofline object of the dominant
kernel (the tiled kernel at M >= 256, timed with HIP events on its stream), the CPU
oracle timed on this host, the hand-written fp16 dequantize-then-GEMM baseline on the
same step, and a compact summary of the 7B-class decode sweep (M = 1..32, memory-bound).
Per-launch tables and the side legs go to --detail.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP16_PEAK_TFLOPS = 2516.6
FP8_PEAK_TFLOPS = 5033.2  # dense fp8 matrix peak (twice fp16)
ROTATE_BYTES = 1 << 30


def algorithmic(M, K, N, group=128):
    """Bytes and flops the method must move / compute for one GEMM."""
    wbytes = K * N // 2 + 2 * (K // group) * N
    return wbytes, wbytes + 2 * M * K + 2 * M * N, 2 * M * N * K


def roof(M, K, N, t, group=128, sparse=False, zero_points=False):
    """Which roofline bounds one GEMM and the fraction of it reached in t seconds:
    t_mem = algorithmic bytes / 8 TB/s, t_mfma = algorithmic flops / fp16 dense peak
    (2:4: M*N*K useful flops; zero-points add K*N/256 weight bytes)."""
    wb, ab, fl = algorithmic(M, K, N, group)
    if zero_points:
        wb += K * N // 256
        ab += K * N // 256
    if sparse:
        wb = K * N // 4 + K * N // 8 + 2 * (K // group) * N
        ab = wb + 2 * M * K + 2 * M * N
        fl = M * N * K
    t_mem = ab / (HBM_PEAK_GBPS * 1e9)
    t_mfma = fl / (FP16_PEAK_TFLOPS * 1e12)
    return dict(bound="hbm" if t_mem >= t_mfma else "mfma",
                roofline_frac=round(max(t_mem, t_mfma) / t, 4))


KERNEL_SOURCES = {"skinny": ("gemm_skinny.hip", "internal.h"),
                  "tiled": ("gemm_tiled.hip", "internal.h")}
TRAFFIC_JSON = {"skinny": os.path.join(ROOT, "profiles", "w4a16_gemm_decode_sweep_traffic.json"),
                "tiled": os.path.join(ROOT, "profiles", "w4a16_tiled_70b_traffic.json")}


def kernel_sha(kind="skinny"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "w4a16_mixed_precision_offline_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kind="tiled"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    p = TRAFFIC_JSON[kind]
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha(kind):
        return None
    return t.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20
PMC_COMMANDS = {
    "tiled": "python -u bench.py --roofline-only --steps 2 --warmup 1 --copy-calibration",
    "skinny": "python -u bench.py --only-decode --copy-calibration",
}


def pmc_summary(fetch_csv, write_csv, kind="tiled"):
    """HBM bytes per fused-GEMM call from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that makes the same counter read the known
    size of a plain 256 MiB device copy in the same run.  kind "tiled": the calls of the
    roofline set (a tiled_kernel dispatch plus, where tiles are cut, its tiled_fixup_kernel
    dispatch); kind "skinny": the skinny_kernel dispatches of the decode sweep."""
    import csv

    def per_dispatch(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = out.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "v": 0.0})
            d["v"] += float(r["Counter_Value"])
        return out

    main = "skinny_kernel" if kind == "skinny" else "tiled_kernel"
    extra = None if kind == "skinny" else "tiled_fixup_kernel"
    res = {}
    for tag, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        disp = per_dispatch(path, counter)
        copies = [d["v"] for d in disp.values() if "copyBuffer" in d["name"]]
        calls = [d["v"] for d in disp.values() if main in d["name"]]
        fix = [d["v"] for d in disp.values() if extra and extra in d["name"]]
        if not copies or not calls:
            raise SystemExit(f"{path}: no copy or no GEMM dispatches with {counter}")
        # the copies are the largest copyBuffer dispatches (the known-size calibration)
        copies.sort()
        calib = copies[-3:]
        factor = (COPY_BYTES / 1024.0) / (sum(calib) / len(calib))
        res[tag] = dict(factor=factor, kib_per_launch=(sum(calls) + sum(fix)) / len(calls),
                        launches=len(calls), fixups=len(fix), copy_kib=sum(calib) / len(calib))
    hbm = (res["fetch"]["kib_per_launch"] * res["fetch"]["factor"] +
           res["write"]["kib_per_launch"] * res["write"]["factor"]) * 1024.0
    cmd = PMC_COMMANDS[kind]
    out = dict(kernel_sha=kernel_sha(kind), hbm_bytes_per_launch=int(hbm),
               fetch_factor=round(res["fetch"]["factor"], 4), write_factor=round(res["write"]["factor"], 4),
               fetch_kib_per_launch=round(res["fetch"]["kib_per_launch"], 1),
               write_kib_per_launch=round(res["write"]["kib_per_launch"], 1),
               launches=res["fetch"]["launches"], fixup_dispatches=res["fetch"]["fixups"],
               commands=[f"rocprofv3 --pmc {c} -d {os.path.dirname(p)} -o run --output-format csv -- {cmd}"
                         for c, p in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))]
               + [f"python bench.py --pmc-kind {kind} --pmc-summary {fetch_csv} {write_csv}"])
    with open(TRAFFIC_JSON[kind], "w") as f:
        json.dump(out, f, indent=1)
    # the same figures as a short table beside the JSON
    alg = (20562816 if kind == "skinny" else 205258752)  # algorithmic bytes per call
    what = ("the 24 decode-sweep GEMMs (`skinny_kernel`), each equally often" if kind == "skinny"
            else "the w4a16_gemm calls at M >= 256 of the 70B-class step (`tiled_kernel` "
                 "dispatches, with the bytes of their `tiled_fixup_kernel` passes counted in)")
    md = [f"# {'Skinny' if kind == 'skinny' else 'Tiled'} kernel: HBM traffic per call "
          "(rocprofv3 counters)", "", "Commands (repository root, one MI355X):", "", "```",
          *out["commands"], "```", "",
          "Calibration: the same runs copy 256 MiB device-to-device three times "
          f"(`--copy-calibration`); FETCH_SIZE reads {1 / out['fetch_factor']:.4f} of the known "
          f"copy size and WRITE_SIZE {1 / out['write_factor']:.4f} of it, so the per-dispatch "
          f"figures are scaled by {out['fetch_factor']} and {out['write_factor']}.", "",
          "| quantity | value |", "|---|---|",
          f"| calls measured | {out['launches']}: {what} |",
          f"| FETCH_SIZE per call (raw) | {out['fetch_kib_per_launch']} KiB |",
          f"| WRITE_SIZE per call (raw) | {out['write_kib_per_launch']} KiB |",
          f"| HBM bytes per call (scaled) | {out['hbm_bytes_per_launch']} |",
          f"| algorithmic bytes per call | {alg} |",
          f"| traffic / algorithmic | {out['hbm_bytes_per_launch'] / alg:.3f} |", "",
          f"Kernel source hash the counters belong to: `{out['kernel_sha']}` (bench.py reports "
          "`traffic` only while the sources hash to it)."]
    with open(TRAFFIC_JSON[kind][:-5] + ".md", "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(out))


TRACE_MD = {"tiled": os.path.join(ROOT, "profiles", "w4a16_tiled_70b_kernel_trace.md"),
            "skinny": os.path.join(ROOT, "profiles", "w4a16_skinny_decode_sweep_kernel_trace.md")}
TRACE_COMMAND = {
    "tiled": ("rocprofv3 --kernel-trace --stats -d rocprof/kt_tiled -o run --output-format csv "
              "-- python -u bench.py --steps 20 --warmup 3 --no-cpu --no-baseline --no-decode"),
    "skinny": ("rocprofv3 --kernel-trace --stats -d rocprof/kt_skinny -o run --output-format csv "
               "-- python -u bench.py --only-decode"),
}


def trace_summary(csv_path, bench_line_path=None, kind="tiled"):
    """Per-kernel durations from a rocprofv3 kernel trace (CSV), and the per-call duration
    of the kernel the bench line's roofline figure covers.  kind "tiled" (the headline): the
    packed-weight tiled kernel with 128-row tiles (template <8, *, *, 0>, the M >= 256
    launches) plus the stream-K fixup passes of those calls (<8, *>), divided by the number
    of such tiled-kernel launches.  kind "skinny" (the decode sweep, --only-decode): every
    skinny_kernel launch.  Writes the markdown summary into profiles/ next to the bench line
    of the same command."""
    import csv
    import re
    rows = list(csv.DictReader(open(csv_path)))
    stats = {}
    roof_t, roof_calls = 0.0, 0
    for r in rows:
        name = r.get("Kernel_Name", "")
        t = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3  # ns -> us
        m = re.search(r"(\w+_kernel)<([^>]*)>", name)
        short = f"{m.group(1)}<{m.group(2)}>" if m else name[:60]
        st = stats.setdefault(short, [0, 0.0, 1e30, 0.0])
        st[0] += 1
        st[1] += t
        st[2] = min(st[2], t)
        st[3] = max(st[3], t)
        if kind == "skinny":
            if m and m.group(1) == "skinny_kernel":
                roof_t += t
                roof_calls += 1
        elif m and m.group(1) == "tiled_kernel":
            a = [int(x) for x in m.group(2).split(",")]
            if a[0] == 8 and a[3] == 0:
                roof_t += t
                roof_calls += 1
        elif m and m.group(1) == "tiled_fixup_kernel":
            a = [int(x) for x in m.group(2).split(",")]
            if a[0] == 8:
                roof_t += t
    title = ("Tiled kernel on the 70B-class sweep" if kind == "tiled"
             else "Skinny kernel on the 7B-class decode sweep")
    lines = [f"# {title}: kernel durations (rocprofv3 kernel trace)", "",
             "Command (repository root, one MI355X):", "", "```", TRACE_COMMAND[kind],
             f"python bench.py --trace-kind {kind} --trace-summary "
             f"rocprof/{'kt_tiled' if kind == 'tiled' else 'kt_skinny'}/run_kernel_trace.csv"
             + (" <the bench line of that run, as a JSON file>" if bench_line_path else ""),
             "```", "",
             "| kernel (template args) | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for k in sorted(stats):
        c, tot, mn, mx = stats[k]
        lines.append(f"| `{k}` | {c} | {tot / c:.3f} | {mn:.3f} | {mx:.3f} |")
    per_call = roof_t / max(1, roof_calls)
    what = ("Roofline set (w4a16_gemm at M >= 256: `tiled_kernel<8, *, *, 0>` plus its "
            "`tiled_fixup_kernel<8, *>` passes)" if kind == "tiled"
            else "Every `skinny_kernel` launch (the 24 GEMMs of the decode sweep, each equally often)")
    lines += ["", f"{what}: {roof_calls} calls, **{per_call:.2f} us** per call (warmup and timed "
                  "steps; each step has the same launches)."]
    if bench_line_path:
        line = json.load(open(bench_line_path))
        if kind == "skinny":
            line = line["decode_sweep"]
            ev = line["avg_launch_us"]
        else:
            line = line["roofline"]
            ev = line["avg_launch_us"]
        src = ("the run traced above" if kind == "tiled" else
               "a run of the same workload without the profiler (under the tracer the "
               "graph replays of these few-microsecond kernels gain gaps between launches)")
        lines += ["", f"The bench line of {src} measured {ev:.2f} us per call with HIP "
                      f"events on the kernels' stream (`avg_launch_us`): "
                      f"{100 * (ev / per_call - 1):+.1f}% from the kernel durations above "
                      "(the events also hold the gaps between launches).",
                  "", "```", json.dumps(line), "```"]
    out = "\n".join(lines) + "\n"
    with open(TRACE_MD[kind], "w") as f:
        f.write(out)
    print(out)


_SIDE = {}


def time_rotated(torch, calls, min_reps=20, target_s=0.02, graph=True):
    """Seconds per call, cycling through `calls` (one per weight copy) back to back.
    After a 20 ms eager warmup on a side stream (which also sizes the library's
    per-stream split-K workspace), the calls are captured once into a HIP graph that is
    replayed until at least `min_reps` calls ran: eager launches from Python would time
    the host's launch rate, not the GPU, for kernels of a few microseconds.  graph=False
    times eager launches (calls that synchronize with the host cannot be captured)."""
    s = _SIDE.setdefault("s", torch.cuda.Stream())
    t0 = time.perf_counter()
    i = 0
    with torch.cuda.stream(s):
        while time.perf_counter() - t0 < 0.02:
            calls[i % len(calls)]()
            i += 1
    torch.cuda.synchronize()
    g = None
    try:
        if not graph:
            raise RuntimeError("not captured")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
    except Exception as e:  # capture unsupported: time eager launches instead
        if graph:
            print(f"bench.py: graph capture failed ({e}); timing eager launches", file=sys.stderr)
        g = None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = max(1, -(-min_reps // len(calls)))
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(reps):
            if g is not None:
                g.replay()
            else:
                for c in calls:
                    c()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (reps * len(calls))


def config_legs(w4, torch, group):
    """Config 4 (2:4 sparse): w4a16_sparse24_gemm against w4a16_gemm on the same pruned
    weights (the dense kernel reads them repacked, code 8 at pruned positions).
    Config 3 (zero-points, awkward shapes): w4a16_gemm with per-group zero-points.
    Seeded inputs from gen/ at the workloads' shapes; weights rotate over copies
    totalling at least 512 MiB so that no launch finds its weights in the 256 MiB
    Infinity Cache."""
    from gen import activations, config_runs, weights
    rot = 512 << 20
    sp_runs = []
    cache = {}
    for w in config_runs(4):
        K, N, M = w.K, w.N, w.M
        if (K, N) not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            d = weights(w)
            q = torch.from_numpy(d["Qp"]).cuda()
            s = torch.from_numpy(d["s"]).cuda()
            dense = w4.alloc_packed(K, N, group, False)
            w4.w4a16_repack(q, s, None, dense[0], dense[1], None, K, N, group)
            sparse = w4.alloc_sparse24(K, N, group)
            w4.w4a16_sparse24_repack(q, s, *sparse, K, N, group)
            del q, s
            nd = max(2, -(-rot // (K * N // 2)))
            ns = max(2, -(-rot // (K * N // 4 + K * N // 8)))
            cache[(K, N)] = ([dense] + [tuple(t.clone() if t is not None else None for t in dense)
                                        for _ in range(nd - 1)],
                             [sparse] + [tuple(t.clone() for t in sparse) for _ in range(ns - 1)])
        dcopies, scopies = cache[(K, N)]
        X = torch.from_numpy(activations(w)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        td = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(X, c[0], c[1], None, Y, M, N, K, group)
                                  for c in dcopies])
        ts = time_rotated(torch, [lambda c=c: w4.w4a16_sparse24_gemm(X, c[0], c[1], c[2], Y, M, N, K,
                                                                     group) for c in scopies])
        sbytes = K * N // 4 + K * N // 8 + 2 * (K // group) * N
        sp_runs.append(dict(M=M, K=K, N=N, dense_us=round(td * 1e6, 2), sparse_us=round(ts * 1e6, 2),
                            speedup=round(td / ts, 3),
                            sparse_weight_GBps=round(sbytes / ts / 1e9, 1),
                            sparse_roofline=roof(M, K, N, ts, group, sparse=True),
                            dense_roofline=roof(M, K, N, td, group),
                            dense_plan=w4.w4a16_gemm_describe(M, N, K, group)["name"]))
    del cache
    torch.cuda.empty_cache()
    sp = dict(kernel="w4a16_sparse24_gemm (v_smfmac_f32_16x16x64_f16) vs w4a16_gemm",
              mean_speedup=round(sum(r["speedup"] for r in sp_runs) / len(sp_runs), 3),
              runs=sp_runs)

    as_runs = []
    cache = {}
    for w in config_runs(3):
        K, N, M = w.K, w.N, w.M
        if (K, N) not in cache:
            cache.clear()
            d = weights(w)
            q = torch.from_numpy(d["Qp"]).cuda()
            s = torch.from_numpy(d["s"]).cuda()
            z = torch.from_numpy(d["Zp"]).cuda()
            pk = w4.alloc_packed(K, N, group, True)
            w4.w4a16_repack(q, s, z, *pk, K, N, group)
            n = max(2, -(-rot // (K * N // 2)))
            cache[(K, N)] = [pk] + [tuple(t.clone() for t in pk) for _ in range(n - 1)]
        copies = cache[(K, N)]
        X = torch.from_numpy(activations(w)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        t = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(X, c[0], c[1], c[2], Y, M, N, K, group)
                                 for c in copies])
        wb = K * N // 2 + 2 * (K // group) * N + (K // group) * N // 2
        as_runs.append(dict(M=M, K=K, N=N, us=round(t * 1e6, 2),
                            TFLOPs=round(2.0 * M * N * K / t / 1e12, 2),
                            weight_GBps=round(wb / t / 1e9, 1), **roof(M, K, N, t, group, zero_points=True),
                            plan=w4.w4a16_gemm_describe(M, N, K, group)["name"]))
    del cache
    torch.cuda.empty_cache()
    (w,) = config_runs(0)
    d = weights(w)
    pk = w4.alloc_packed(w.K, w.N, group, False)
    w4.w4a16_repack(torch.from_numpy(d["Qp"]).cuda(), torch.from_numpy(d["s"]).cuda(), None,
                    *pk, w.K, w.N, group)
    copies = [pk] + [tuple(t.clone() if t is not None else None for t in pk) for _ in range(63)]
    X = torch.from_numpy(activations(w)).cuda()
    Y = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    t = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(X, c[0], c[1], None, Y, w.M, w.N, w.K, group)
                             for c in copies])
    tiny = dict(M=w.M, K=w.K, N=w.N, us=round(t * 1e6, 2),
                TFLOPs=round(2.0 * w.M * w.N * w.K / t / 1e12, 2),
                weight_GBps=round(algorithmic(w.M, w.K, w.N, group)[0] / t / 1e9, 1),
                **roof(w.M, w.K, w.N, t, group),
                plan=w4.w4a16_gemm_describe(w.M, w.N, w.K, group)["name"])
    del copies, pk
    return sp, dict(kernel="w4a16_gemm with 4-bit zero-points", runs=as_runs), tiny


def group64_leg(w4, torch):
    """Groups of 64 and of 256 rows against groups of 128 on the same codes: decode shapes
    from the 7B-class sweep and one large-M layer, symmetric and with zero-points.  Seeded
    synthetic weights (codes uniform 0..15, scales U[0.002, 0.02], zero-points uniform
    0..15) generated on the device; weights rotate over copies totalling at least 512 MiB."""
    rot = 512 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(64)
    runs = []
    groups = (128, 64, 256)
    for (K, N, Ms) in [(4096, 11008, (1, 16, 32)), (8192, 10240, (1024,))]:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        packs = {}
        for g in groups:
            s = (torch.rand((K // g, N), device="cuda", generator=gen) * 0.018 + 0.002).half()
            z = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // g, N // 8), dtype=torch.int32,
                              device="cuda", generator=gen)
            for asym in (False, True):
                pk = w4.alloc_packed(K, N, g, asym)
                w4.w4a16_repack(q, s, z if asym else None, *pk, K, N, g)
                n = max(2, -(-rot // (K * N // 2)))
                packs[(g, asym)] = [pk] + [tuple(t.clone() if t is not None else None for t in pk)
                                           for _ in range(n - 1)]
        for M in Ms:
            X = torch.randn((M, K), device="cuda", generator=gen).half()
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            for asym in (False, True):
                t = {}
                for g in groups:
                    t[g] = time_rotated(torch, [lambda c=c, g=g: w4.w4a16_gemm(X, c[0], c[1], c[2], Y,
                                                                             M, N, K, g)
                                                for c in packs[(g, asym)]])
                runs.append(dict(M=M, K=K, N=N, zero_points=asym, g128_us=round(t[128] * 1e6, 2),
                                 g64_us=round(t[64] * 1e6, 2), g256_us=round(t[256] * 1e6, 2),
                                 g64_over_g128_time=round(t[64] / t[128], 3),
                                 g256_over_g128_time=round(t[256] / t[128], 3)))
            del X, Y
        del q, packs
        torch.cuda.empty_cache()
    return dict(kernel="w4a16_gemm with groups of 64 and 256 rows vs 128", runs=runs)


def bf16_leg(w4, torch):
    """bf16 activations (w4a16_gemm_bf16: skinny kernel up to 32 rows, fp16 rows on the
    tiled kernel above) against fp16 activations (w4a16_gemm) on the same repacked weights,
    at the decode-sweep shapes with M = 1 / 16 / 32 and on 8192 x 10240 with M = 64 / 256 /
    1024 / 4096.  Seeded synthetic inputs on the device; weights rotate over copies
    totalling at least 512 MiB."""
    rot = 512 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(16)
    runs = []
    for (K, N, Ms) in [(4096, 4096, (1, 16, 32)), (4096, 12288, (1, 16, 32)),
                       (11008, 4096, (1, 16, 32)), (8192, 10240, (64, 256, 1024, 4096))]:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        s = (torch.rand((K // 128, N), device="cuda", generator=gen) * 0.018 + 0.002).half()
        pk = w4.alloc_packed(K, N, 128, False)
        w4.w4a16_repack(q, s, None, *pk, K, N, 128)
        n = max(2, -(-rot // (K * N // 2)))
        copies = [pk] + [tuple(t.clone() if t is not None else None for t in pk) for _ in range(n - 1)]
        for M in Ms:
            x = torch.randn((M, K), device="cuda", generator=gen)
            Xh, Xb = x.half(), x.bfloat16()
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            Yb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            th = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(Xh, c[0], c[1], None, Y, M, N, K, 128)
                                      for c in copies])
            tb = time_rotated(torch, [lambda c=c: w4.w4a16_gemm_bf16(Xb, c[0], c[1], None, Yb, M, N, K,
                                                                     128) for c in copies])
            wb = K * N // 2 + 2 * (K // 128) * N
            runs.append(dict(M=M, K=K, N=N, fp16_us=round(th * 1e6, 2), bf16_us=round(tb * 1e6, 2),
                             bf16_over_fp16_time=round(tb / th, 3),
                             bf16_weight_GBps=round(wb / tb / 1e9, 1)))
        del q, s, pk, copies
        torch.cuda.empty_cache()
    return dict(kernel="w4a16_gemm_bf16 vs w4a16_gemm (same weights)", runs=runs)


def w4a8_leg(w4, torch):
    """FP8 E4M3 activations with per-row fp32 scales (w4a8_gemm, automatic plan: the fp8
    skinny kernel up to 32 rows, fp16 rows on the fp16 tiled kernel above) against fp16
    activations (w4a16_gemm, automatic plan) on the same repacked weights: decode shapes at
    M = 1 / 16 / 32 and a 70B-class layer at M = 16 / 64 / 256 / 1024 / 4096.  Seeded
    synthetic inputs (activations quantized per row on the host); weights rotate over
    copies totalling at least 512 MiB."""
    rot = 512 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(18)
    runs = []
    for (K, N), Ms in [((4096, 4096), (1, 16, 32)), ((4096, 12288), (1, 16, 32)),
                       ((11008, 4096), (1, 16, 32)), ((8192, 28672), (16, 64, 256, 1024, 4096))]:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        s = (torch.rand((K // 128, N), device="cuda", generator=gen) * 0.018 + 0.002).half()
        pk = w4.alloc_packed(K, N, 128, False)
        w4.w4a16_repack(q, s, None, *pk, K, N, 128)
        n = max(2, -(-rot // (K * N // 2)))
        copies = [pk] + [tuple(t.clone() if t is not None else None for t in pk) for _ in range(n - 1)]
        for M in Ms:
            x = torch.randn((M, K), device="cuda", generator=gen)
            Xh = x.half()
            a = (x.abs().amax(dim=1) / 448.0).float()
            X8 = (x / a[:, None]).cpu().to(torch.float8_e4m3fn).view(torch.uint8).cuda()
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            th = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(Xh, c[0], c[1], None, Y, M, N, K, 128)
                                      for c in copies])
            t8 = time_rotated(torch, [lambda c=c: w4.w4a8_gemm(X8, a, c[0], c[1], None, Y, M, N, K, 128)
                                      for c in copies])
            wb = K * N // 2 + 2 * (K // 128) * N
            fl = 2.0 * M * N * K
            # roofline of the fp8 path: weight + fp8 activation + fp16 output bytes at 8 TB/s
            # against fp8 matrix work at the dense fp8 peak
            t_mem = (wb + M * K + 2 * M * N) / (HBM_PEAK_GBPS * 1e9)
            t_mfma = fl / (FP8_PEAK_TFLOPS * 1e12)
            runs.append(dict(M=M, K=K, N=N, fp16_us=round(th * 1e6, 2), fp8_us=round(t8 * 1e6, 2),
                             fp8_over_fp16_time=round(t8 / th, 3),
                             fp8_weight_GBps=round(wb / t8 / 1e9, 1),
                             fp8_TFLOPs=round(fl / t8 / 1e12, 1),
                             bound="hbm" if t_mem >= t_mfma else "mfma_fp8",
                             roofline_frac=round(max(t_mem, t_mfma) / t8, 4),
                             plan=w4.w4a16_gemm_describe(M, N, K, 128)["name"]))
        del q, s, pk, copies
        torch.cuda.empty_cache()
    return dict(kernel="w4a8_gemm (E4M3 activations: skinny kernel v_mfma_f32_16x16x32_fp8_fp8, "
                       "tiled kernel v_mfma_scale_f32_16x16x128_f8f6f4) vs w4a16_gemm (same weights)",
                fp8_peak_TFLOPs=FP8_PEAK_TFLOPS, runs=runs)


def mxfp4_leg(w4, torch):
    """MXFP4 weights (E2M1 codes, E8M0 scale per 32 rows; w4a8_mx_gemm, the scales applied
    by the block-scaled matrix instruction, no unpacking) against INT4 weights with fp8
    activations (w4a8_gemm) and with fp16 activations (w4a16_gemm), same shapes and the
    same fp8 activations: the 70B-class layers at decode and prefill M.  Seeded synthetic
    inputs generated on the device (codes uniform, scale bytes uniform in [119, 124],
    X ~ N(0,1) quantized per row); weights rotate over copies totalling at least 512 MiB."""
    rot = 512 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20)
    runs = []
    for (K, N) in [(8192, 28672), (28672, 8192), (8192, 10240)]:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        s = (torch.rand((K // 128, N), device="cuda", generator=gen) * 0.018 + 0.002).half()
        e = torch.randint(119, 125, (K // 32, N), dtype=torch.uint8, device="cuda", generator=gen)
        pk = w4.alloc_packed(K, N, 128, False)
        w4.w4a16_repack(q, s, None, *pk, K, N, 128)
        mx = w4.alloc_mx(K, N)
        w4.w4a8_mx_repack(q, e, *mx, K, N)
        n = max(2, -(-rot // (K * N // 2)))
        copies = [(pk, mx)] + [((pk[0].clone(), pk[1].clone()), (mx[0].clone(), mx[1].clone()))
                               for _ in range(n - 1)]
        for M in (1, 16, 256, 1024, 4096):
            x = torch.randn((M, K), device="cuda", generator=gen)
            Xh = x.half()
            a = (x.abs().amax(dim=1) / 448.0).float()
            X8 = (x / a[:, None]).cpu().to(torch.float8_e4m3fn).view(torch.uint8).cuda()
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            th = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(Xh, c[0][0], c[0][1], None, Y, M, N,
                                                                 K, 128) for c in copies])
            t8 = time_rotated(torch, [lambda c=c: w4.w4a8_gemm(X8, a, c[0][0], c[0][1], None, Y, M,
                                                                N, K, 128) for c in copies])
            tm = time_rotated(torch, [lambda c=c: w4.w4a8_mx_gemm(X8, a, c[1][0], c[1][1], Y, M, N,
                                                                   K) for c in copies])
            wb = K * N // 2 + K * N // 32
            fl = 2.0 * M * N * K
            # roofline: weight + fp8 activation + fp16 output bytes at 8 TB/s against the
            # matrix work at the dense fp8 peak (the instruction's rate with an fp8 operand)
            t_mem = (wb + M * K + 2 * M * N) / (HBM_PEAK_GBPS * 1e9)
            t_mfma = fl / (FP8_PEAK_TFLOPS * 1e12)
            runs.append(dict(M=M, K=K, N=N, w4a16_us=round(th * 1e6, 2), w4a8_us=round(t8 * 1e6, 2),
                             mxfp4_us=round(tm * 1e6, 2), mxfp4_TFLOPs=round(fl / tm / 1e12, 1),
                             mxfp4_weight_GBps=round(wb / tm / 1e9, 1),
                             w4a8_over_mxfp4_time=round(t8 / tm, 3),
                             w4a16_over_mxfp4_time=round(th / tm, 3),
                             bound="hbm" if t_mem >= t_mfma else "mfma_fp8",
                             roofline_frac=round(max(t_mem, t_mfma) / tm, 4)))
        del q, s, e, pk, mx, copies
        torch.cuda.empty_cache()
    return dict(kernel="w4a8_mx_gemm (tiled kernel, v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 "
                       "codes and their E8M0 block scales) vs w4a8_gemm and w4a16_gemm",
                fp8_peak_TFLOPs=FP8_PEAK_TFLOPS, runs=runs)


def offline_leg(w4, torch):
    """The load-time kernels, timed apart from the GEMM (they run once per weight
    matrix): w4a16_repack (codes + scales, and zero-points), w4a16_unpack, the 2:4
    compress w4a16_sparse24_repack (its call includes the read-back of the 2:4 check, a
    host synchronization) and the baseline's w4a16_dequant.  Bytes are what each reads
    plus what it writes, once; the rate is set against the 8 TB/s HBM peak."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(19)
    runs = []
    for (K, N) in [(4096, 4096), (4096, 12288), (11008, 4096), (8192, 28672)]:
        G = K // 128
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        s = (torch.rand((G, N), device="cuda", generator=gen) * 0.018 + 0.002).half()
        z = torch.randint(-2 ** 31, 2 ** 31 - 1, (G, N // 8), dtype=torch.int32, device="cuda",
                          generator=gen)
        pk = w4.alloc_packed(K, N, 128, False)
        pz = w4.alloc_packed(K, N, 128, True)
        qb = torch.empty_like(q)
        sb = torch.empty_like(s)
        Wt = torch.empty((N, K), dtype=torch.float16, device="cuda")
        q24 = q & torch.tensor(0x00FF00FF, dtype=torch.int32, device="cuda")  # 2 of 4 nibbles = 0...
        q24 = q24 | torch.tensor(0x88008800 - (1 << 32), dtype=torch.int32, device="cuda")  # ...to code 8
        sv = w4.alloc_sparse24(K, N, 128)
        kn2, gn2 = K * N // 2, 2 * G * N
        items = [  # (name, call, bytes, capturable: the 2:4 compress reads its check back)
            ("w4a16_repack", lambda: w4.w4a16_repack(q, s, None, *pk, K, N, 128), 2 * (kn2 + gn2)),
            ("w4a16_repack_zero_points", lambda: w4.w4a16_repack(q, s, z, *pz, K, N, 128),
             2 * (kn2 + gn2 + G * N // 2)),
            ("w4a16_unpack", lambda: w4.w4a16_unpack(*pk, qb, sb, None, K, N, 128), 2 * (kn2 + gn2)),
            ("w4a16_dequant", lambda: w4.w4a16_dequant(q, s, None, Wt, K, N, 128), kn2 + gn2 + 2 * K * N),
            ("w4a16_sparse24_repack", lambda: w4.w4a16_sparse24_repack(q24, s, *sv, K, N, 128),
             kn2 + gn2 + K * N // 4 + K * N // 8 + gn2),
        ]
        for name, fn, nbytes in items:
            # ten calls per captured graph, so the graph launch itself is amortized
            t = time_rotated(torch, [fn] * 10, min_reps=10, graph=name != "w4a16_sparse24_repack")
            runs.append(dict(kernel=name, K=K, N=N, us=round(t * 1e6, 2), bytes=nbytes,
                             GBps=round(nbytes / t / 1e9, 1),
                             frac_of_hbm_peak=round(nbytes / t / 1e9 / HBM_PEAK_GBPS, 3)))
        del q, s, z, pk, pz, qb, sb, Wt, q24, sv
        torch.cuda.empty_cache()
    return dict(note="load-time kernels (once per weight matrix), not part of the GEMM metric",
                runs=runs)


def profile_tiled(w4, torch):
    """A short workload for counter runs: W4A16 (fp16 activations), W4A8 (fp8 E4M3
    activations, on the fp8 tiled variant 128 x 256: the automatic plan would rewrite the
    rows in fp16) and MXFP4 weights with fp8 activations (block scales inside the matrix
    instruction) on the tiled kernel, 8192 x 28672 at M = 4096, three eager launches each
    after one warmup launch; prints the per-launch times."""
    K, N, M = 8192, 28672, 4096
    gen = torch.Generator(device="cuda")
    gen.manual_seed(21)
    q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                      generator=gen)
    s = (torch.rand((K // 128, N), device="cuda", generator=gen) * 0.009 + 0.001).half()
    pk = w4.alloc_packed(K, N, 128, False)
    w4.w4a16_repack(q, s, None, *pk, K, N, 128)
    e = torch.randint(119, 125, (K // 32, N), dtype=torch.uint8, device="cuda", generator=gen)
    mx = w4.alloc_mx(K, N)
    w4.w4a8_mx_repack(q, e, *mx, K, N)
    x = torch.randn((M, K), device="cuda", generator=gen)
    Xh = x.half()
    a = (x.abs().amax(dim=1) / 448.0).float()
    X8 = (x / a[:, None]).cpu().to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    v8 = [v for v in range(w4.w4a16_gemm_variants())
          if w4.w4a16_gemm_variant_name(v) == "tiled_bm128_bn256_s3"][0]
    out = {}
    for name, fn in (("w4a16_gemm", lambda: w4.w4a16_gemm(Xh, pk[0], pk[1], None, Y, M, N, K, 128)),
                     ("w4a8_gemm", lambda: w4.w4a8_gemm_plan(X8, a, pk[0], pk[1], None, Y, M, N, K,
                                                             128, v8, 0)),
                     ("w4a8_mx_gemm", lambda: w4.w4a8_mx_gemm(X8, a, mx[0], mx[1], Y, M, N, K))):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / 3 * 1e3, 1)
    print(json.dumps(dict(profile_tiled=dict(M=M, K=K, N=N, us_per_launch=out))), flush=True)


HEADLINE_CFG = 2  # the large-layer sweep: 70B-class shapes, M = 16 .. 4096
ROOF_MIN_M = 256  # launches at or above this M form the roofline set (tiled kernel, MFMA-bound)


def headline_inputs(w4, torch, roofline_only=False):
    """Seeded synthetic inputs of the 70B-class large-layer sweep, resident in HBM: the
    three shapes' weights repacked once, one distinct device copy per launch of a step
    (15 copies, 1.36 GiB, so that no launch finds its weights in L2 or the 256 MiB
    Infinity Cache), X and Y for every (M, K, N), and the dequantized fp16 weights of the
    unfused baseline.  The launch list of one step is M outer, shape inner."""
    from gen import CONFIGS, activations, config_runs, weights
    runs = config_runs(HEADLINE_CFG)
    shapes = []
    for w in runs:
        if (w.K, w.N) not in shapes:
            shapes.append((w.K, w.N))
    Ms = [M for M in CONFIGS[HEADLINE_CFG]["Ms"] if M >= ROOF_MIN_M or not roofline_only]
    group = 128
    packed, fp16w, host = {}, {}, {}
    for (K, N) in shapes:
        w = next(r for r in runs if (r.K, r.N) == (K, N))
        d = weights(w)
        host[(K, N)] = dict(Qp=d["Qp"], s=d["s"])
        q = torch.from_numpy(d["Qp"]).cuda()
        s = torch.from_numpy(d["s"]).cuda()
        wp, sp, _ = w4.alloc_packed(K, N, group, False)
        w4.w4a16_repack(q, s, None, wp, sp, None, K, N, group)
        packed[(K, N)] = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(len(Ms) - 1)]
        if not roofline_only:
            Wt = torch.empty((N, K), dtype=torch.float16, device="cuda")
            w4.w4a16_dequant(q, s, None, Wt, K, N, group)
            fp16w[(K, N)] = Wt
        del q, s, d
    X, Y, Xh = {}, {}, {}
    for w in runs:
        if w.M not in Ms:
            continue
        a = activations(w)
        if w.M == ROOF_MIN_M:
            Xh[(w.K, w.N)] = a  # the CPU oracle's sample
        X[(w.M, w.K, w.N)] = torch.from_numpy(a).cuda()
        Y[(w.M, w.K, w.N)] = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    launches = [(M, K, N, i) for i, M in enumerate(Ms) for (K, N) in shapes]
    return dict(shapes=shapes, Ms=Ms, packed=packed, fp16w=fp16w, host=host, X=X, Y=Y, Xh=Xh,
                launches=launches, group=group)


def time_eager_steps(torch, stream, launch_fns, steps, warmup):
    """Runs `warmup` untimed steps, then `steps` timed steps of the launch functions in
    order on `stream`, with a HIP event recorded after every launch.  Returns (seconds per
    step, per-launch durations in seconds as [steps][launches]).  The durations are GPU
    event deltas on the stream the kernels run on; the host enqueues far ahead of the GPU
    (a step takes milliseconds of GPU time), so no host gap enters them after the first
    launches of the first step."""
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            for f in launch_fns:
                f()
    torch.cuda.synchronize()
    n = len(launch_fns)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n)] for _ in range(steps)]
    e0 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for st in range(steps):
            for i, f in enumerate(launch_fns):
                f()
                evs[st][i].record(stream)
    torch.cuda.synchronize()
    dur = []
    prev = e0
    for st in range(steps):
        row = []
        for i in range(n):
            row.append(prev.elapsed_time(evs[st][i]) / 1e3)
            prev = evs[st][i]
        dur.append(row)
    total = e0.elapsed_time(evs[-1][-1]) / 1e3
    return total / steps, dur


def roof_times(M, K, N, group=128):
    """(t_mem, t_mfma) in seconds: algorithmic bytes at the HBM peak, flops at the fp16
    dense matrix peak."""
    _, ab, fl = algorithmic(M, K, N, group)
    return ab / (HBM_PEAK_GBPS * 1e9), fl / (FP16_PEAK_TFLOPS * 1e12)


def headline_leg(w4, torch, inp, stream, steps, warmup, roofline_only=False):
    """The timed step of the 70B-class sweep through w4a16_gemm (automatic plans)."""
    group = inp["group"]
    fns = []
    for (M, K, N, c) in inp["launches"]:
        wp, sp = inp["packed"][(K, N)][c]
        fns.append(lambda X=inp["X"][(M, K, N)], Y=inp["Y"][(M, K, N)], wp=wp, sp=sp, M=M, K=K, N=N:
                   w4.w4a16_gemm(X, wp, sp, None, Y, M, N, K, group))
    t_step, dur = time_eager_steps(torch, stream, fns, steps, warmup)
    launches = inp["launches"]
    per_launch = [sum(d[i] for d in dur) / len(dur) for i in range(len(launches))]
    step_fl = sum(algorithmic(M, K, N)[2] for (M, K, N, _) in launches)
    step_w = sum(algorithmic(M, K, N)[0] for (M, K, N, _) in launches)
    # per M: the three shapes together
    per_m = {}
    for M in inp["Ms"]:
        idx = [i for i, l in enumerate(launches) if l[0] == M]
        t = sum(per_launch[i] for i in idx)
        fl = sum(algorithmic(*launches[i][:3])[2] for i in idx)
        wb = sum(algorithmic(*launches[i][:3])[0] for i in idx)
        tr = sum(max(roof_times(*launches[i][:3])) for i in idx)
        per_m[str(M)] = dict(us=round(t * 1e6, 1), TFLOPs=round(fl / t / 1e12, 1),
                             weight_GBps=round(wb / t / 1e9, 1), roofline_frac=round(tr / t, 3))
    # the roofline kernel: the tiled kernel at M >= 256 (MFMA-bound), one w4a16_gemm call
    # = its launch plus, where stripes cut tiles, the stream-K fixup launch
    ridx = [i for i, l in enumerate(launches) if l[0] >= ROOF_MIN_M]
    r_t = sum(per_launch[i] for i in ridx)
    r_fl = sum(algorithmic(*launches[i][:3])[2] for i in ridx)
    r_ab = sum(algorithmic(*launches[i][:3])[1] for i in ridx)
    table = [dict(M=M, K=K, N=N, us=round(per_launch[i] * 1e6, 2),
                  TFLOPs=round(algorithmic(M, K, N)[2] / per_launch[i] / 1e12, 1),
                  roofline_frac=round(max(roof_times(M, K, N)) / per_launch[i], 4),
                  plan=w4.w4a16_gemm_describe(M, N, K, group)["name"])
             for i, (M, K, N, _) in enumerate(launches)]
    return dict(t_step=t_step, step_flops=step_fl, step_wbytes=step_w, per_m=per_m, table=table,
                roof=dict(n=len(ridx), t=r_t, flops=r_fl, alg_bytes=r_ab),
                frac_all=sum(max(roof_times(*l[:3])) for l in launches) / sum(per_launch))


def fp16_baseline_leg(w4, torch, inp, stream, steps):
    """The unfused baseline on the same step: the fp16 weights the hand-written dequant
    kernel wrote (once, not timed), then the hand-written fp16 GEMM; torch's fp16 matmul
    (hipBLASLt) on the same weights as context.  fp16 weights are 4x the bytes, so the
    other shapes' weights between two uses of one shape's weights exceed the Infinity
    Cache: no copies are needed."""
    fns = [lambda X=inp["X"][(M, K, N)], Y=inp["Y"][(M, K, N)], Wt=inp["fp16w"][(K, N)], M=M, K=K, N=N:
           w4.w4a16_fp16_gemm(X, Wt, Y, M, N, K) for (M, K, N, _) in inp["launches"]]
    t16, dur = time_eager_steps(torch, stream, fns, steps, 1)
    tfn = [lambda X=inp["X"][(M, K, N)], Wt=inp["fp16w"][(K, N)]: torch.nn.functional.linear(X, Wt)
           for (M, K, N, _) in inp["launches"]]
    tt, _ = time_eager_steps(torch, stream, tfn, max(2, steps // 2), 1)
    per_launch = [sum(d[i] for d in dur) / len(dur) for i in range(len(fns))]
    per_m = {}
    for M in inp["Ms"]:
        idx = [i for i, l in enumerate(inp["launches"]) if l[0] == M]
        t = sum(per_launch[i] for i in idx)
        fl = sum(algorithmic(*inp["launches"][i][:3])[2] for i in idx)
        per_m[str(M)] = round(fl / t / 1e12, 1)
    return dict(t_step=t16, t_torch=tt, per_m_TFLOPs=per_m)


def decode_sweep_leg(w4, torch, steps, warmup, use_graph=True):
    """The 7B-class decode sweep (24 GEMMs, M = 1..32, memory-bound), weights rotated over
    copies totalling over 1 GiB, timed over HIP-graph replays; beside it a plain streaming
    read of the same packed codes, launch for launch (the achievable ceiling at these
    sizes).  Returns a compact summary and the per-launch table."""
    from gen import CONFIGS, activations, config_runs, weights
    runs = config_runs(1)
    shapes = []
    for w in runs:
        if (w.K, w.N) not in shapes:
            shapes.append((w.K, w.N))
    Ms = CONFIGS[1]["Ms"]
    group = 128
    step_wbytes = sum(algorithmic(1, K, N)[0] for (K, N) in shapes)
    per_step = len(Ms)
    cycle = max(1, -(-ROTATE_BYTES // (step_wbytes * per_step)))
    R = per_step * cycle
    packed = {}
    for (K, N) in shapes:
        d = weights(next(r for r in runs if (r.K, r.N) == (K, N)))
        q = torch.from_numpy(d["Qp"]).cuda()
        s = torch.from_numpy(d["s"]).cuda()
        wp, sp, _ = w4.alloc_packed(K, N, group, False)
        w4.w4a16_repack(q, s, None, wp, sp, None, K, N, group)
        packed[(K, N)] = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(R - 1)]
        del q, s
    Xs = {(w.M, w.K, w.N): torch.from_numpy(activations(w)).cuda() for w in runs}
    Ys = {k: torch.empty((k[0], k[2]), dtype=torch.float16, device="cuda") for k in Xs}
    stream = torch.cuda.Stream()
    probe_out = torch.zeros(4, dtype=torch.int32, device="cuda")

    def launches(step_idx):
        cyc = step_idx % cycle
        return [(M, K, N, cyc * per_step + i) for i, M in enumerate(Ms) for (K, N) in shapes]

    def gemm_step(step_idx):
        for (M, K, N, c) in launches(step_idx):
            wp, sp = packed[(K, N)][c]
            w4.w4a16_gemm(Xs[(M, K, N)], wp, sp, None, Ys[(M, K, N)], M, N, K, group)

    def read_step(step_idx):
        for (M, K, N, c) in launches(step_idx):
            w4.w4a16_probe_read(packed[(K, N)][c][0], K * N // 2, probe_out)

    def timed(run_step, nsteps):
        with torch.cuda.stream(stream):
            for i in range(max(warmup, cycle)):
                run_step(i)
        torch.cuda.synchronize()
        graphs = None
        if use_graph:
            graphs = []
            for c in range(cycle):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    run_step(c)
                graphs.append(g)
            with torch.cuda.stream(stream):
                for i in range(warmup):
                    graphs[i % cycle].replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for i in range(nsteps):
                if graphs is not None:
                    graphs[i % cycle].replay()
                else:
                    run_step(i)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / nsteps

    t = timed(gemm_step, steps)
    tr = timed(read_step, max(5, steps // 2))
    L = launches(0)
    n = len(L)
    wb = sum(algorithmic(M, K, N)[0] for (M, K, N, _) in L)
    ab = sum(algorithmic(M, K, N)[1] for (M, K, N, _) in L)
    out = dict(workload="decode-shape sweep, 7B-class: (K,N) in {(4096,4096),(4096,12288),"
                        "(4096,11008),(11008,4096)} x M in {1,2,4,8,16,32}; 24 GEMMs per step",
               ms_per_step=round(t * 1e3, 4), weight_GBps=round(wb / t / 1e9, 1),
               avg_launch_us=round(t / n * 1e6, 3),
               hbm_frac=round(ab / n / (t / n) / 1e9 / HBM_PEAK_GBPS, 4),
               read_ceiling_us_per_launch=round(tr / n * 1e6, 3),
               gemm_over_read_time=round(t / tr, 3), launch="hip_graph" if use_graph else "eager",
               algorithmic_bytes_per_launch=int(ab / n),
               traffic=traffic_from_profiles("skinny"))
    del packed, Xs, Ys
    torch.cuda.empty_cache()
    return out


def cpu_oracle_leg(inp):
    """The CPU oracle as it stands, on this host: the three 70B-class shapes at M = 256
    (unpack + exact fp64 dequant + fp64 matmul, NumPy), repeated until at least 10 s of
    work (bounded at 30 s); reported in TFLOP/s of the GEMM's algorithmic flops."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    passes = 0
    fl = 0
    while True:
        for (K, N) in inp["shapes"]:
            h = inp["host"][(K, N)]
            oracle.gemm(inp["Xh"][(K, N)], h["Qp"], h["s"], None, inp["group"])
            fl += 2.0 * ROOF_MIN_M * K * N
        passes += 1
        tc = time.perf_counter() - t0
        if tc >= 10.0 or tc * (passes + 1) / passes > 30.0:
            break
    return dict(value=round(fl / tc / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{passes} pass(es) over the three 70B-class shapes at M = {ROOF_MIN_M} "
                       "(unpack + exact fp64 dequant + fp64 matmul, NumPy)",
                seconds=round(tc, 2))


def build_line(h, steps, warmup, traffic, cpu, base, decode):
    """The one JSON line of the run (kept compact: the driver reads the tail of stdout)."""
    t_step = h["t_step"]
    r = h["roof"]
    n_roof = r["n"]
    roof_avg_s = r["t"] / n_roof
    achieved = r["flops"] / r["t"] / 1e12
    return {
        "metric": "W4A16 GEMM TFLOP/s + weight HBM GB/s vs M (1..4096), % of roofline",
        "value": round(h["step_flops"] / t_step / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "large-layer sweep, 70B-class: (K,N) in {(8192,28672),(28672,8192),"
                        "(8192,10240)} x M in {%s}, group 128 along K, symmetric INT4, fp16 X ~ "
                        "N(0,1), scales U[0.001,0.01]; %d GEMMs per step"
                        % (",".join(str(m) for m in inp_ms(h)), len(h["table"])),
            "launch": "eager, one HIP event after each launch",
            "weight_copies": len(h["table"]),
            "parallelism": "single GPU",
        },
        "weight_GBps": round(h["step_wbytes"] / t_step / 1e9, 1),
        "roofline_frac_all_launches": round(h["frac_all"], 4),
        "per_M": h["per_m"],
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": FP16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / FP16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "tiled_kernel (+ its stream-K fixup where tiles are cut): the w4a16_gemm "
                      "launches at M >= %d, %d per step" % (ROOF_MIN_M, n_roof),
            "avg_launch_us": round(roof_avg_s * 1e6, 2),
            "algorithmic_bytes_per_launch": int(r["alg_bytes"] / n_roof),
        },
        "cpu_baseline": cpu,
        "fp16_baseline": base,
        "decode_sweep": decode,
    }


SMALL_LAUNCHES = 24  # eager launches per case of --profile-small
SMALL_MD = os.path.join(ROOT, "profiles", "small_layers_and_2to4_counters.md")
SMALL_SQ = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_VALU_MFMA_BUSY_CYCLES "
            "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")


def small_cases():
    """Configuration 0 (tiny), every run of configuration 3 (zero-points, awkward shapes)
    and configuration 4 with the dense and the 2:4 kernel on the same pruned weights."""
    from gen import config_runs
    out = [(w, "dense") for w in config_runs(0)] + [(w, "dense") for w in config_runs(3)]
    for w in config_runs(4):
        out += [(w, "dense"), (w, "2:4")]
    return out


def profile_small(w4, torch, group=128):
    """--profile-small: SMALL_LAUNCHES eager launches of each case of small_cases(), one
    case after the other, weights rotated over copies of at least 512 MiB; for rocprofv3
    traces and counters, which --small-summary splits back into the cases by dispatch
    order.  Prints the case list as the last stdout line."""
    from gen import activations, weights
    rot = 512 << 20
    cases, cache = [], {}
    for w, kind in small_cases():
        K, N, M = w.K, w.N, w.M
        key = (w.cfg, K, N)
        if key not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            d = weights(w)
            q = torch.from_numpy(d["Qp"]).cuda()
            s = torch.from_numpy(d["s"]).cuda()
            z = torch.from_numpy(d["Zp"]).cuda() if d["Zp"] is not None else None
            dense = w4.alloc_packed(K, N, group, z is not None)
            w4.w4a16_repack(q, s, z, *dense, K, N, group)
            nd = max(2, -(-rot // (K * N // 2)))
            ent = dict(dense=[dense] + [tuple(t.clone() if t is not None else None for t in dense)
                                        for _ in range(nd - 1)])
            if w.sparse24:
                sp = w4.alloc_sparse24(K, N, group)
                w4.w4a16_sparse24_repack(q, s, *sp, K, N, group)
                ns = max(2, -(-rot // (K * N // 4 + K * N // 8)))
                ent["2:4"] = [sp] + [tuple(t.clone() for t in sp) for _ in range(ns - 1)]
            cache[key] = ent
            del q, s, z
        X = torch.from_numpy(activations(w)).cuda()
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        if kind == "dense":
            calls = [lambda c=c: w4.w4a16_gemm(X, c[0], c[1], c[2], Y, M, N, K, group)
                     for c in cache[key]["dense"]]
        else:
            calls = [lambda c=c: w4.w4a16_sparse24_gemm(X, c[0], c[1], c[2], Y, M, N, K, group)
                     for c in cache[key]["2:4"]]
        for i in range(SMALL_LAUNCHES):
            calls[i % len(calls)]()
        torch.cuda.synchronize()
        cases.append(dict(cfg=w.cfg, K=K, N=N, M=M, kind=kind, zero_points=w.asym))
    print(json.dumps(dict(profile_small=cases, launches=SMALL_LAUNCHES)), flush=True)


def small_summary(cases_path, trace_csv, sq_csv, fetch_csv, write_csv):
    """Per-case figures of a --profile-small run: kernel and duration per call from the
    kernel trace (the stream-K second pass counted in), HBM traffic from FETCH_SIZE /
    WRITE_SIZE scaled by a plain 256 MiB copy in the same run, and SQ counters.  The
    GEMM dispatches are assigned to the cases in order, SMALL_LAUNCHES each; a second-pass
    dispatch belongs to the call before it.  Writes SMALL_MD."""
    import csv
    import re
    info = None
    for ln in open(cases_path):
        if ln.startswith('{"profile_small"'):
            info = json.loads(ln)
    if info is None:
        raise SystemExit(f"{cases_path}: no profile_small line")
    cases, L = info["profile_small"], info["launches"]

    def is_main(n):
        return "skinny_kernel" in n or "tiled_kernel<" in n

    def assign(disp):
        """disp: [(name, value)] in dispatch order -> per case [main values], [fixup values]."""
        per = [([], [], []) for _ in cases]
        c, n = 0, 0
        for name, v in disp:
            if is_main(name):
                if n == L:
                    c, n = c + 1, 0
                per[c][0].append(v)
                per[c][2].append(name)
                n += 1
            elif "tiled_fixup_kernel" in name and n > 0:
                per[c][1].append(v)
        if c != len(cases) - 1 or n != L:
            raise SystemExit(f"dispatches do not split into {len(cases)} cases of {L}")
        return per

    def counters(path):
        by = {}
        for r in csv.DictReader(open(path)):
            d = by.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [by[k] for k in sorted(by)]

    trace = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Dispatch_Id"]))
    tper = assign([(r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                   for r in trace])
    sq = counters(sq_csv)
    sper = assign([(d["name"], d) for d in sq])
    traffic = []
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        disp = counters(path)
        cop = sorted(d[counter] for d in disp if "copyBuffer" in d["name"] and counter in d)[-3:]
        factor = (COPY_BYTES / 1024.0) / (sum(cop) / len(cop))
        traffic.append((assign([(d["name"], d.get(counter, 0.0)) for d in disp]), factor))
    rows = []
    for i, cs in enumerate(cases):
        M, K, N = cs["M"], cs["K"], cs["N"]
        main_t, fix_t, names = tper[i]
        t_us = (sum(main_t) + sum(fix_t)) / L
        m = re.search(r"(skinny_kernel|tiled_kernel)<([^>]*)>", names[0])
        kern = f"{m.group(1)}<{m.group(2)}>" if m else names[0][:40]
        wb, ab, fl = algorithmic(M, K, N)
        if cs["zero_points"]:
            ab += K * N // 256
        if cs["kind"] == "2:4":
            ab += K * N // 4 + K * N // 8 - K * N // 2
        hbm = 0.0
        for per, factor in traffic:
            hbm += (sum(per[i][0]) + sum(per[i][1])) / L * factor * 1024.0
        sm = sper[i][0]

        def avg(c):
            return sum(d.get(c, 0.0) for d in sm) / len(sm)
        grbm = avg("GRBM_GUI_ACTIVE") / 8
        rows.append(dict(cfg=cs["cfg"], shape=f"{K}x{N}", M=M, kind=cs["kind"], kernel=kern,
                         us=round(t_us, 2),
                         fixup_share=round(sum(fix_t) / L / t_us, 3) if fix_t else 0.0,
                         alg_frac=round(ab / (t_us * 1e-6) / (HBM_PEAK_GBPS * 1e9), 3),
                         traffic_ratio=round(hbm / ab, 3), waves=int(avg("SQ_WAVES")),
                         mfma_busy=round(avg("SQ_VALU_MFMA_BUSY_CYCLES") / 1024 / grbm, 3) if grbm else 0,
                         valu_k=round(avg("SQ_INSTS_VALU") / 1e3, 1),
                         lds_conflict_k=round(avg("SQ_LDS_BANK_CONFLICT") / 1e3, 1)))
    cmds = [f"rocprofv3 --kernel-trace --stats -d {os.path.dirname(trace_csv)} -o run --output-format csv "
            "-- python -u bench.py --profile-small",
            f"rocprofv3 --pmc {SMALL_SQ} -d {os.path.dirname(sq_csv)} -o run --output-format csv "
            "-- python -u bench.py --profile-small"]
    cmds += [f"rocprofv3 --pmc {c} -d {os.path.dirname(p_)} -o run --output-format csv -- python -u "
             "bench.py --profile-small --copy-calibration"
             for c, p_ in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))]
    cmds.append(f"python bench.py --small-summary <the last stdout line of the trace run, as a file> "
                f"{trace_csv} {sq_csv} {fetch_csv} {write_csv}")
    md = ["# Small and awkward layers (configurations 0 and 3) and 2:4 against dense "
          "(configuration 4): kernel trace and counters", "",
          "Commands (repository root, one MI355X; each counter pass in its own run):", "", "```",
          *cmds, "```", "",
          f"Each case runs {L} eager launches of the automatic plan (weights rotated over copies of "
          "at least 512 MiB); the figures are means per call. `us`: kernel duration from the "
          "trace, the stream-K second pass included (`2nd pass`: its share). `HBM frac`: "
          "algorithmic bytes (codes, scales, zero-points, X and Y) / duration / 8 TB/s. "
          "`traffic`: FETCH_SIZE and WRITE_SIZE of the call, scaled by a plain 256 MiB copy in "
          f"the same runs (factors {traffic[0][1]:.4f} and {traffic[1][1]:.4f}), over the "
          "algorithmic bytes. `MFMA busy`: SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over "
          "GRBM_GUI_ACTIVE / 8 XCDs. `VALU`: SQ_INSTS_VALU per call (thousands, MFMA "
          "included). `LDS conflicts`: SQ_LDS_BANK_CONFLICT cycles per call (thousands). "
          "Counter runs serialize dispatches, so durations come from the trace run only.", "",
          "| cfg | layer | M | weights | kernel | us | 2nd pass | HBM frac | traffic | waves | "
          "MFMA busy | VALU (k) | LDS conflicts (k) |",
          "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {r['cfg']} | {r['shape']} | {r['M']} | {r['kind']} | `{r['kernel']}` | {r['us']} | "
                  f"{r['fixup_share']} | {r['alg_frac']} | {r['traffic_ratio']} | {r['waves']} | "
                  f"{r['mfma_busy']} | {r['valu_k']} | {r['lds_conflict_k']} |")
    with open(SMALL_MD, "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rows))


def copy_calibration(torch):
    """Three plain device copies of COPY_BYTES: the known-size traffic that scales the
    FETCH_SIZE / WRITE_SIZE counters of the same run."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-baseline", action="store_true", help="skip the fp16 baseline")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-sweep leg")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the roofline set (M >= 256 launches of the step), for profiler runs")
    ap.add_argument("--detail", default=None, help="write per-launch tables and extra legs (JSON) here")
    ap.add_argument("--all-legs", action="store_true",
                    help="also run the side legs (configs 0/3/4, groups of 64/256, bf16, fp8, "
                         "MXFP4, load-time kernels) into the --detail file")
    ap.add_argument("--profile-tiled", action="store_true",
                    help="only a short W4A16 / W4A8 tiled-kernel workload (for counter runs)")
    ap.add_argument("--only-activations", action="store_true",
                    help="run only the bf16 and fp8 activation legs (w4a16_gemm_bf16, w4a8_gemm "
                         "beside w4a16_gemm) and print them, e.g. under a kernel trace of the "
                         "row conversion")
    ap.add_argument("--only-mxfp4", action="store_true",
                    help="only the MXFP4 leg (for a kernel trace of its kernels)")
    ap.add_argument("--profile-small", action="store_true",
                    help="configurations 0, 3 and 4 (dense and 2:4), a fixed number of eager "
                         "launches each, for rocprofv3 traces and counters")
    ap.add_argument("--small-summary", nargs=5,
                    metavar=("CASES", "TRACE_CSV", "SQ_CSV", "FETCH_CSV", "WRITE_CSV"), default=None,
                    help="summarize the rocprofv3 runs of --profile-small into profiles/ and exit")
    ap.add_argument("--only-decode", action="store_true",
                    help="only the decode-sweep leg (for counter runs of the skinny kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain device copies of known size (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "this script into profiles/ and exit")
    ap.add_argument("--pmc-kind", choices=("tiled", "skinny"), default="tiled",
                    help="which kernel --pmc-summary summarizes")
    ap.add_argument("--trace-kind", choices=("tiled", "skinny"), default="tiled",
                    help="which kernel --trace-summary summarizes")
    ap.add_argument("--trace-summary", nargs="+", metavar="CSV", default=None,
                    help="summarize a rocprofv3 kernel trace of the headline run (and the "
                         "bench line it printed, as a JSON file) into profiles/ and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, kind=args.pmc_kind)
        return
    if args.trace_summary:
        trace_summary(*args.trace_summary, kind=args.trace_kind)
        return
    if args.small_summary:
        small_summary(*args.small_summary)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; the W4A16 GEMM has no multi-GPU "
              "path here (it would shard by output columns with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import w4a16_mixed_precision_offline_amd as w4

    torch.cuda.set_device(0)
    if args.profile_tiled:
        profile_tiled(w4, torch)
        return
    if args.only_mxfp4:
        print(json.dumps(dict(mxfp4_in_mfma_dequant=mxfp4_leg(w4, torch))), flush=True)
        return
    if args.only_activations:
        print(json.dumps(dict(bf16_activations=bf16_leg(w4, torch))), flush=True)
        print(json.dumps(dict(w4a8_fp8_activations=w4a8_leg(w4, torch))), flush=True)
        return
    if args.profile_small:
        if args.copy_calibration:
            copy_calibration(torch)
        profile_small(w4, torch)
        return
    if args.only_decode:
        if args.copy_calibration:
            copy_calibration(torch)
        print(json.dumps(dict(decode_sweep=decode_sweep_leg(w4, torch, 5, 2))), flush=True)
        return

    stream = torch.cuda.Stream()
    inp = headline_inputs(w4, torch, roofline_only=args.roofline_only)
    if args.copy_calibration:
        copy_calibration(torch)
    print(f"bench.py: inputs resident, timing {args.steps} steps", file=sys.stderr, flush=True)
    h = headline_leg(w4, torch, inp, stream, args.steps, args.warmup, args.roofline_only)
    t_step = h["t_step"]
    traffic = traffic_from_profiles("tiled")

    base = None
    if not args.no_baseline and not args.roofline_only:
        b = fp16_baseline_leg(w4, torch, inp, stream, max(3, args.steps // 2))
        base = dict(kind="w4a16_dequant (once) + w4a16_fp16_gemm, hand-written, fp16 weights",
                    ms_per_step=round(b["t_step"] * 1e3, 3),
                    TFLOPs=round(h["step_flops"] / b["t_step"] / 1e12, 1),
                    w4_speedup=round(b["t_step"] / t_step, 3),
                    per_m_TFLOPs=b["per_m_TFLOPs"],
                    torch_matmul_ms_per_step=round(b["t_torch"] * 1e3, 3),
                    w4_speedup_vs_torch_matmul=round(b["t_torch"] / t_step, 3))
    cpu = None
    if not args.no_cpu and not args.roofline_only:
        print("bench.py: CPU oracle leg", file=sys.stderr, flush=True)
        cpu = cpu_oracle_leg(inp)
    detail = dict(headline_table=h["table"])
    del inp
    torch.cuda.empty_cache()

    decode = None
    if not args.no_decode and not args.roofline_only:
        print("bench.py: decode-sweep leg", file=sys.stderr, flush=True)
        decode = decode_sweep_leg(w4, torch, 30, 5)

    if args.all_legs:
        print("bench.py: side legs", file=sys.stderr, flush=True)
        sparse24, asym, tiny = config_legs(w4, torch, 128)
        detail.update(sparse24_vs_dense=sparse24, asym_zero_point=asym, tiny_config=tiny,
                      group64_and_256=group64_leg(w4, torch), bf16_activations=bf16_leg(w4, torch),
                      w4a8_fp8_activations=w4a8_leg(w4, torch),
                      mxfp4_in_mfma_dequant=mxfp4_leg(w4, torch),
                      load_time_kernels=offline_leg(w4, torch))
    detail_path = args.detail
    if detail_path is None and args.all_legs:
        os.makedirs(os.path.join(ROOT, "bench_out"), exist_ok=True)
        detail_path = os.path.join(ROOT, "bench_out", "bench_detail.json")

    line = build_line(h, args.steps, args.warmup, traffic, cpu, base, decode)
    if detail_path:
        with open(detail_path, "w") as f:
            json.dump(dict(line=line, **detail, kernel_sha_tiled=kernel_sha("tiled"),
                           kernel_sha_skinny=kernel_sha("skinny")), f, indent=1)
    print(json.dumps(line), flush=True)


def inp_ms(h):
    ms = []
    for row in h["table"]:
        if row["M"] not in ms:
            ms.append(row["M"])
    return ms


if __name__ == "__main__":
    main()

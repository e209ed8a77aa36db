#!/usr/bin/env python3
"""Benchmark of the fused W4A16 GEMM on one MI355X.

Workload (one "step"): the 7B-class decode sweep -- every (K, N) in
{(4096,4096), (4096,12288), (4096,11008), (11008,4096)} times every M in
{1,2,4,8,16,32}, group 128 along K, symmetric INT4, fp16 activations ~N(0,1),
scales uniform in [0.002, 0.02]: 24 launches of w4a16_gemm through the C ABI.
Inputs are seeded, synthetic, repacked once and resident in HBM before timing.

Weights are rotated over enough distinct device copies that no launch reads
weights an earlier launch left in L2 or the 256 MiB Infinity Cache (every weight
byte a launch reads was last touched more than 1 GiB of weight traffic earlier),
as in decoding where each layer's weights are read once per token.  Activations
may stay cached.

Prints ONE JSON line.  `value` is the packed-weight HBM throughput of the whole
step (weight bytes of the 24 GEMMs / step time); the same line carries TFLOP/s,
the per-launch roofline figure, the fp16 (dequantize-then-GEMM) baseline on the
same shapes, and the CPU oracle timed on this host over one step.
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


def kernel_sha():
    h = hashlib.sha256()
    for f in ("gemm_skinny.hip", "internal.h"):
        with open(os.path.join(ROOT, "w4a16_mixed_precision_offline_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "w4a16_gemm_decode_sweep_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "w4a16_gemm_decode_sweep_traffic.json")


def pmc_summary(fetch_csv, write_csv):
    """HBM bytes per fused-GEMM launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that makes the same counter read the known
    size of a plain 256 MiB device copy in the same run."""
    import csv

    def per_dispatch(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = out.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "v": 0.0})
            d["v"] += float(r["Counter_Value"])
        return out

    res = {}
    for tag, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        disp = per_dispatch(path, counter)
        copies = [d["v"] for d in disp.values() if "copyBuffer" in d["name"]]
        gemms = [d["v"] for d in disp.values() if "skinny_kernel" in d["name"]]
        if not copies or not gemms:
            raise SystemExit(f"{path}: no copy or no GEMM dispatches with {counter}")
        # the copies are the largest copyBuffer dispatches (the known-size calibration)
        copies.sort()
        calib = copies[-3:]
        factor = (COPY_BYTES / 1024.0) / (sum(calib) / len(calib))
        res[tag] = dict(factor=factor, kib_per_launch=sum(gemms) / len(gemms), launches=len(gemms),
                        copy_kib=sum(calib) / len(calib))
    hbm = (res["fetch"]["kib_per_launch"] * res["fetch"]["factor"] +
           res["write"]["kib_per_launch"] * res["write"]["factor"]) * 1024.0
    out = dict(kernel_sha=kernel_sha(), hbm_bytes_per_launch=int(hbm),
               fetch_factor=round(res["fetch"]["factor"], 4), write_factor=round(res["write"]["factor"], 4),
               fetch_kib_per_launch=round(res["fetch"]["kib_per_launch"], 1),
               write_kib_per_launch=round(res["write"]["kib_per_launch"], 1),
               launches=res["fetch"]["launches"],
               commands=[f"rocprofv3 --pmc {c} -d {os.path.dirname(p)} -o run --output-format csv -- "
                         "python -u bench.py --steps 2 --warmup 1 --no-cpu --no-baseline --no-graph "
                         "--no-large --no-configs --copy-calibration"
                         for c, p in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv))]
               + [f"python bench.py --pmc-summary {fetch_csv} {write_csv}"])
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def large_m_sweep(w4, torch, group):
    """TFLOP/s of w4a16_gemm (automatic plan) on the 70B-class shapes at M >= 256, next to
    the hand-written fp16 GEMM on the dequantized weights (w4a16_fp16_gemm, the unfused
    baseline's GEMM) and torch's fp16 matmul on the same weights (context).  Inputs are seeded and
    synthetic with the workload's distributions (codes uniform 0..15, scales U[0.001,
    0.01], X ~ N(0,1)), generated on the device; each shape is timed over back-to-back
    launches after a warmup."""
    shapes = [(8192, 28672), (28672, 8192), (8192, 10240)]
    Ms = [16, 64, 256, 1024, 4096]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2024)
    out = []

    def timed(fn, reps):
        # warm up for ~50 ms: the clock ramps under sustained matrix load
        t0 = time.perf_counter()
        while True:
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > 0.05:
                break
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    # measured ceiling: dense fp16 matrix instructions with no memory traffic, after the
    # same 50 ms warmup (the clock settles lower under sustained matrix load)
    probe_out = torch.zeros(4, dtype=torch.float32, device="cuda")
    pw, pi = 1024, 2000  # about 0.4 ms per launch
    tp = timed(lambda: w4.w4a16_probe_mfma(pw, pi, probe_out), 5)
    mfma_probe = w4.w4a16_probe_mfma_flops(pw, pi) / tp / 1e12

    for (K, N) in shapes:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        s = (torch.rand((K // group, N), device="cuda", generator=gen) * 0.009 + 0.001).half()
        wp, sp, _ = w4.alloc_packed(K, N, group, False)
        w4.w4a16_repack(q, s, None, wp, sp, None, K, N, group)
        Wt = torch.empty((N, K), dtype=torch.float16, device="cuda")
        w4.w4a16_dequant(q, s, None, Wt, K, N, group)
        del q
        # the memory-bound runs (M = 16, 64) rotate over weight copies totalling at least
        # 512 MiB, so that no launch finds its weights in the 256 MiB Infinity Cache
        ncop = max(2, -(-(512 << 20) // (K * N // 2)))
        copies = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(ncop - 1)]
        for M in Ms:
            X = torch.randn((M, K), device="cuda", generator=gen).half()
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            fl = 2.0 * M * N * K
            reps = max(3, min(50, int(2e13 / fl)))
            if M < 256:
                t = time_rotated(torch, [lambda c=c: w4.w4a16_gemm(X, c[0], c[1], None, Y, M, N, K,
                                                                   group) for c in copies])
            else:
                t = timed(lambda: w4.w4a16_gemm(X, wp, sp, None, Y, M, N, K, group), reps)
            tb = timed(lambda: w4.w4a16_fp16_gemm(X, Wt, Y, M, N, K), reps)
            tt = timed(lambda: torch.nn.functional.linear(X, Wt), reps)
            plan = w4.w4a16_gemm_describe(M, N, K, group)
            wbytes = algorithmic(M, K, N, group)[0]
            out.append(dict(M=M, K=K, N=N, us=round(t * 1e6, 2), TFLOPs=round(fl / t / 1e12, 1),
                            weight_GBps=round(wbytes / t / 1e9, 1), **roof(M, K, N, t, group),
                            mfma_frac=round(fl / t / 1e12 / FP16_PEAK_TFLOPS, 4),
                            frac_of_mfma_probe=round(fl / t / 1e12 / mfma_probe, 4),
                            plan=plan["name"],
                            fp16_baseline_TFLOPs=round(fl / tb / 1e12, 1),
                            torch_fp16_TFLOPs=round(fl / tt / 1e12, 1)))
            del X, Y
        del wp, sp, s, Wt, copies
    torch.cuda.synchronize()
    big = [r for r in out if r["M"] >= 1024]
    small = [r for r in out if r["M"] <= 32]
    return dict(peak_TFLOPs=FP16_PEAK_TFLOPS, unit="TFLOP/s",
                mfma_probe_TFLOPs=round(mfma_probe, 1),
                min_mfma_frac_M_ge_1024=min(r["mfma_frac"] for r in big),
                mean_mfma_frac_M_ge_1024=round(sum(r["mfma_frac"] for r in big) / len(big), 4),
                mean_hbm_frac_M_le_32=round(sum(r["roofline_frac"] for r in small) / len(small), 4),
                runs=out)


_SIDE = {}
STEP_STATS = {}  # per-step time percentiles (ms) of each timed step function


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
    """Groups of 64 rows (two scale rows per 128-row block) against groups of 128 on the
    same codes: decode shapes from the 7B-class sweep and one large-M layer, symmetric
    and with zero-points.  Seeded synthetic weights (codes uniform 0..15, scales
    U[0.002, 0.02], zero-points uniform 0..15) generated on the device; weights rotate
    over copies totalling at least 512 MiB."""
    rot = 512 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(64)
    runs = []
    for (K, N, Ms) in [(4096, 11008, (1, 16, 32)), (8192, 10240, (1024,))]:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        packs = {}
        for g in (128, 64):
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
                for g in (128, 64):
                    t[g] = time_rotated(torch, [lambda c=c, g=g: w4.w4a16_gemm(X, c[0], c[1], c[2], Y,
                                                                             M, N, K, g)
                                                for c in packs[(g, asym)]])
                wb64 = K * N // 2 + 4 * (K // 128) * N + ((K // 64) * N // 2 if asym else 0)
                runs.append(dict(M=M, K=K, N=N, zero_points=asym, g128_us=round(t[128] * 1e6, 2),
                                 g64_us=round(t[64] * 1e6, 2),
                                 g64_over_g128_time=round(t[64] / t[128], 3),
                                 g64_weight_GBps=round(wb64 / t[64] / 1e9, 1),
                                 g64_TFLOPs=round(2.0 * M * N * K / t[64] / 1e12, 1)))
            del X, Y
        del q, packs
        torch.cuda.empty_cache()
    return dict(kernel="w4a16_gemm with groups of 64 rows vs 128", runs=runs)


def bf16_leg(w4, torch):
    """bf16 activations (w4a16_gemm_bf16, skinny kernel for every M) against fp16
    activations (w4a16_gemm) on the same repacked weights, at the decode-sweep shapes and
    M = 1 / 16 / 32.  Seeded synthetic inputs on the device; weights rotate over copies
    totalling at least 512 MiB."""
    rot = 512 << 20
    gen = torch.Generator(device="cuda")
    gen.manual_seed(16)
    runs = []
    for (K, N) in [(4096, 4096), (4096, 12288), (11008, 4096)]:
        q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda",
                          generator=gen)
        s = (torch.rand((K // 128, N), device="cuda", generator=gen) * 0.018 + 0.002).half()
        pk = w4.alloc_packed(K, N, 128, False)
        w4.w4a16_repack(q, s, None, *pk, K, N, 128)
        n = max(2, -(-rot // (K * N // 2)))
        copies = [pk] + [tuple(t.clone() if t is not None else None for t in pk) for _ in range(n - 1)]
        for M in (1, 16, 32):
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
    """FP8 E4M3 activations with per-row fp32 scales (w4a8_gemm, skinny kernel for every M)
    against fp16 activations (w4a16_gemm, automatic plan) on the same repacked weights:
    decode shapes at M = 1 / 16 / 32 and a 70B-class layer at M = 16 / 64 / 256.  Seeded
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
    activations) and MXFP4 weights with fp8 activations (block scales inside the matrix
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
    out = {}
    for name, fn in (("w4a16_gemm", lambda: w4.w4a16_gemm(Xh, pk[0], pk[1], None, Y, M, N, K, 128)),
                     ("w4a8_gemm", lambda: w4.w4a8_gemm(X8, a, pk[0], pk[1], None, Y, M, N, K, 128)),
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of HIP graphs")
    ap.add_argument("--no-baseline", action="store_true", help="skip the fp16 baseline")
    ap.add_argument("--variant", type=int, default=-1, help="force a kernel variant (tuning)")
    ap.add_argument("--splits", type=int, default=0, help="force split-K slices (tuning)")
    ap.add_argument("--detail", default=None, help="write per-launch detail JSON here")
    ap.add_argument("--no-large", action="store_true",
                    help="skip the large-M (70B-class, MFMA-bound) sweep")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 2:4-sparse and zero-point workload legs")
    ap.add_argument("--no-table", action="store_true",
                    help="skip the per-shape table (a kernel trace then holds only the step's launches)")
    ap.add_argument("--profile-tiled", action="store_true",
                    help="only a short W4A16 / W4A8 tiled-kernel workload (for counter runs)")
    ap.add_argument("--only-mxfp4", action="store_true",
                    help="only the MXFP4 leg (for a kernel trace of its kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain device copies of known size (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "this script into profiles/ and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only; the W4A16 GEMM has no multi-GPU "
              "path here (it would shard by output columns with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import w4a16_mixed_precision_offline_amd as w4
    from gen import CONFIGS, activations, config_runs, weights

    torch.cuda.set_device(0)
    if args.profile_tiled:
        profile_tiled(w4, torch)
        return
    if args.only_mxfp4:
        print(json.dumps(dict(mxfp4_in_mfma_dequant=mxfp4_leg(w4, torch))), flush=True)
        return
    runs = config_runs(1)
    shapes = []
    for w in runs:
        if (w.K, w.N) not in shapes:
            shapes.append((w.K, w.N))
    Ms = CONFIGS[1]["Ms"]
    group = 128

    # ---- inputs, resident in HBM -----------------------------------------------------
    step_wbytes = sum(algorithmic(1, K, N)[0] for (K, N) in shapes)
    copies_per_step = len(Ms)  # each launch of a shape within a step uses a distinct copy
    steps_per_cycle = max(1, -(-ROTATE_BYTES // (step_wbytes * copies_per_step)))
    R = copies_per_step * steps_per_cycle
    host = {}
    packed = {}
    for (K, N) in shapes:
        w = next(r for r in runs if (r.K, r.N) == (K, N))
        d = weights(w)
        host[(K, N)] = d
        q = torch.from_numpy(d["Qp"]).cuda()
        s = torch.from_numpy(d["s"]).cuda()
        wp, sp, _ = w4.alloc_packed(K, N, group, False)
        w4.w4a16_repack(q, s, None, wp, sp, None, K, N, group)
        packed[(K, N)] = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(R - 1)]
        del q, s
    Xs, Ys, Xh = {}, {}, {}
    for w in runs:
        X = activations(w)
        Xh[(w.M, w.K, w.N)] = X
        Xs[(w.M, w.K, w.N)] = torch.from_numpy(X).cuda()
        Ys[(w.M, w.K, w.N)] = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()

    # launch list of one step: M outer, shape inner; copy index advances per launch
    def step_launches(step_idx):
        out = []
        cyc = step_idx % steps_per_cycle
        for i, M in enumerate(Ms):
            for (K, N) in shapes:
                out.append((M, K, N, cyc * copies_per_step + i))
        return out

    def run_step_w4(step_idx):
        for (M, K, N, c) in step_launches(step_idx):
            wp, sp = packed[(K, N)][c]
            w4.w4a16_gemm_plan(Xs[(M, K, N)], wp, sp, None, Ys[(M, K, N)], M, N, K, group,
                               args.variant, args.splits)

    stream = torch.cuda.Stream()

    def time_steps(run_step, nsteps, warmup, use_graph):
        """Returns (seconds per step, mode)."""
        with torch.cuda.stream(stream):
            for i in range(max(warmup, steps_per_cycle if use_graph else 0)):
                run_step(i)
        torch.cuda.synchronize()
        graphs = None
        if use_graph:
            try:
                graphs = []
                for c in range(steps_per_cycle):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        run_step(c)
                    graphs.append(g)
                torch.cuda.synchronize()
                with torch.cuda.stream(stream):
                    for i in range(warmup):
                        graphs[i % steps_per_cycle].replay()
                torch.cuda.synchronize()
            except Exception as e:  # capture unsupported: fall back to eager launches
                print(f"bench.py: graph capture failed ({e}); timing eager launches",
                      file=sys.stderr)
                graphs = None
        # one event between consecutive steps: the first and last bracket the timed steps,
        # the ones between give the per-step distribution
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            evs[0].record(stream)
            for i in range(nsteps):
                if graphs is not None:
                    graphs[i % steps_per_cycle].replay()
                else:
                    run_step(i)
                evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(nsteps))
        pct = lambda f: per_step[min(nsteps - 1, int(f * (nsteps - 1) + 0.5))]
        STEP_STATS[run_step.__name__] = dict(p10=round(pct(0.1), 5), p50=round(pct(0.5), 5),
                                             p90=round(pct(0.9), 5))
        return evs[0].elapsed_time(evs[-1]) / 1e3 / nsteps, ("hip_graph" if graphs is not None else "eager")

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    t_step, mode = time_steps(run_step_w4, args.steps, args.warmup, not args.no_graph)

    # ---- per-shape durations for the per-run table: for each GEMM of the step, one HIP
    #      graph of back-to-back launches over all R weight copies, replayed; eager launches
    #      from Python would time the host's launch rate, not the GPU, at these sizes -----
    per_launch = []
    launches = step_launches(0)
    for (M, K, N, _) in ([] if args.no_table else launches):
        calls = [(lambda wp=wp, sp=sp, M=M, K=K, N=N: w4.w4a16_gemm_plan(
            Xs[(M, K, N)], wp, sp, None, Ys[(M, K, N)], M, N, K, group, args.variant, args.splits,
            stream=stream.cuda_stream)) for (wp, sp) in packed[(K, N)]]
        with torch.cuda.stream(stream):
            for f in calls[:2]:
                f()
        torch.cuda.synchronize()
        if args.no_graph:
            g = None
        else:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for f in calls:
                    f()
            g.replay()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 3
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(reps):
                if g is not None:
                    g.replay()
                else:
                    for f in calls:
                        f()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * len(calls))
        del g
        wb, ab, fl = algorithmic(M, K, N)
        plan = w4.w4a16_gemm_describe(M, N, K, group)
        per_launch.append(dict(M=M, K=K, N=N, us=round(us, 3), weight_GBps=round(wb / us / 1e3, 1),
                               TFLOPs=round(fl / us / 1e6, 2), hbm_frac=round(ab / us / 1e3 / HBM_PEAK_GBPS, 4),
                               plan=plan["name"], splits=plan["splits"]))

    n_launch = len(launches)
    step_w = sum(algorithmic(M, K, N)[0] for (M, K, N, _) in launches)
    step_alg = sum(algorithmic(M, K, N)[1] for (M, K, N, _) in launches)
    step_fl = sum(algorithmic(M, K, N)[2] for (M, K, N, _) in launches)
    value = step_w / t_step / 1e9
    avg_launch_s = t_step / n_launch
    achieved = step_alg / n_launch / avg_launch_s / 1e9
    traffic = traffic_from_profiles()

    # ---- fp16 baseline: hand-written dequant once, then the hand-written fp16 GEMM ----
    baseline = None
    if not args.no_baseline:
        Wt = {}
        for (K, N) in shapes:
            d = host[(K, N)]
            t0 = torch.empty((N, K), dtype=torch.float16, device="cuda")
            w4.w4a16_dequant(torch.from_numpy(d["Qp"]).cuda(), torch.from_numpy(d["s"]).cuda(),
                             None, t0, K, N, group)
            Wt[(K, N)] = [t0] + [t0.clone() for _ in range(copies_per_step - 1)]
        torch.cuda.synchronize()

        def run_step_fp16(step_idx):
            for i, M in enumerate(Ms):
                for (K, N) in shapes:
                    w4.w4a16_fp16_gemm(Xs[(M, K, N)], Wt[(K, N)][i], Ys[(M, K, N)], M, N, K)

        t16, _ = time_steps(run_step_fp16, max(5, args.steps // 2), 2, not args.no_graph)

        def run_step_torch(step_idx):
            for i, M in enumerate(Ms):
                for (K, N) in shapes:
                    torch.nn.functional.linear(Xs[(M, K, N)], Wt[(K, N)][i])

        ttorch, _ = time_steps(run_step_torch, max(5, args.steps // 2), 2, False)
        baseline = dict(kind="w4a16_dequant + w4a16_fp16_gemm (hand-written, fp16 weights)",
                        ms_per_step=round(t16 * 1e3, 4),
                        fp16_weight_GBps=round(sum(2 * K * N for (_, K, N, _) in launches) / t16 / 1e9, 1),
                        w4_speedup=round(t16 / t_step, 3),
                        speedup_ceiling_bytes=round(16 / (4 + 16 / 128), 3),
                        torch_matmul_ms_per_step=round(ttorch * 1e3, 4),
                        w4_speedup_vs_torch_matmul=round(ttorch / t_step, 3))
        del Wt

    # ---- measured ceiling: a plain streaming read of each launch's packed codes -------
    # (calibration kernel of the library, same launch list, weight rotation and HIP
    # graphs): at 8-25 MiB per launch, launch and ramp keep any kernel far below the
    # 8 TB/s spec, so the GEMM is also set against what a read-only kernel achieves
    plain_read = None
    if not args.no_baseline:
        probe_out = torch.zeros(4, dtype=torch.int32, device="cuda")

        def run_step_read(step_idx):
            cyc = step_idx % steps_per_cycle
            for i, M in enumerate(Ms):
                for (K, N) in shapes:
                    wp, _ = packed[(K, N)][cyc * copies_per_step + i]
                    w4.w4a16_probe_read(wp, K * N // 2, probe_out)

        tread, _ = time_steps(run_step_read, max(5, args.steps // 2), 2, not args.no_graph)
        code_bytes = sum(K * N // 2 for (_, K, N, _) in launches)
        plain_read = dict(kernel="w4a16_probe_read over each launch's packed codes (16-byte "
                                 "non-temporal streaming read, nothing else)",
                          GBps=round(code_bytes / tread / 1e9, 1),
                          us_per_launch=round(tread / n_launch * 1e6, 3),
                          frac_of_peak=round(code_bytes / tread / 1e9 / HBM_PEAK_GBPS, 4),
                          gemm_time_over_read_time=round(t_step / tread, 3))

    # ---- large-M sweep: 70B-class single-GPU shapes, where the matrix cores bound ------
    large = None
    if not args.no_large:
        large = large_m_sweep(w4, torch, group)

    # ---- 2:4 sparse vs dense on the same pruned weights; zero-point workload ---------
    sparse24 = asym = tiny = None
    if not args.no_configs:
        sparse24, asym, tiny = config_legs(w4, torch, group)

    group64 = bf16 = fp8 = mxfp4 = offline = None
    if not args.no_configs:
        group64 = group64_leg(w4, torch)
        bf16 = bf16_leg(w4, torch)
        fp8 = w4a8_leg(w4, torch)
        mxfp4 = mxfp4_leg(w4, torch)
        offline = offline_leg(w4, torch)

    # ---- CPU oracle on this host over one step (bounded sample) -----------------------
    cpu = None
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = len(os.sched_getaffinity(0))
        # repeat whole steps until at least 10 s of oracle work (bounded at 30 s)
        t0 = time.perf_counter()
        passes = 0
        while True:
            for (M, K, N, _) in launches:
                d = host[(K, N)]
                oracle.gemm(Xh[(M, K, N)], d["Qp"], d["s"], None, group)
            passes += 1
            tc = time.perf_counter() - t0
            if tc >= 10.0 or tc * (passes + 1) / passes > 30.0:
                break
        cpu = dict(value=round(passes * step_w / tc / 1e9, 4), unit="GB/s", cores=threads,
                   kind="oracle",
                   sample=f"{passes} full step(s) of the decode sweep (24 GEMMs each): unpack + "
                          "exact fp64 dequant + fp64 matmul, NumPy/OpenBLAS",
                   seconds=round(tc, 3))

    line = {
        "metric": "W4A16 GEMM TFLOP/s + weight HBM GB/s vs M (1..4096), % of roofline",
        "value": round(value, 2),
        "unit": "GB/s",
        "value_is": "packed INT4 weights + fp16 scales of the 24 GEMMs / step time",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 5),
        "ms_per_step_percentiles": STEP_STATS.get("run_step_w4"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "decode-shape sweep, 7B-class linear layers: (K,N) in "
                        "{(4096,4096),(4096,12288),(4096,11008),(11008,4096)} x M in "
                        "{1,2,4,8,16,32}, group 128 along K, symmetric INT4, fp16 X ~ N(0,1), "
                        "scales U[0.002,0.02]; 24 GEMMs per step",
            "launch": mode,
            "weight_copies_rotated": R,
            "parallelism": "single GPU",
        },
        "tflops": round(step_fl / t_step / 1e12, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "w4a16 fused GEMM (skinny_kernel), mean over the 24 launches of a step",
            "algorithmic_bytes_per_launch": int(step_alg / n_launch),
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
            "measured_ceiling": plain_read,
        },
        "cpu_baseline": cpu,
        "fp16_baseline": baseline,
        "large_m_sweep": large,
        "sparse24_vs_dense": sparse24,
        "asym_zero_point": asym,
        "tiny_config": tiny,
        "group64": group64,
        "bf16_activations": bf16,
        "w4a8_fp8_activations": fp8,
        "mxfp4_in_mfma_dequant": mxfp4,
        "load_time_kernels": offline,
        "per_launch_us": [[p["M"], p["K"], p["N"], p["us"]] for p in per_launch],
        "decode_runs": [dict(M=p["M"], K=p["K"], N=p["N"], us=p["us"], weight_GBps=p["weight_GBps"],
                             TFLOPs=p["TFLOPs"], bound="hbm", roofline_frac=p["hbm_frac"],
                             plan=p["plan"]) for p in per_launch],
    }
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(dict(line=line, per_launch=per_launch, kernel_sha=kernel_sha()), f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

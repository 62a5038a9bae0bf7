#!/usr/bin/env python
"""Benchmark of the BaKron hot path on one MI355X.

One step = the whole hot path on one synthetic layer, inputs already in HBM:
one bakron_quantize call, i.e. the factorisations of A and B (damping,
reverse Cholesky, normalised inverse; independent, so they run on two
library streams at once) and the solve (leaf sweeps, error propagation,
objective), which starts on the factors' leading blocks while their last
products run.  The same work as three calls (bakron_factor twice, then
bakron_solve) is timed too, for the factor / solve split, and must give the
same results.
Default workload: the 8192 x 8192 layer (mixed 2/3-bit grids, 2.80 bits per
weight, log-normal channel scales, 8192 samples per factor).

Prints ONE JSON line.  `value` is seconds per step (time-like: lower is
better).  `roofline` describes the kernel with the largest share of the
step, timed with HIP events around each of its launches (the *_profiled
entry points, on the stream the kernels run on) in a separate pass over the
same inputs.  `cpu_baseline` is the float64 oracle (numpy factorisations,
C / OpenMP recursive solve) on the whole layer, timed on the host cores.

Only --gpus 1 is supported: the solve of one matrix runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
PAGES_8192_SECONDS = 1.839        # the pages' BaKron time at 8192 x 8192 (another GPU): context
PAGES_GPTQ_8192_SECONDS = 0.059   # the pages' GPTQ time on the same matrix and GPU: context


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="sq8192_mixed")
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="edge of the leading block the oracle baseline solves (-1 = the whole layer, 0 = skip)")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel roofline pass")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the secondary paths (the one-sided case B = I) measured beside the step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES (counter calibration) and exit")
    ap.add_argument("--pmc-digest", nargs="+", metavar="DIR",
                    help="only summarise rocprofv3 --pmc output directories (per kernel, per dispatch) and exit")
    ap.add_argument("--traffic-digest", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="only turn FETCH_SIZE / WRITE_SIZE runs and their copy calibrations into "
                         "profiles/traffic_<config>.{json,md} and exit")
    ap.add_argument("--stats-digest", metavar="DIR",
                    help="only summarise a rocprofv3 --kernel-trace --stats output directory and exit "
                         "(with --bench-log, the per-kernel times of that bench run's profiled pass beside it)")
    ap.add_argument("--bench-log", default="", help="stderr of the bench run that --stats-digest profiled")
    ap.add_argument("--digest-title", default="", help="title line of the --pmc-digest summary")
    ap.add_argument("--digest-command", default="", help="command line recorded in a digest")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.pmc_digest:
        print(pmc_digest(args.pmc_digest, args.digest_title, args.digest_command))
        return
    if args.traffic_digest:
        traffic_digest(args.traffic_digest, args.config, args.digest_command)
        return
    if args.stats_digest:
        print(stats_digest(args.stats_digest, args.bench_log, args.digest_title, args.digest_command))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: only --gpus 1 is supported; the BaKron solve of one matrix runs on one GPU "
              "(layers are independent, so more GPUs would take more layers, not split one).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import two_sided_hessian_amd as B
    import workloads as WL

    spec = WL.by_name(args.config)
    m, n = spec.m, spec.n
    t0 = time.time()
    d = WL.generate(spec)
    log(f"[bench] generated {spec.name} {m}x{n} in {time.time() - t0:.1f}s")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(dev) for k in ("W", "A", "B", "scale", "zero", "maxq")}
    # the grid contract is checked once here; the calls below reuse the same
    # grid and skip the check (it reads the grid back to the host)
    B.check_grid(T["scale"], T["zero"], T["maxq"])
    fa = (torch.empty((n, n), device=dev), torch.empty((n, n), device=dev), torch.zeros(1, dtype=torch.int32, device=dev))
    fb = (torch.empty((m, m), device=dev), torch.empty((m, m), device=dev), torch.zeros(1, dtype=torch.int32, device=dev))
    ws_fa = B._binding.workspace(B.factor_workspace_bytes(n), dev)
    ws_fb = B._binding.workspace(B.factor_workspace_bytes(m), dev)
    ws_s = B._binding.workspace(B.solve_workspace_bytes(m, n), dev)
    out = {"V": torch.empty((m, n), device=dev), "codes": torch.empty((m, n), dtype=torch.uint8, device=dev),
           "objective": torch.empty(1, dtype=torch.float64, device=dev)}
    stream = torch.cuda.current_stream()
    # The step: bakron_quantize, both factorisations and the solve in one
    # call (the library overlaps the solve's start with the factors' last
    # products).  `separate` below runs the same work as three calls (the two
    # factors on two streams of their own, default priority, then the solve)
    # to report the factor / solve split and the per-kernel profile.
    ws_q = B._binding.workspace(B.quantize_workspace_bytes(m, n), dev)
    qout = {"V": out["V"], "codes": out["codes"], "objective": out["objective"], "L_A": fa[0], "P_A": fa[1],
            "info_A": fa[2], "L_B": fb[0], "P_B": fb[1], "info_B": fb[2]}

    def fused():
        B.quantize(T["W"], T["A"], T["B"], T["scale"], T["zero"], T["maxq"], 0.01, out=qout, ws=ws_q,
                   stream=stream, check=False)

    sA = sB = None
    fork, joinA, joinB = (torch.cuda.Event() for _ in range(3))

    def separate(ev=None, profile=None):
        fork.record(stream)
        sA.wait_event(fork)
        sB.wait_event(fork)
        if profile is None:
            B.factor(T["A"], 0.01, out=fa, ws=ws_fa, stream=sA)
            B.factor(T["B"], 0.01, out=fb, ws=ws_fb, stream=sB)
        else:
            # the profiled entry points drain their stream before returning:
            # one host thread per factor keeps the two running concurrently
            import threading
            pa, pb = [], []
            th = [threading.Thread(target=B.factor, args=(T["A"], 0.01),
                                   kwargs=dict(out=fa, ws=ws_fa, stream=sA, profile=pa)),
                  threading.Thread(target=B.factor, args=(T["B"], 0.01),
                                   kwargs=dict(out=fb, ws=ws_fb, stream=sB, profile=pb))]
            for x in th:
                x.start()
            for x in th:
                x.join()
            profile.extend(pa + pb)
        joinA.record(sA)
        joinB.record(sB)
        stream.wait_event(joinA)
        stream.wait_event(joinB)
        if ev is not None:
            ev.record(stream)
        B.solve(T["W"], fa[0], fa[1], fb[0], fb[1], T["scale"], T["zero"], T["maxq"], out=out, ws=ws_s,
                stream=stream, profile=profile, check=False)

    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    starts[0].record(stream)
    for k in range(args.steps):
        fused()
        starts[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    step_ms = [starts[k].elapsed_time(starts[k + 1]) for k in range(args.steps)]
    ms_per_step = float(np.mean(step_ms))
    info = (int(fa[2].item()), int(fb[2].item()))
    obj = float(out["objective"].item())
    codes_fused = out["codes"].clone()

    # the same work as three calls, timed apart (after the fused timing, so
    # that its streams do not change how the fused call's streams map to
    # hardware queues)
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(args.warmup):
        separate()
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    starts[0].record(stream)
    for k in range(args.steps):
        separate(mids[k])
        starts[k + 1].record(stream)
    torch.cuda.synchronize()
    sep_ms = [starts[k].elapsed_time(starts[k + 1]) for k in range(args.steps)]
    factor_ms = [starts[k].elapsed_time(mids[k]) for k in range(args.steps)]
    solve_ms = [mids[k].elapsed_time(starts[k + 1]) for k in range(args.steps)]
    same = bool(torch.equal(codes_fused, out["codes"])) and float(out["objective"].item()) == obj
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step fused; as three calls {np.mean(sep_ms):.3f} ms "
        f"(factor {np.mean(factor_ms):.3f} ms, solve {np.mean(solve_ms):.3f} ms), wall {wall:.3f}s, info {info}, "
        f"objective {obj:.6e}, same results {same}")
    if info != (0, 0):
        raise SystemExit(f"factor reported a non-positive pivot: {info}")
    if not same:
        raise SystemExit("the fused call and the three calls disagree")

    alg_solve = float(m) * n * (m + n)
    alg_factor = 2.0 * (float(m) ** 3 + float(n) ** 3) / 3.0
    solve_s = float(np.median(solve_ms)) / 1e3

    roofline = roofline_mfma = None
    kernels = stages = None
    if not args.no_profile:
        prof = []
        separate(profile=prof)
        torch.cuda.synchronize()
        agg = {}
        for r in prof:
            a = agg.setdefault(r["name"], {"launches": 0, "total_ms": 0.0, "alg_flops": 0.0, "alg_bytes": 0.0})
            for k in ("launches", "total_ms", "alg_flops", "alg_bytes"):
                a[k] += r[k]
        kernels = {k: {"launches": v["launches"], "total_ms": round(v["total_ms"], 4),
                       "avg_us": round(1e3 * v["total_ms"] / v["launches"], 3),
                       "alg_tflops": round(v["alg_flops"] / (v["total_ms"] * 1e-3) / 1e12, 3) if v["total_ms"] > 0 else None,
                       "alg_gbs": round(v["alg_bytes"] / (v["total_ms"] * 1e-3) / 1e9, 1) if v["total_ms"] > 0 else None}
                   for k, v in sorted(agg.items(), key=lambda kv: -kv[1]["total_ms"])}
        traffic = load_traffic(spec.name)
        # The far parts of the solve run beside the caller's stream on a
        # capped grid (their launches are the *_far kernels): their summed
        # durations overlap the rest of the step, so the dominant kernel is
        # chosen among the kernels of the step's own stream order.
        main = [kv for kv in agg.items() if not kv[0].endswith("_far")]
        dom = max(main, key=lambda kv: kv[1]["total_ms"])
        roofline = roofline_entry(*dom, traffic)
        mf = [kv for kv in main if kernel_bound(kv[0]) == "mfma"]
        if mf:
            # the MFMA kernel with the most block products; its flops are the
            # executed block products (recomputation of the divide and
            # conquer included), so its fraction is an executed-work one
            roofline_mfma = roofline_entry(*max(mf, key=lambda kv: kv[1]["alg_flops"]), traffic)
            roofline_mfma["work"] = "executed block products"
        stages = stage_fractions(agg, m, n)
        log(f"[bench] kernels: {json.dumps(kernels)}")
        log(f"[bench] propagation stages: {json.dumps(stages)}")

    nxt = None
    if not args.no_next:
        traffic = None if args.no_profile else load_traffic(spec.name)
        nxt = {"gptq": bench_gptq(B, T, fa, m, n, args, traffic)}
        nxt.update(bench_factors(B, WL, spec, dev, args, traffic))
        nxt["batch"] = bench_batch(B, WL, dev, args)
        nxt["grouped"] = bench_grouped(B, WL, spec, T, fa, fb, dev, args)
        nxt["antidiagonal"] = bench_antidiagonal(B, WL, T, fa, fb, m, n, dev, args)

    cpu = None
    if args.cpu_sample != 0:
        cpu = cpu_baseline(d, max(m, n) if args.cpu_sample < 0 else args.cpu_sample, m, n)
        cpu["small_forms"] = cpu_small_forms(WL)

    res = {
        "metric": "seconds per m×n BaKron solve (8192×8192 fp32) + achieved fp32 MFMA TFLOP/s",
        "value": round(ms_per_step / 1e3, 6),
        "unit": "s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": round((ms_per_step / 1e3) / PAGES_8192_SECONDS, 6) if (m, n) == (8192, 8192) else None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "m": m, "n": n, "samples": spec.samples,
                   "bits": "mixed 2/3 (2.80 bpw)" if spec.mixed_low_rows else spec.bits,
                   "damping": 0.01,
                   "step": "bakron_quantize: factor(A) || factor(B) on library streams, solve overlapping their end"},
        "separate_s": round(float(np.mean(sep_ms)) / 1e3, 6),
        "solve_s": round(solve_s, 6),
        "factor_s": round(float(np.median(factor_ms)) / 1e3, 6),
        "solve_alg_tflops": round(alg_solve / solve_s / 1e12, 3),
        "solve_alg_frac": round(alg_solve / solve_s / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
        "factor_alg_tflops": round(alg_factor / (float(np.median(factor_ms)) / 1e3) / 1e12, 3),
        "objective": obj,
        "roofline": roofline,
        "roofline_mfma": roofline_mfma,
        "stages": stages,
        "kernels": kernels,
        "next": nxt,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_gptq(B, T, fa, m, n, args, traffic):
    """The one-sided case B = I (bakron_gptq) on the same layer and the same
    factor of A, inputs resident: mean time over args.steps calls after
    args.warmup, its algorithmic rate (m n^2 flops: the triangular product
    E P_A^T), and the roofline object of its dominant kernel."""
    import torch
    dev = T["W"].device
    ws = B._binding.workspace(B.gptq_workspace_bytes(m, n), dev)
    out = {"V": torch.empty((m, n), device=dev), "codes": torch.empty((m, n), dtype=torch.uint8, device=dev),
           "objective": torch.empty(1, dtype=torch.float64, device=dev)}
    stream = torch.cuda.current_stream()

    def call(profile=None):
        B.gptq(T["W"], fa[0], fa[1], T["scale"], T["zero"], T["maxq"], out=out, ws=ws, stream=stream,
               profile=profile, check=False)

    for _ in range(args.warmup):
        call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(args.steps):
        call()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    alg = float(m) * n * n
    res = {"entry": "bakron_gptq", "ms": round(ms, 4), "alg_tflops": round(alg / (ms * 1e-3) / 1e12, 3),
           "vs_pages": round(ms * 1e-3 / PAGES_GPTQ_8192_SECONDS, 5) if (m, n) == (8192, 8192) else None,
           "objective": float(out["objective"].item()), "roofline": None, "kernels": None}
    log(f"[bench] one-sided (B = I): {ms:.3f} ms per call")
    if not args.no_profile:
        prof = []
        call(profile=prof)
        agg = {r["name"]: r for r in prof}
        res["kernels"] = {k: {"launches": v["launches"], "total_ms": round(v["total_ms"], 4),
                              "avg_us": round(1e3 * v["total_ms"] / v["launches"], 3)} for k, v in agg.items()}
        dom = max(agg.items(), key=lambda kv: kv[1]["total_ms"])
        res["roofline"] = roofline_entry(*dom, traffic)
    return res


def bench_factors(B, WL, spec, dev, args, traffic):
    """Kronecker-factor construction from the layer's per-sample inputs
    (X: N x n activations, G: N x m output gradients, sample-major, resident):
    K-FAC A = E[a a^T], B = E[b b^T], and one-step Shampoo A = E[|b|^2 a a^T],
    B = E[|a|^2 b b^T].  Mean time over args.steps after args.warmup; the
    algorithmic rate counts the lower triangles, N n (n + 1) flops per factor
    (plus the weights and the norms for Shampoo)."""
    import torch
    S = WL.samples(spec)
    X = torch.from_numpy(S["X"]).to(dev)
    G = torch.from_numpy(S["G"]).to(dev)
    del S
    N, n = X.shape
    m = G.shape[1]
    A = torch.zeros((n, n), device=dev)
    Bm = torch.zeros((m, m), device=dev)
    wa = torch.empty(N, device=dev)
    wb = torch.empty(N, device=dev)
    stream = torch.cuda.current_stream()

    def kfac(profile=None):
        B.moment(X, out=A, stream=stream, profile=profile)
        B.moment(G, out=Bm, stream=stream, profile=profile)

    def shampoo(profile=None):
        B.row_sqnorms(X, out=wa, stream=stream)
        B.row_sqnorms(G, out=wb, stream=stream)
        B.moment(X, wb, out=A, stream=stream, profile=profile)
        B.moment(G, wa, out=Bm, stream=stream, profile=profile)

    fl = float(N) * (n * (n + 1.0) + m * (m + 1.0))
    res = {}
    for name, fn, extra in (("kfac", kfac, 0.0), ("shampoo", shampoo, 4.0 * N * (n + m))):
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        r = {"entry": "bakron_moment" + (" + bakron_row_sqnorms" if extra else ""), "N": N, "n": n, "m": m,
             "ms": round(ms, 4), "alg_tflops": round((fl + extra) / (ms * 1e-3) / 1e12, 3), "roofline": None}
        log(f"[bench] {name} factors: {ms:.3f} ms")
        if not args.no_profile:
            prof = []
            fn(profile=prof)
            agg = {}
            for x in prof:
                a = agg.setdefault(x["name"], {"launches": 0, "total_ms": 0.0, "alg_flops": 0.0, "alg_bytes": 0.0})
                for k in ("launches", "total_ms", "alg_flops", "alg_bytes"):
                    a[k] += x[k]
            r["roofline"] = roofline_entry(*max(agg.items(), key=lambda kv: kv[1]["total_ms"]), traffic)
        res[name] = r
    return res


def bench_batch(B, WL, dev, args, layers=16, name="sq1024"):
    """Batched solves of independent layers (bakron_solve_batch): `layers`
    layers of the 1024 x 1024 recipe (seeds 0 ..), factors from
    bakron_factor, inputs resident; the batch on one stream against the
    batch spread over four streams (the hardware queues of a process).
    Reports layers per second and algorithmic TFLOP/s (mn(m+n) per layer)."""
    import torch
    spec = WL.by_name(name)
    probs = []
    for k in range(layers):
        d = WL.generate(spec, seed=k)
        T = {key: torch.from_numpy(np.ascontiguousarray(d[key])).to(dev) for key in ("W", "A", "B", "scale", "zero", "maxq")}
        LA, PA, _ = B.factor(T["A"], 0.01)
        LB, PB, _ = B.factor(T["B"], 0.01)
        B.check_grid(T["scale"], T["zero"], T["maxq"])
        probs.append({"W": T["W"], "LA": LA, "PA": PA, "LB": LB, "PB": PB, "scale": T["scale"],
                      "zero": T["zero"], "maxq": T["maxq"]})
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    res = {"entry": "bakron_solve_batch", "layers": layers, "shape": [spec.m, spec.n]}
    alg = layers * float(spec.m) * spec.n * (spec.m + spec.n)
    for ns in (1, 4):
        streams = [main] if ns == 1 else [torch.cuda.Stream() for _ in range(ns)]

        def run():
            for s in streams:
                if s is not main:
                    s.wait_stream(main)
            B.solve_batch(probs, streams, check=False)
            for s in streams:
                if s is not main:
                    main.wait_stream(s)

        for _ in range(args.warmup):
            run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(main)
        for _ in range(args.steps):
            run()
        ev[1].record(main)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        res[f"streams{ns}"] = {"ms": round(ms, 4), "layers_per_s": round(layers / (ms * 1e-3), 1),
                               "alg_tflops": round(alg / (ms * 1e-3) / 1e12, 3)}
        log(f"[bench] batch of {layers} {spec.m}x{spec.n} layers on {ns} stream(s): {ms:.3f} ms")
    return res


def bench_grouped(B, WL, spec, T, fa, fb, dev, args, group=128):
    """Per-group grids (groups of `group` input columns, grids from the
    original W's group slices) on the same layer and the step's factors: the
    two-sided solve (bakron_solve_grouped) and the one-sided call
    (bakron_gptq_grouped), mean time over args.steps calls after args.warmup."""
    import torch
    m, n = spec.m, spec.n
    d = WL.generate(spec, group_size=group)
    g = [torch.from_numpy(np.ascontiguousarray(d[k])).to(dev) for k in ("scale", "zero", "maxq")]
    B.check_grid(*g)
    ws = B._binding.workspace(B.solve_workspace_bytes(m, n), dev)
    out = {"V": torch.empty((m, n), device=dev), "codes": torch.empty((m, n), dtype=torch.uint8, device=dev),
           "objective": torch.empty(1, dtype=torch.float64, device=dev)}
    stream = torch.cuda.current_stream()
    res = {"group_size": group, "grid": f"{m}x{g[0].shape[1]}"}
    for name, fn in (("solve_grouped", lambda: B.solve(T["W"], fa[0], fa[1], fb[0], fb[1], *g, out=out, ws=ws,
                                                       stream=stream, check=False, group_size=group)),
                     ("gptq_grouped", lambda: B.gptq(T["W"], fa[0], fa[1], *g, out=out, ws=ws, stream=stream,
                                                     check=False, group_size=group))):
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        res[name] = {"ms": round(ms, 4), "objective": float(out["objective"].item())}
        log(f"[bench] {name} (groups of {group}): {ms:.3f} ms")
    return res


def bench_antidiagonal(B, WL, T, fa, fb, m, n, dev, args, limit_s=60.0):
    """BaKron-antidiagonal (bakron_solve_antidiagonal: m + n - 1 dependent
    steps, each a rank-|D| update of the bottom-right remainder) against the
    solve: one call on the 4096 x 4096 Student-t layer (its own GPU factors)
    and one on this layer (the step's factors) when the 4096^2 time predicts
    it within `limit_s` (the work grows as m^2 n^2).  Algorithmic work
    m (m + 1) n (n + 1) / 2 flops: every entry pushes its error into its
    whole bottom-right block."""
    import torch
    stream = torch.cuda.current_stream()

    def one(W, LA, PA, LB, PB, s, z, q, mm, nn):
        ws = B._binding.workspace(B.lib().bakron_solve_antidiagonal_workspace_bytes(mm, nn), dev)
        out = {"V": torch.empty((mm, nn), device=dev), "codes": torch.empty((mm, nn), dtype=torch.uint8, device=dev),
               "objective": torch.empty(1, dtype=torch.float64, device=dev)}
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        B.solve_antidiagonal(W, LA, PA, LB, PB, s, z, q, out=out, ws=ws, stream=stream, check=False)
        ev[1].record(stream)
        torch.cuda.synchronize()
        sec = ev[0].elapsed_time(ev[1]) / 1e3
        alg = float(mm) * (mm + 1) * nn * (nn + 1) / 2.0
        return {"s": round(sec, 4), "alg_tflops": round(alg / sec / 1e12, 3),
                "alg_frac": round(alg / sec / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
                "objective": float(out["objective"].item())}

    res = {"entry": "bakron_solve_antidiagonal"}
    spec = WL.by_name("sq4096_t5")
    d = WL.generate(spec)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(dev) for k in ("W", "A", "B", "scale", "zero", "maxq")}
    LA, PA, _ = B.factor(t["A"], 0.01)
    LB, PB, _ = B.factor(t["B"], 0.01)
    ws_s = B._binding.workspace(B.solve_workspace_bytes(spec.m, spec.n), dev)
    B.solve(t["W"], LA, PA, LB, PB, t["scale"], t["zero"], t["maxq"], ws=ws_s, check=False)   # warm
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(args.steps):
        B.solve(t["W"], LA, PA, LB, PB, t["scale"], t["zero"], t["maxq"], ws=ws_s, check=False)
    ev[1].record(stream)
    torch.cuda.synchronize()
    solve_s = ev[0].elapsed_time(ev[1]) / args.steps / 1e3
    r = one(t["W"], LA, PA, LB, PB, t["scale"], t["zero"], t["maxq"], spec.m, spec.n)
    r["solve_s"] = round(solve_s, 6)
    r["vs_solve"] = round(r["s"] / solve_s, 1)
    res[spec.name] = r
    log(f"[bench] antidiagonal {spec.name}: {r['s']:.3f} s ({r['alg_tflops']} TFLOP/s algorithmic), "
        f"solve {solve_s * 1e3:.3f} ms, ratio {r['vs_solve']}")
    del t, LA, PA, LB, PB, ws_s
    predicted = r["s"] * (float(m) * m * n * n) / (float(spec.m) ** 2 * spec.n ** 2)
    if predicted <= limit_s:
        r = one(T["W"], fa[0], fa[1], fb[0], fb[1], T["scale"], T["zero"], T["maxq"], m, n)
        res[f"{m}x{n}"] = r
        log(f"[bench] antidiagonal {m}x{n}: {r['s']:.3f} s ({r['alg_tflops']} TFLOP/s algorithmic)")
    else:
        res[f"{m}x{n}"] = {"skipped": f"predicted {predicted:.0f} s > {limit_s:.0f} s"}
    return res


# Which roofline bounds each kernel: the dense contractions run on the fp32
# MFMA units; the copy, damping and finishing passes stream HBM; the rest
# (the leaf sweep, the diagonal-block factor, the schedule and the objective
# reduction) are chains of dependent vector arithmetic and LDS traffic,
# priced against the fp32 vector peak.
MFMA_KERNELS = {"k_prop_rows", "k_prop_rows_t", "k_prop_cols", "k_prop_cols_t", "k_prop_rows_far",
                "k_prop_rows_t_far",
                "k_prop_cols_far", "k_prop_cols_t_far", "k_f_panel", "k_f_right",
                "k_f_left", "k_f_tile<0>", "k_f_tile<1>", "k_f_tile<2>", "k_f_tile<3>", "k_f_tile<4>", "k_f_update",
                "k_gptq_update",
                "k_gptq_update_t", "k_moment<false>", "k_moment<true>", "k_ad_update"}
HBM_KERNELS = {"k_copy_pad", "k_load_damped", "k_f_finish", "k_diag_mean", "k_clear_info", "k_gptq_load",
               "k_row_sqnorms", "k_ad_prep", "k_ad_quant"}
# fp32 vector peak of the instructions the library's kernels issue: 256 CUs x 4 SIMDs
# x 16 lanes x 2 flops (FMA) x 2.4 GHz = 78.6 TFLOP/s.  MI355X's published
# 157.3 TFLOP/s fp32 vector figure counts packed fp32 (two FMAs per lane per
# instruction), which the library is compiled without.
PEAK_FP32_VECTOR_TFLOPS = 78.6
PEAK_FP32_VECTOR_PACKED_TFLOPS = 157.3

# Kernels of the two propagation stages of the solve.  (The propagation of a
# node of two leaves runs inside the second leaf, k_leaf: its few microseconds
# of block products are counted neither here nor in a stage's time.)
STAGE1_KERNELS = ("k_prop_rows", "k_prop_rows_t", "k_prop_rows_far", "k_prop_rows_t_far")
STAGE2_KERNELS = ("k_prop_cols", "k_prop_cols_t", "k_prop_cols_far", "k_prop_cols_t_far")


def kernel_bound(name):
    return "mfma" if name in MFMA_KERNELS else ("hbm" if name in HBM_KERNELS else "alu")


def sources_digest():
    """sha256 over the library's device and host code (csrc/, comments and
    blank space left out): the HBM counters in profiles/ are valid only for
    the code they were taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "two_sided_hessian_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        path = os.path.join(csrc, f)
        if path.endswith((".hip", ".hpp")):
            with open(path, encoding="utf-8") as fh:
                code = fh.read()
            code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
            code = re.sub(r"//[^\n]*", " ", code)
            code = " ".join(code.split())
            h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()


def load_traffic(workload):
    """Per-launch HBM bytes (FETCH_SIZE + WRITE_SIZE, calibrated against a
    plain copy) from profiles/traffic_<workload>.json, or None when missing or
    taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("sources_sha256") != sources_digest():
        log("[bench] profiles traffic counters were taken on other kernel sources: traffic = null")
        return None
    return t


def roofline_entry(name, v, traffic):
    bound = kernel_bound(name)
    secs = v["total_ms"] * 1e-3
    if bound == "hbm":
        ach, peak, unit = v["alg_bytes"] / secs / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        ach = v["alg_flops"] / secs / 1e12
        peak = PEAK_FP32_MFMA_TFLOPS if bound == "mfma" else PEAK_FP32_VECTOR_TFLOPS
        unit = "TFLOP/s"
    tr = None
    if traffic and name in traffic.get("kernels", {}):
        tr = traffic["kernels"][name]["hbm_bytes_per_launch"]
    r = {"kernel": name, "bound": bound, "achieved": round(ach, 3), "peak": peak, "unit": unit,
         "frac": round(ach / peak, 4), "traffic": tr, "launches": v["launches"],
         "avg_launch_us": round(1e6 * secs / v["launches"], 3),
         "alg_flops_per_launch": v["alg_flops"] / v["launches"],
         "alg_bytes_per_launch": v["alg_bytes"] / v["launches"]}
    if bound == "alu":
        r["peak_note"] = ("non-packed fp32 FMA (the build disables packed fp32); against the packed "
                          f"{PEAK_FP32_VECTOR_PACKED_TFLOPS} TFLOP/s the fraction is "
                          f"{round(ach / PEAK_FP32_VECTOR_PACKED_TFLOPS, 4)}")
    return r


def stage_fractions(agg, m, n):
    """Algorithmic rate of each propagation stage: its share of the solve's
    algorithmic work (stage 1 the triangular product E P_A^T, m n (n + 1)
    flops; stage 2 P_B Y, m (m + 1) n flops; the leaf's in-tile parts of both
    included, since the total is the whole product) over the summed duration
    of the stage's kernels, and the executed block products of those kernels
    for comparison (the divide and conquer recomputes partial products)."""
    out = {}
    for stage, names, alg in (("stage1", STAGE1_KERNELS, float(m) * n * (n + 1)),
                              ("stage2", STAGE2_KERNELS, float(m) * (m + 1) * n)):
        ms = sum(agg[k]["total_ms"] for k in names if k in agg)
        ex = sum(agg[k]["alg_flops"] for k in names if k in agg)
        if ms <= 0:
            continue
        out[stage] = {"kernels_ms": round(ms, 4), "alg_flops": alg,
                      "alg_tflops": round(alg / (ms * 1e-3) / 1e12, 3),
                      "alg_frac": round(alg / (ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
                      "executed_flops": ex,
                      "executed_tflops": round(ex / (ms * 1e-3) / 1e12, 3)}
    return out


def copy_calibration(nbytes):
    """A plain device-to-device copy of nbytes, five times: the reference
    dispatch for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "copies": 5}), flush=True)


def _kernel_key(name):
    """Short kernel name from a profiler's demangled one: the function name
    with its template arguments, without return type, namespaces or
    parameters (e.g. 'k_f_tile<1>')."""
    n = name.strip().replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    n = n[:cut]
    depth, start = 0, 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == ":" and depth == 0 and i + 1 < len(n) and n[i + 1] == ":":
            start = i + 2
    return n[start:].replace(" ", "")


def _read_counters(directory):
    """{kernel: {counter: [value per dispatch]}} from the counter-collection
    CSV files rocprofv3 wrote under `directory`."""
    import csv
    import glob
    out = {}
    files = glob.glob(os.path.join(directory, "**", "*counter_collection*.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection csv under {directory}")
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                k = _kernel_key(row["Kernel_Name"])
                c = row["Counter_Name"]
                out.setdefault(k, {}).setdefault(c, []).append(float(row["Counter_Value"]))
    return out


PMC_DERIVED = (
    # name, formula over per-dispatch means, meaning
    ("valu/wave", lambda c: c["SQ_INSTS_VALU"] / c["SQ_WAVES"], "VALU instructions issued per wave"),
    ("lds/wave", lambda c: c["SQ_INSTS_LDS"] / c["SQ_WAVES"], "LDS instructions issued per wave"),
    ("conflict/lds", lambda c: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"],
     "LDS bank-conflict cycles per LDS instruction"),
    ("ldswait/wavecyc", lambda c: c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"],
     "share of wave cycles spent waiting to issue an LDS instruction"),
    ("valuactive/wavecyc", lambda c: c["SQ_ACTIVE_INST_VALU"] / c["SQ_WAVE_CYCLES"],
     "share of wave cycles issuing VALU instructions"),
    ("mfma_gflop", lambda c: 512.0 * c["SQ_INSTS_VALU_MFMA_MOPS_F32"] / 1e9,
     "fp32 MFMA work executed (MOPS x 512 flops), GFLOP per dispatch"),
    ("mfma_busy", lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8.0 * 1024.0),
     "MFMA busy share of a SIMD: busy cycles (summed over the 1024 SIMDs) over the dispatch's GPU-active "
     "cycles (GRBM_GUI_ACTIVE, summed over the 8 XCDs)"),
    ("l2_hit", lambda c: c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"]), "L2 hit rate"),
)


def pmc_digest(dirs, title, command):
    """Markdown summary of rocprofv3 --pmc runs: per kernel, the number of
    dispatches and the mean of each counter per dispatch, then the derived
    ratios whose counters were collected."""
    per = {}
    for d in dirs:
        for k, cs in _read_counters(d).items():
            dst = per.setdefault(k, {})
            for c, vals in cs.items():
                dst.setdefault(c, []).extend(vals)
    counters = sorted({c for cs in per.values() for c in cs})
    lines = [f"# {title}" if title else "# rocprofv3 counters", ""]
    if command:
        lines += ["Commands (from the repository root, on a machine with the GPU):", "", "```", command, "```", ""]
    lines += ["Mean per dispatch of each counter (a counter is summed over the whole GPU for a dispatch).", ""]
    lines.append("| kernel | dispatches | " + " | ".join(counters) + " |")
    lines.append("|---|---|" + "---|" * len(counters))
    order = sorted(per.items(), key=lambda kv: -max(len(v) for v in kv[1].values()))
    for k, cs in order:
        nd = max(len(v) for v in cs.values())
        lines.append(f"| {k} | {nd} | " + " | ".join(
            (f"{np.mean(cs[c]):.4g}" if c in cs else "") for c in counters) + " |")
    lines += ["", "Derived (only where the counters were collected):", ""]
    lines.append("| kernel | " + " | ".join(d[0] for d in PMC_DERIVED) + " |")
    lines.append("|---|" + "---|" * len(PMC_DERIVED))
    for k, cs in order:
        means = {c: float(np.mean(v)) for c, v in cs.items()}
        vals = []
        for _, f, _ in PMC_DERIVED:
            try:
                vals.append(f"{f(means):.4g}")
            except (KeyError, ZeroDivisionError):
                vals.append("")
        if any(vals):
            lines.append(f"| {k} | " + " | ".join(vals) + " |")
    lines += [""] + [f"- {n}: {m}" for n, _, m in PMC_DERIVED]
    return "\n".join(lines)


def stats_digest(directory, bench_log, title, command):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: calls,
    total and mean duration per kernel (short names), next to the mean
    launch time the bench's own profiled pass measured with HIP events (from
    its stderr), and the bench's step line."""
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats csv under {directory}")
    rows = {}
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                k = _kernel_key(r["Name"])
                a = rows.setdefault(k, [0, 0.0])
                a[0] += int(r["Calls"])
                a[1] += float(r["TotalDurationNs"])
    bench_us, step = {}, ""
    if bench_log:
        with open(bench_log) as fh:
            for line in fh:
                if line.startswith("[bench] kernels: "):
                    for k, v in json.loads(line[len("[bench] kernels: "):]).items():
                        bench_us[k] = v["avg_us"]
                elif "ms/step" in line:
                    step = line.strip()
    lines = [f"# {title}" if title else "# Kernel time", ""]
    if command:
        lines += ["Command (from the repository root, on a machine with the GPU):", "", "```", command, "```", ""]
    if step:
        lines += ["Bench line of the same run: `" + step + "`", ""]
    lines += ["| kernel | calls | total ms | avg us (rocprof) | avg us (bench, HIP events) |", "|---|---|---|---|---|"]
    for k, (calls, ns) in sorted(rows.items(), key=lambda kv: -kv[1][1]):
        b = bench_us.get(k, "")
        lines.append(f"| {k} | {calls} | {ns / 1e6:.3f} | {ns / 1e3 / calls:.2f} | {b} |")
    lines += leaf_width_table(directory)
    return "\n".join(lines)


def leaf_width_table(directory):
    """Leaf launches of a kernel trace grouped by their workgroups (tiles on
    the anti-diagonal): a leaf's in-tile sweep is the same at every width, so
    a difference between the groups is what the rest of the GPU does to it.
    Each group is split by whether, at the launch's midpoint, the workgroups
    of the other running kernels (at most 256 counted per kernel) plus the
    leaf's own exceed the 256 CUs, i.e. whether some of its tiles had to
    share a CU."""
    import bisect
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    leaves, edges = [], []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
                t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
                if _kernel_key(r["Kernel_Name"]) == "k_leaf":
                    leaves.append((t0, t1, wg))
                else:
                    edges += [(t0, min(wg, 256)), (t1, -min(wg, 256))]
    if not leaves:
        return []
    edges.sort()
    times = [t for t, _ in edges]
    running, acc = [], 0
    for _, d in edges:
        acc += d
        running.append(acc)
    groups = {}
    for t0, t1, wg in leaves:
        i = bisect.bisect_right(times, (t0 + t1) // 2) - 1
        others = running[i] if i >= 0 else 0
        hi = 1 << max(0, (wg - 1).bit_length())   # groups (hi/2, hi]
        g = groups.setdefault(hi, [0, 0, 0, 0])
        k = 2 if others + wg > 256 else 0
        g[k] += 1
        g[k + 1] += t1 - t0
    out = ["", "`k_leaf` launches by tiles per launch (from the kernel trace), and split by whether the other "
           "kernels' workgroups running at the launch's midpoint left a CU for each of its tiles:", "",
           "| tiles | calls | avg us | calls with a CU per tile | avg us | calls short of CUs | avg us |",
           "|---|---|---|---|---|---|---|"]

    def avg(ns, c):
        return f"{ns / 1e3 / c:.2f}" if c else ""

    for hi in sorted(groups):
        c0, n0, c1, n1 = groups[hi]
        lo = hi // 2 + 1
        label = f"{hi}" if lo >= hi else f"{lo}-{hi}"
        out.append(f"| {label} | {c0 + c1} | {avg(n0 + n1, c0 + c1)} | {c0} | {avg(n0, c0)} | {c1} | {avg(n1, c1)} |")
    return out


def traffic_digest(dirs, workload, command):
    """HBM bytes per dispatch from FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the counter reads for a plain 1 GiB device
    copy (bench.py --copy-calibration); written with the kernel sources'
    digest to profiles/traffic_<workload>.json and .md."""
    fetch, write, cal_f, cal_w = (_read_counters(d) for d in dirs)

    def copy_kib(cal, counter):
        vals = [v for k, cs in cal.items() for c, vs in cs.items() if c == counter for v in vs]
        return float(np.median(vals))

    copy_kib_total = 1 << 20   # the calibration copies 1 GiB
    fac_f = copy_kib_total / copy_kib(cal_f, "FETCH_SIZE")
    fac_w = copy_kib_total / copy_kib(cal_w, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        fv = fetch.get(k, {}).get("FETCH_SIZE", [])
        wv = write.get(k, {}).get("WRITE_SIZE", [])
        f = float(np.mean(fv)) if fv else 0.0
        w = float(np.mean(wv)) if wv else 0.0
        kernels[k] = {"dispatches": max(len(fv), len(wv)), "fetch_kib_per_dispatch": round(f, 1),
                      "write_kib_per_dispatch": round(w, 1),
                      "hbm_bytes_per_launch": int(round(1024.0 * (f * fac_f + w * fac_w)))}
    out = {"workload": workload, "sources_sha256": sources_digest(), "commands": command,
           "calibration": {"copy_bytes": 1 << 30, "FETCH_SIZE": {"factor": fac_f}, "WRITE_SIZE": {"factor": fac_w}},
           "kernels": kernels}
    base = os.path.join(ROOT, "profiles", f"traffic_{workload}")
    with open(base + ".json", "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    lines = [f"# HBM traffic per dispatch, {workload}", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the dispatches of the run), each in a run of "
             "its own, scaled by what the same counter reads for a plain 1 GiB device copy.", "",
             "```", command, "```", "",
             f"Copy calibration factors: FETCH_SIZE {fac_f:.4f}, WRITE_SIZE {fac_w:.4f}.", "",
             f"Kernel sources sha256 (bench.py uses these numbers only while it matches): `{out['sources_sha256']}`",
             "", "| kernel | dispatches | FETCH KiB | WRITE KiB | HBM bytes per launch (calibrated) |",
             "|---|---|---|---|---|"]
    for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["hbm_bytes_per_launch"] * kv[1]["dispatches"]):
        lines.append(f"| {k} | {v['dispatches']} | {v['fetch_kib_per_dispatch']} | {v['write_kib_per_dispatch']} | "
                     f"{v['hbm_bytes_per_launch']:,} |")
    with open(base + ".md", "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(base + ".json")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, sample, m, n):
    """The float64 oracle, timed on the host cores: both factorisations
    (damping, reverse Cholesky, normalised inverse; numpy / LAPACK) and the
    recursive solve (C, OpenMP) of the leading sample x sample block of the
    same layer (same grid rows, the leading blocks of A and B) -- by default
    the whole layer, so nothing is extrapolated.  A smaller block is scaled
    to the full layer by the work ratio mn(m+n) / (ms ns (ms+ns))."""
    from oracle import recursive as O2
    from oracle import reference as R
    ms, ns = min(m, sample), min(n, sample)
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    threads = int(os.environ["OMP_NUM_THREADS"])
    W = d["W"][:ms, :ns]
    log(f"[bench] cpu oracle on {ms}x{ns} with {threads} threads ...")
    t0 = time.perf_counter()
    fa, fb = R.factor(d["A"][:ns, :ns]), R.factor(d["B"][:ms, :ms])
    tf = time.perf_counter() - t0
    log(f"[bench] cpu oracle factors: {tf:.2f}s")
    O2.bakron_recursive(W, fa["P"], fb["P"], d["scale"][:ms], d["zero"][:ms], d["maxq"][:ms])
    t = time.perf_counter() - t0
    scale = (float(m) * n * (m + n)) / (float(ms) * ns * (ms + ns))
    model = cpu_model()
    log(f"[bench] cpu oracle on {ms}x{ns}: {t:.2f}s ({tf:.2f}s factors) with {threads} threads on {model}")
    if (ms, ns) == (m, n):
        sample_txt = (f"the whole {m}x{n} layer: both float64 factorisations ({tf:.2f}s) and the recursive "
                      f"float64 solve, measured, on {model}")
    else:
        sample_txt = (f"leading {ms}x{ns} block of the same layer (factors + recursive solve, float64), "
                      f"{t:.2f}s measured on {model}, scaled by the cubic work ratio {scale:.2f}")
    return {"value": round(t * scale, 3), "unit": "s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "measured_s": round(t, 3), "sample": sample_txt}


def cpu_small_forms(WL):
    """Every oracle form timed once on the 64 x 64 workload (seconds, float64,
    host cores): brute-force GPTQ on vec(W) with the explicit Kronecker
    Hessian, BaKron-naive (column-major order), BaKron-antidiagonal and the
    recursive C solve, each including its own factorisation."""
    from oracle import recursive as O2
    from oracle import reference as R
    d = WL.generate(WL.by_name("tiny64"))
    out = {"workload": "tiny64 (64x64)"}

    def timed(name, fn):
        t0 = time.perf_counter()
        fn()
        out[name] = round(time.perf_counter() - t0, 4)

    def factors():
        return R.factor(d["A"]), R.factor(d["B"])

    def brute():
        R.gptq_vectorized(d["W"], R.damp(d["A"]), R.damp(d["B"]), d["scale"], d["zero"], d["maxq"])

    def naive():
        fa, fb = factors()
        R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])

    def antidiag():
        fa, fb = factors()
        R.bakron_antidiagonal(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])

    def recursive():
        fa, fb = factors()
        O2.bakron_recursive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])

    timed("brute_force_vec_gptq_s", brute)
    timed("naive_s", naive)
    timed("antidiagonal_s", antidiag)
    timed("recursive_s", recursive)
    log(f"[bench] cpu oracle forms on 64x64: {out}")
    return out


if __name__ == "__main__":
    main()

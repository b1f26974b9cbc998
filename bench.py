#!/usr/bin/env python3
"""e-means training-step benchmark on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload embedding]

A step is one batch through the whole hot path: batch sampling, fused
assignment, bucketing, per-cluster sums, EMA update (and the revival check
every fifth step). The timed region is one emeans_train call that runs
exactly K steps of the workload's schedule (K = all steps of the 5-pass run
by default), with the data resident in HBM; a separate run with event
profiling gives each kernel class's device time. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "assign TFLOP/s (% MFMA peak) + s to Lloyd-25 MSE, 1M×768 k=4096"
# MI355X dense (i8: TOP/s)
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6, "f16": 2516.6, "i8": 5033.2, "u8": 5033.2,
                    "f8": 5033.2}
HBM_PEAK_GBS = 8000.0

DESCR = {
    "tiny": "tiny: 10k x 16 fp32, 64-component mixture (sigma 0.3), k=64, T=5",
    "embedding": "embedding-like: 1M x 768 fp32, unit-normalised 4096-component mixture, "
                 "Zipf(1.1) weights, sigma 0.5; k=4096, T=5",
    "deep": "deep-descriptor-like: 1M x 96 fp32, unit-normalised rank-32 Gaussian + noise 0.1; "
            "k=16384, T=5",
    "sift": "local-descriptor-like: 1M x 128 fp32 integers in [0,255], 30% zeros; k=16384, T=5",
    "large": "large: 100M x 128 bf16, unit-normalised 65536-component mixture (sigma 0.4); "
             "k=65536, T=3",
}


def kernel_source_sha() -> str:
    """Hash of the assign kernels' sources: counter readings are only reused
    while it is unchanged."""
    h = hashlib.sha256()
    for f in ("assign.hip", "assign_bf16.hip", "assign_i8r.hip", "assign_wide.hip",
              "common.hpp"):  # the sources that define the assign kernels
        with open(os.path.join(HERE, "mini_means_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def assign_kernel_name(dtype: str, d: int) -> str:
    """The assign kernel the library launches for 16-byte aligned rows of this
    dtype and width (the dispatch rule of launch_assign in assign.hip)."""
    if dtype in ("bf16", "f16") and d in (32, 64, 96, 128):
        return f"assign_bf16_kernel (points resident in registers, 32x32x16 {dtype} MFMA)"
    if dtype in ("i8", "u8") and d % 32 == 0 and 32 <= d <= 256:
        return "assign_i8r_kernel (points resident in registers, 32x32x32 int8 MFMA)"
    if dtype in ("i8", "u8") and d in (512, 768):
        return "assign_i8w_kernel (64 points per wave resident, 16x16x64 int8 MFMA)"
    if dtype == "f8" and d in (512, 768):
        return "assign_f8w_kernel (64 points per wave resident, 16x16x128 FP8 MFMA)"
    if d % {"bf16": 8, "f16": 8, "i8": 16, "u8": 16, "f8": 16}.get(dtype, 4) == 0:
        return "assign_ring_kernel (direct-to-LDS stage ring, 16x16 MFMA)"
    return "assign_kernel (register-staged stages, 16x16 MFMA)"


def committed_traffic(workload: str):
    """HBM bytes per assign launch from the committed counter summary
    (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size),
    or None when there is none or the kernel changed since it was taken."""
    path = os.path.join(HERE, "profiles", f"assign_{workload}_traffic.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.strip().startswith("- "):
                key, val = line.strip()[2:].split(":", 1)
                vals[key.strip()] = val.strip().strip("`")
    if vals.get("source_sha256") != kernel_source_sha():
        return None, "kernel changed since the counters were taken"
    return float(vals["hbm_bytes_per_launch"]), path


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def batch_sizes(rc: dict) -> list:
    out = []
    for rows_e, steps in zip(rc["epoch_rows"], rc["steps_per_pass"]):
        out += [min(rc["batch_size"], rows_e - s * rc["batch_size"]) for s in range(steps)]
    return out


def make_data(name: str, W: dict, torch, codes: str = "", mm=None, fp16: bool = False,
              u8: bool = False):
    """Training data, held-out data (fp32 or bf16, on the GPU) and the host
    copy of the training data (None when it is made on the GPU). codes
    ("int8" or "fp8"): the training rows as codes, calibrated on the first
    65536 rows (the data is an iid draw) and encoded on the GPU; returns the
    codes, the held-out data, the host codes (int8, or E4M3 bit patterns) and
    (shift, scale, encode seconds, decode function). fp16: the training rows
    converted once to fp16 on the GPU (held-out rows stay fp32). u8: the
    rows (integers in [0, 255]) stored as uint8 on the GPU, exactly."""
    from mini_means_amd import datagen
    t0 = time.time()
    if u8:
        Xf = torch.from_numpy(datagen.make(W["gen"], W["n"], W["d"])).cuda()
        Xh = torch.from_numpy(datagen.make(W["gen"], W["heldout"], W["d"], split=1)).cuda()
        X = Xf.to(torch.uint8)
        if not torch.equal(X.float(), Xf):
            raise SystemExit("--uint8 needs integer data in [0, 255] (the sift workload)")
        del Xf
        torch.cuda.synchronize()
        log(f"uint8 data {tuple(X.shape)}; data in {time.time() - t0:.1f}s")
        return X, Xh, X.cpu().numpy().view(datagen.U8), None
    if fp16:
        Xf = torch.from_numpy(datagen.make(W["gen"], W["n"], W["d"])).cuda()
        Xh = torch.from_numpy(datagen.make(W["gen"], W["heldout"], W["d"], split=1)).cuda()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        X = Xf.half()
        torch.cuda.synchronize()
        conv_s = time.perf_counter() - t1
        del Xf
        log(f"fp16 data {tuple(X.shape)} converted in {conv_s:.4f}s; data in "
            f"{time.time() - t0:.1f}s")
        return X, Xh, X.cpu().numpy(), None
    if codes:
        cal, enc, dec = ((mm.int8_calibrate, mm.int8_encode, mm.int8_decode) if codes == "int8"
                         else (mm.fp8_calibrate, mm.fp8_encode, mm.fp8_decode))
        Xf = torch.from_numpy(datagen.make(W["gen"], W["n"], W["d"])).cuda()
        Xh = torch.from_numpy(datagen.make(W["gen"], W["heldout"], W["d"], split=1)).cuda()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        shift, scale = cal(Xf[:65536])
        X = enc(Xf, shift, scale)
        torch.cuda.synchronize()
        enc_s = time.perf_counter() - t1
        del Xf
        log(f"{codes} codes {tuple(X.shape)} (scale {scale}) calibrated + encoded in "
            f"{enc_s:.4f}s; data in {time.time() - t0:.1f}s")
        host = X.cpu().numpy() if codes == "int8" else X.view(torch.uint8).cpu().numpy()
        return X, Xh, host, (shift, scale, enc_s, lambda C: dec(C, shift, scale))
    if W["dtype"] == "bf16":
        X = datagen.large_device(n=W["n"], d=W["d"])
        Xh = datagen.large_device(n=W["heldout"], d=W["d"], split=1)
        Xhost = None
    else:
        Xhost = datagen.make(W["gen"], W["n"], W["d"])
        X = torch.from_numpy(Xhost).cuda()
        Xh = torch.from_numpy(datagen.make(W["gen"], W["heldout"], W["d"], split=1)).cuda()
    torch.cuda.synchronize()
    log(f"data {tuple(X.shape)} {X.dtype} + held-out {tuple(Xh.shape)} in {time.time() - t0:.1f}s")
    return X, Xh, Xhost, None


def heldout_mse(mm, Xh, C, torch) -> float:
    _, dist = mm.assign(Xh, C)
    return float(dist.double().mean().item())


def time_to_target(mm, X, Xh, k, target, seeds, Ts, torch, tkw=None, decode=None) -> dict:
    """Smallest median wall-clock among pass counts whose finalised held-out MSE
    reaches the Lloyd-25 held-out MSE (median over training seeds). decode:
    code-space centroids to data space (int8 codes), outside the clock. tkw:
    the run's search options."""
    import statistics
    rows = []
    best = None
    for T in Ts:
        walls, mses = [], []
        for s in seeds:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            out = mm.train(X, k, T, s, capture_labels=True, **(tkw or {}))
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t0)
            C = out.centroids if decode is None else decode(out.centroids)
            mses.append(heldout_mse(mm, Xh, C, torch))
        w, m = statistics.median(walls), statistics.median(mses)
        rows.append(dict(T=T, seconds=round(w, 4), heldout_mse=m))
        log(f"T={T}: {w:.3f}s held-out MSE {m:.6f} (target {target:.6f})")
        if m <= target and (best is None or w < best["seconds"]):
            best = dict(T=T, seconds=w)
    return dict(target_heldout_mse=target, sweep=rows,
                seconds=None if best is None else round(best["seconds"], 4),
                T=None if best is None else best["T"])


def first_crossing(mm, X, Xh, k, T, rc, target, seed, torch, tkw=None, decode=None) -> dict:
    """Secondary time-to-target: the T-pass run's EMA centroids at the end of
    each pass (finalisation off), each prefix timed on its own and evaluated
    outside the clock; the first pass whose held-out MSE reaches the target."""
    rows, hit = [], None
    steps = 0
    for e, st in enumerate(rc["steps_per_pass"]):
        steps += st
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = mm.train(X, k, T, seed, max_steps=steps, finalize=False, capture_labels=False,
                       **(tkw or {}))
        torch.cuda.synchronize()
        w = time.perf_counter() - t0
        C = out.centroids if decode is None else decode(out.centroids)
        m = heldout_mse(mm, Xh, C, torch)
        rows.append(dict(passes=e + 1, seconds=round(w, 4), heldout_mse=m))
        if hit is None and m <= target:
            hit = dict(passes=e + 1, seconds=round(w, 4))
    return dict(T=T, per_pass=rows, first=hit)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(Xhost, C, k, d, budget_s: float, unit: str = "TFLOP/s", workload: str = "",
                 T: float = 5.0) -> dict:
    """The CPU oracle's assignment (fp64 brute force, OpenMP over rows) on a
    bounded sample of the workload's rows, in the metric's unit (codes and
    uint8 data: against the centroids rounded to the search format), on all
    the machine's cores and on one core. The oracle's whole e-means run (T passes)
    and Lloyd-25 run are extrapolated from the multi-core rate (their cost is
    the assignment of every row once per pass or iteration, plus the final
    MSE evaluations) and labelled as such; the times the stored targets took
    when they were made are given beside them."""
    import numpy as np
    import oracle
    C = oracle.search_centroids(C, Xhost)
    rng = np.random.default_rng(0)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    n = len(Xhost)
    npr = 2048
    probe = Xhost[rng.choice(n, npr, replace=False)]
    t0 = time.perf_counter()
    oracle.assign(probe, C, nthreads=cores)
    per_row = (time.perf_counter() - t0) / npr
    rows = int(max(256, min(n, budget_s / max(per_row, 1e-9))))
    sample = Xhost[rng.choice(n, rows, replace=False)]
    t0 = time.perf_counter()
    oracle.assign(sample, C, nthreads=cores)
    dt = time.perf_counter() - t0
    tflops = 2.0 * rows * k * d / dt / 1e12
    # one core, on a sample about a tenth of a second long at that rate
    r1 = int(max(64, min(n, 0.1 * cores / max(dt / rows, 1e-12) / cores)))
    one = sample[:min(r1, rows)]
    t0 = time.perf_counter()
    oracle.assign(one, C, nthreads=1)
    dt1 = time.perf_counter() - t0
    sec_per_row = dt / rows
    out = dict(value=round(tflops, 6), unit=unit, cores=cores, kind="oracle",
               sample=f"{rows} random training rows x all {k} centroids (fp64 brute force, "
                      f"{dt:.1f}s)",
               cpu_model=cpu_model(),
               single_thread={"value": round(2.0 * len(one) * k * d / dt1 / 1e12, 6),
                              "unit": unit, "rows": len(one), "seconds": round(dt1, 3)},
               extrapolated={
                   "emeans_seconds": round((T + 1.0) * n * sec_per_row, 1),
                   "lloyd25_seconds": round(26.0 * n * sec_per_row, 1),
                   "basis": f"{n} rows assigned once per pass ({T:g} passes) or per Lloyd "
                            "iteration (25), plus one final MSE pass, at the sampled "
                            "multi-core rate; grouping and the held-out MSE are left out"})
    measured = {}
    for kind, fname, key in (("emeans", f"freerun_{workload}.json", "oracle_train_seconds"),
                             ("lloyd25", f"lloyd25_{workload}.json", "cpu_seconds")):
        path = os.path.join(HERE, "tests", "golden", fname)
        if workload and os.path.exists(path):
            with open(path) as f:
                g = json.load(f)
            measured[kind] = {"seconds": round(g[key], 1),
                              "threads": g.get("threads"),
                              "where": "when the stored target was written (another host)"}
    if measured:
        out["target_runs"] = measured
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0 = the whole run)")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="embedding")
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-ttt", action="store_true", help="skip the time-to-target sweep")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--ttt-seeds", type=int, default=5)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run a plain device copy of BYTES (counter calibration)")
    ap.add_argument("--search", choices=["bf16", "f16", "f8"], default=None,
                    help="README \"Data precision\", keep FP32 and convert on the fly: the rows "
                         "converted batch by batch for the search (f8: the FP8 converter "
                         "calibrated on the first 65536 rows)")
    ap.add_argument("--center", action="store_true",
                    help="with --search bf16 / f16: subtract the mean of the first 65536 rows "
                         "before rounding (centering)")
    ap.add_argument("--bf16-search", action="store_true",
                    help="search fp32 data in bf16 (README \"Data precision\": the pages' GPU "
                         "default); the held-out MSE is still evaluated in fp32")
    ap.add_argument("--spherical", action="store_true",
                    help="spherical e-means (README \"Spherical e-means\"); no time-to-target")
    ap.add_argument("--int8", action="store_true",
                    help="README \"Data precision\", INT8: calibrate on the first 65536 rows, "
                         "encode on the GPU, train on the codes (exact integer search); "
                         "held-out MSE of the decoded centroids in fp32")
    ap.add_argument("--fp8", action="store_true",
                    help="README \"Data precision\", FP8: as --int8 with E4M3 codes (products "
                         "in FP8, sums in fp32)")
    ap.add_argument("--fp16", action="store_true",
                    help="README \"Data precision\", FP16: the rows converted once to fp16 on "
                         "the GPU (fp16 search, fp32 sums); held-out MSE in fp32")
    ap.add_argument("--uint8", action="store_true",
                    help="README \"Data precision\", UINT8: the SIFT-like rows (integers in "
                         "[0, 255]) stored as uint8 (exact integer search); held-out MSE in fp32")
    ap.add_argument("--print-source-sha", action="store_true")
    args = ap.parse_args()
    if args.print_source_sha:
        print(kernel_source_sha())
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2

    import torch

    import mini_means_amd as mm
    from mini_means_amd import datagen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    mm.lib()
    W = datagen.WORKLOADS[args.workload]
    n, d, k, T = W["n"], W["d"], W["k"], W["T"]
    rc = mm.recipe(n, d, k, T)
    S = rc["total_steps"]
    K = args.steps if args.steps > 0 else S
    K = min(K, S)
    Wm = min(args.warmup, S)
    sizes = batch_sizes(rc)[:K]
    codes_fmt = ("int8" if args.int8 else "fp8" if args.fp8 else "") if W["dtype"] == "f32" else ""
    i8 = codes_fmt == "int8"
    f16 = bool(args.fp16) and W["dtype"] == "f32" and not codes_fmt
    u8 = bool(args.uint8) and W["dtype"] == "f32" and not codes_fmt and not f16
    es = 2 if (W["dtype"] == "bf16" or f16) else (1 if (codes_fmt or u8) else 4)
    flops = float(sum(2.0 * b * k * d for b in sizes))
    # fp32 rows converted on the fly for the search (--search, --bf16-search)
    search = args.search or ("bf16" if args.bf16_search else None)
    if W["dtype"] != "f32" or codes_fmt or f16 or u8:
        search = None
    center = bool(args.center) and search is not None
    # arithmetic type of the search
    sdtype = (search if search else "f16" if f16 else "u8" if u8
              else {"int8": "i8", "fp8": "f8"}.get(codes_fmt, W["dtype"]))
    sph = bool(args.spherical) and not codes_fmt
    tag = (args.workload + (f"_{search}search" if search else "") + ("_centered" if center else "")
           + ("_spherical" if sph else "") + (f"_{codes_fmt}" if codes_fmt else "")
           + ("_fp16" if f16 else "") + ("_uint8" if u8 else ""))
    if sph:
        args.no_ttt = True   # the Lloyd-25 target is Euclidean

    X, Xh, Xhost, codes = make_data(args.workload, W, torch, codes_fmt, mm, f16, u8)
    # the run's search options: the converter's shift and scale come from the
    # first 65536 rows (FP8: calibrated; casts with --center: their mean)
    tkw, conv_info = {}, None
    if search:
        tkw["search"] = search
        t1 = time.perf_counter()
        if search == "f8":
            shift, scale = mm.fp8_calibrate(X[:65536])
            tkw.update(search_shift=shift, search_scale=scale)
            conv_info = {"calibration_rows": 65536, "scale": scale}
        elif center:
            tkw["search_shift"] = X[:65536].double().mean(dim=0).float().contiguous()
            conv_info = {"centering_rows": 65536}
        torch.cuda.synchronize()
        if conv_info is not None:
            conv_info["setup_s"] = round(time.perf_counter() - t1, 4)

    # warm-up (untimed)
    if Wm > 0:
        mm.train(X, k, T, args.seed, max_steps=Wm, spherical=sph, **tkw)
        torch.cuda.synchronize()

    # timed: exactly K steps of the schedule
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = mm.train(X, k, T, args.seed, max_steps=K, spherical=sph, **tkw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    value = flops / wall / 1e12
    log(f"timed {K} steps in {wall:.4f}s -> {value:.2f} assign TFLOP/s (whole step)")

    if args.copy_calibration > 0:
        # a plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copied {args.copy_calibration} bytes x3 for counter calibration")

    # profiled run: device time per kernel class (HIP events on the launch stream)
    prof = mm.train(X, k, T, args.seed, max_steps=K, profile=True, **tkw,
                    spherical=sph).stats
    torch.cuda.synchronize()
    a_ms = prof["ms_assign"]
    assign_tflops = flops / (a_ms / 1e3) / 1e12 if a_ms > 0 else None
    peak = MFMA_PEAK_TFLOPS[sdtype]
    unit = "TOP/s" if (i8 or u8) else "TFLOP/s"
    group_bytes = float(sum(b * d * es + 4 * b + 4 * k * d for b in sizes))
    update_bytes = float(K * (4 * 4 * k * d))   # read s, S, C; write S, C (+ counts, small)
    g_ms = prof["ms_group"]
    u_ms = prof["ms_update"]
    log(f"device ms: assign {a_ms:.2f} bucket {prof['ms_bucket']:.2f} group {g_ms:.2f} "
        f"update {u_ms:.2f} revive {prof['ms_revive']:.2f} sample {prof['ms_sample']:.2f}")

    traffic, tsrc = committed_traffic(tag)
    log(f"traffic: {traffic} ({tsrc})")

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sdtype,
        "data": "synthetic",
        "config": {"workload": DESCR[args.workload], "n": n, "d": d, "k": k, "T": T,
                   "batch": rc["batch_size"], "alpha0": round(rc["alpha0"], 6),
                   "steps_per_run": S,
                   "search": (f"{search} (fp32 rows converted on the fly"
                              + (", centered" if center else "") + "; sums in fp32)") if search
                   else "int8 codes (exact integer search; sums in fp32)" if i8
                   else "FP8 E4M3 codes (FP8 products, fp32 sums)" if codes_fmt == "fp8"
                   else "fp16 data (fp16 products, fp32 sums)" if f16
                   else "uint8 data (exact integer search; sums in fp32)" if u8
                   else ("bf16" if W["dtype"] == "bf16" else "fp32 (exact)"),
                   "mode": "spherical" if sph else "euclidean"},
        "mfma_peak_frac": round(value / peak, 4),
        "roofline": {
            "kernel": assign_kernel_name(sdtype, d),
            "bound": "mfma",
            "achieved": round(assign_tflops, 3) if assign_tflops else None,
            "peak": peak,
            "unit": unit,
            "frac": round(assign_tflops / peak, 4) if assign_tflops else None,
            "traffic": traffic,
            "launches": K,
            "avg_launch_ms": round(a_ms / K, 4),
        },
        "grouping": {
            "group_GBs": round(group_bytes / (g_ms / 1e3) / 1e9, 1) if g_ms > 0 else None,
            "update_GBs": round(update_bytes / (u_ms / 1e3) / 1e9, 1) if u_ms > 0 else None,
            "hbm_peak_GBs": HBM_PEAK_GBS,
            "group_avg_launch_ms": round(g_ms / K, 4),
            "update_avg_launch_ms": round(u_ms / K, 4),
        },
        "device_ms": {c: round(prof[f"ms_{c}"], 3) for c in
                      ("assign", "bucket", "group", "update", "revive", "sample")},
    }

    if codes is not None:
        line["config"][codes_fmt] = {"calibration_rows": 65536, "scale": codes[1],
                                     "calibrate_encode_s": round(codes[2], 4)}
    if conv_info is not None:
        line["config"]["converter"] = conv_info

    if not args.no_ttt:
        dec = codes[3] if codes is not None else None
        # GPU Lloyd-25 on the same resident data, from the same starting rows:
        # the baseline e-means is timed against (and, where the oracle has no
        # stored target, the target itself)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lout = mm.train(X, k, 25.0, args.seed, lloyd=True, capture_labels=False,
                        **tkw)
        torch.cuda.synchronize()
        lloyd_s = time.perf_counter() - t0
        lloyd_mse = heldout_mse(mm, Xh, lout.centroids if dec is None else dec(lout.centroids),
                                torch)
        log(f"GPU Lloyd-25: {lloyd_s:.3f}s, held-out MSE {lloyd_mse:.6f}")
        path = os.path.join(HERE, "tests", "golden", f"lloyd25_{args.workload}.json")
        stored = None
        if os.path.exists(path):
            with open(path) as f:
                stored = json.load(f)
            # a target stored without a record of its splits came from plain Lloyd,
            # which matches the splitting Lloyd only where no cluster empties
            if "empty_cluster_splits" not in stored and lout.stats["n_splits"] > 0:
                log("stored Lloyd-25 target predates the empty-cluster splits: not used")
                stored = None
        if stored is not None:
            target = stored["heldout_mse"]
            source = "oracle Lloyd-25 (tests/golden)"
        else:
            target = lloyd_mse
            source = "GPU Lloyd mode, 25 iterations (parity-tested against the oracle's Lloyd)"
        seeds = [args.seed + i for i in range(args.ttt_seeds)]
        Ts = [1.0, 1.5, 2.0, 2.5, 3.0] if T <= 3.0 else [1.0, 1.25, 1.5, 2.0, 2.5, 3.0, 5.0]
        ttt = time_to_target(mm, X, Xh, k, target, seeds, Ts, torch, tkw, dec)
        ttt.update(target_source=source, gpu_lloyd25_seconds=round(lloyd_s, 4),
                   gpu_lloyd25_heldout_mse=lloyd_mse)
        ttt["first_crossing"] = first_crossing(mm, X, Xh, k, T, rc, target, args.seed, torch,
                                               tkw, dec)
        log(f"first crossing: {ttt['first_crossing']['first']}")
        line["s_to_lloyd25"] = ttt["seconds"]
        line["time_to_target"] = ttt
        # the two closing choices of one run at the workload's T (untimed):
        # the last pass's exact means, the EMA itself and the slow EMA (kappa 2)
        r2 = mm.train(X, k, T, args.seed, slow_ema=2.0, capture_labels=False,
                      **tkw)
        r1 = mm.train(X, k, T, args.seed, slow_ema=1.0, capture_labels=False,
                      **tkw)

        def _ho(C):
            return heldout_mse(mm, Xh, C if dec is None else dec(C), torch)

        line["finalization"] = {"T": T, "heldout_mse": {
            "closing_mean": _ho(r2.centroids), "ema": _ho(r1.slow_centroids),
            "slow_ema_kappa2": _ho(r2.slow_centroids)}}
        log(f"finalization: {line['finalization']}")

    if not args.no_cpu and Xhost is not None:
        C = out.centroids.cpu().numpy()
        line["cpu_baseline"] = cpu_baseline(Xhost, C, k, d, args.cpu_seconds, unit,
                                            args.workload, T)
        log(f"cpu baseline {line['cpu_baseline']}")

    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

#!/usr/bin/env python3
"""Benchmark of the excursion-set hot path on one MI355X.

Metric: POTRF+TRMM FP64-equivalent Tflop/s, (N^3/3 + N^2 nsim) / (T_potrf + T_trmm), and
conditional simulations per second, nsim / (T_trmm + T_scan), on the N = 100,000 workload
(uniform locations in [0,1]^2 in Morton order, Matern nu = 3/2, sigma^2 = 1, range 0.3,
nugget 1e-4, tile 1024, adaptive FP64/FP32/FP16 tiles at tolerance 1e-8, 2,000 seeded N(0,1)
columns, threshold 0.5).

One step = covariance tiles + stats + plan (gpex_cov_gen), mixed-precision tile Cholesky
(gpex_potrf_mp), seeded normals + FP16 compensation + TRMM (gpex_trmm_sim) and the exceedance
scan (gpex_excursion_regions, counts); inputs (locations) are resident in HBM before timing.
Phase times come from HIP events on the library's stream; the dominant kernel's roofline uses
the library's own per-launch events.  The CPU baseline times the oracle on a bounded leading
block of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--trmm-sweep | --krige | --study]
"""
import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TF = {"fp64": 78.6, "fp32": 157.3, "fp16": 2516.6}   # MI355X dense matrix-core peaks
HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def tile_flops(pmap, nt, nb, nsim, amp, diag16=False):
    """Algorithmic flops per compute precision of the tiled Cholesky + TRMM (tiles of nb); diag16:
    the TRMM's diagonal tiles ran on FP16 matrix cores (as two FP16 parts) instead of FP32."""
    f = {"fp64": 0.0, "fp32": 0.0, "fp16": 0.0}
    name = {0: "fp64", 1: "fp32", 2: "fp16"}
    nb3 = float(nb) ** 3
    for k in range(nt):
        f["fp64"] += nb3 / 3.0                                   # POTRF of the diagonal tile
        f["fp64"] += (nt - k - 1) * nb3                          # panel solves, FP64 for every tile
        for j in range(k + 1, nt):
            f["fp64"] += nb3                                     # SYRK of diagonal tile j
            for i in range(j + 1, nt):
                f[name[int(pmap[i, j])]] += 2.0 * nb3            # GEMM in the output tile's precision
    nb2s = float(nb) * nb * nsim
    if amp:
        f["fp16" if diag16 else "fp32"] += nt * nb2s             # diagonal TRMM tiles
        f["fp16"] += nt * (nt - 1) / 2 * 2.0 * nb2s              # off-diagonal tiles in FP16
    else:
        f["fp64"] += nt * nb2s + nt * (nt - 1) * nb2s
    return f


def hbm_rates(info, n, nsim, t_gen_ms, t_scan_ms):
    """Phase-level HBM rates: covariance tiles written by the generator (each lower tile in its
    storage precision; the phase also holds the statistics pass and the host plan) and the S
    entries read by the scan (the phase also holds the host quantile step)."""
    esz = {0: 8, 1: 4, 2: 2}
    pm, nt, nb = info["map"], info["nt"], info["nb"]
    wbytes = sum(esz[int(pm[i, j])] for i in range(nt) for j in range(i + 1)) * float(nb) * nb
    rbytes = float(n) * nsim * 8
    return {"cov_gen": {"bytes_written": wbytes, "GB_per_s": round(wbytes / (t_gen_ms * 1e-3) / 1e9, 1)},
            "scan": {"bytes_read": rbytes, "GB_per_s": round(rbytes / (t_scan_ms * 1e-3) / 1e9, 1)},
            "peak_GB_per_s": HBM_GBS}


# Sources of the trailing-update kernel and its FP64 launches; the counter summary is valid only
# for the code it was taken on.
GEMM_SOURCES = ("gp_conditional_simulation_amd/csrc/gemm_kernel.h", "gp_conditional_simulation_amd/csrc/gemm_f64.hip")


def gemm_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def traffic_per_launch(prec):
    """HBM bytes per trailing-update launch from the committed counter summary, if it was taken
    on the current GEMM source (else None)."""
    path = os.path.join(ROOT, "profiles", f"potrf_update_{prec}_unif100k_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != gemm_source_sha256():
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_baseline(w, rows):
    """Oracle (plain C, FP64, OpenMP) on the leading rows x rows block with all nsim columns."""
    import oracle
    x, y = w.locations()
    m = min(rows, w.n)
    t0 = time.perf_counter()
    V = oracle.cov_matrix(x[:m], y[:m], w.kind, w.sigma2, w.beta, w.nu, nugget=w.nugget)
    t1 = time.perf_counter()
    L, info = oracle.potrf(V)
    t2 = time.perf_counter()
    Z = oracle.normals(w.seed_sim, 0, w.n, w.nsim, rows=(0, m))
    t3 = time.perf_counter()
    M = oracle.trmm(L, Z)
    t4 = time.perf_counter()
    oracle.scan(M, w.u)
    flops = m ** 3 / 3.0 + float(m) ** 2 * w.nsim
    return {"value": flops / ((t2 - t1) + (t4 - t3)) / 1e12, "unit": "Tflop/s (FP64-equivalent)",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"leading {m} x {m} principal block of the same workload (its factor is the leading block "
                      f"of the full factor) with all {w.nsim} columns: Cholesky {t2 - t1:.2f} s + TRMM {t4 - t3:.2f} s "
                      f"(covariance {t1 - t0:.2f} s, normals {t3 - t2:.2f} s not counted), info {info}"}


SWEEP_N = (16384, 32768, 65536, 98304, 131072)
SWEEP_BETA = (("weak", 0.033), ("medium", 0.1), ("strong", 0.234))


def trmm_sweep(args):
    """Single-GPU TRMM throughput against N at three correlation levels, after the shape of the
    pages' single-node TRMM figure ("Mixed-Precision GPU Acceleration for Confidence Regions of
    Spatial Excursion Sets", Fig. 6): N uniform locations (Morton order), Matern nu = 1/2,
    sigma^2 = 1, nugget 1e-4, range 0.033 / 0.1 / 0.234, tile 1024, tolerance 1e-8, nsim columns.
    The factor is computed once per point; the TRMM (seeded normals, B = Z/s in FP16, diagonal at
    about FP32 accuracy, FP16 off-diagonal, FP64 output) is timed over three runs after a warm-up.  Reported
    as N^2 nsim / T and as a multiple of the FP64 matrix-core peak."""
    import numpy as np
    import torch

    import gp_conditional_simulation_amd as g
    import gpex_synth as syn

    dev = torch.device("cuda:0")
    ctx = g.Context(0)
    nsim, nb = args.sweep_nsim, 1024
    sizes = [n for n in SWEEP_N if n <= args.sweep_max_n]
    if args.sweep_n:
        sizes = [int(v) for v in args.sweep_n.split(",")]
    rows = []
    for n in sizes:
        x, y = syn.uniform_locations(n, 1005)
        x, y, _ = syn.ordered_locations(x, y)
        loc = torch.tensor(np.r_[x, y], dtype=torch.float64, device=dev)
        M = g.colmajor(n, nsim, ctx)
        for level, beta in SWEEP_BETA:
            params = {"kind": 0, "sigma2": 1.0, "range": beta, "nu": 0.5, "nugget": 1e-4}
            A = g.cov_gen(ctx, loc, n, params, nb, amp=1, tol=1e-8)
            info = g.potrf_mp(ctx, A)
            if info != 0:
                raise RuntimeError(f"factorisation failed at column {info} (N={n}, range {beta})")
            times = []
            for r in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.trmm_sim(ctx, A, nsim, seed=2005, M=M, want_diag=False)
                e1.record()
                torch.cuda.synchronize()
                if r:
                    times.append(e0.elapsed_time(e1))
            t = statistics.median(times)
            tf = float(n) ** 2 * nsim / (t * 1e-3) / 1e12
            rows.append({"n": n, "correlation": level, "range": beta, "tiles_fp64_fp32_fp16": A.diag["tiles"],
                         "trmm_ms": round(t, 3), "tflops": round(tf, 1),
                         "x_fp64_peak": round(tf / PEAK_TF["fp64"], 2)})
            log(f"N {n} {level}: trmm {t:.2f} ms  {tf:.1f} Tflop/s  {tf / PEAK_TF['fp64']:.2f}x FP64 peak")
            A.close()
        del M, loc
        torch.cuda.empty_cache()
    best = {lv: max(r["x_fp64_peak"] for r in rows if r["correlation"] == lv) for lv, _ in SWEEP_BETA}
    print(json.dumps({"metric": "single-GPU TRMM Tflop/s vs N (N^2 nsim / T_trmm)", "nsim": nsim, "nb": nb,
                      "fp64_peak_tflops": PEAK_TF["fp64"], "max_x_fp64_peak": best, "points": rows}), flush=True)


def krige_bench(args):
    """The kriging workload's conditional path, one step: universal kriging (W, z_hat, v), joint
    covariance tiles + factor, seeded simulations, conditioning + scan + calibration of the regions
    (20,000 prediction + 20,000 observation locations, Matern nu = 3/2, range 0.1, trend
    (0.5, 1, -1), tau^2 = 0.01, FP64, 1,000 simulations, u = 1, level 0.9).  The observations are
    the trend plus seeded N(0, 1) noise: the work does not depend on their values.  Reported as
    nsim / (T_trmm + T_cond+scan) with the factor amortised, and per phase.  The same step with the
    joint factor in mixed precision (tolerance 1e-8, FP16 simulation product; the kriging stays
    FP64) is reported beside it, with the share of cells whose region membership differs from the
    FP64 step's."""
    import numpy as np
    import torch

    import gp_conditional_simulation_amd as g
    import gpex_synth as syn

    w = syn.workload("krige20k")
    if args.nb:
        w = dataclasses.replace(w, nb=args.nb)
    x, y = w.locations()
    n_p, n_o = w.n_pred, w.n_obs
    dev = torch.device("cuda:0")
    f64 = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device=dev)   # noqa: E731
    xp, yp, xo, yo = x[:n_p], y[:n_p], x[n_p:], y[n_p:]
    y_o = syn.trend_mean(xo, yo, w.trend) + np.random.default_rng(w.seed_sim).standard_normal(n_o)
    params = {"kind": w.kind, "sigma2": w.sigma2, "range": w.beta, "nu": w.nu}
    diag_add = f64(np.r_[np.zeros(n_p), np.full(n_o, w.tau2)])
    loc, loc_o, loc_p, dy = f64(np.r_[x, y]), f64(np.r_[xo, yo]), f64(np.r_[xp, yp]), f64(y_o)
    ctx = g.Context(0)
    M = g.colmajor(w.n, w.nsim, ctx)
    torch.cuda.synchronize()

    def step(amp=w.amp, tol=w.tol, dadd=diag_add):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record()
        W, zhat, v, info = g.krige(ctx, loc_o, n_o, loc_p, n_p, dy, 3, params, w.tau2, w.nb)
        ev[1].record()
        A = g.cov_gen(ctx, loc, w.n, dict(params, nugget=0.0), w.nb, amp=amp, tol=tol, diag_add=dadd)
        tiles = A.diag["tiles"]
        ev[2].record()
        fi = g.potrf_mp(ctx, A)
        ev[3].record()
        g.trmm_sim(ctx, A, w.nsim, seed=w.seed_sim, M=M, want_diag=False)
        ev[4].record()
        out = g.excursion_regions(ctx, M, n_p, n_o, w.nsim, w.u, w.level, W=W, y_o=dy, zhat=zhat, v=v)
        ev[5].record()
        torch.cuda.synchronize()
        A.close()
        if info != 0 or fi != 0 or out["status"] != 0:
            raise RuntimeError(f"kriging workload failed: krige {info}, potrf {fi}, regions {out['status']}")
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(5)]
        return dict(zip(("krige", "cov_gen", "potrf", "trmm", "cond_scan_regions"), ms),
                    cin=int(out["cin"].sum().item()), cout=int(out["cout"].sum().item()), tiles=tiles,
                    cin_mask=out["cin"].clone(), cout_mask=out["cout"].clone())

    keys = ("krige", "cov_gen", "potrf", "trmm", "cond_scan_regions")
    # The mixed-precision joint factor of the latent block (no nugget) can lose definiteness: then
    # the mixed-precision steps add 1e-4 sigma^2 on the prediction rows (a documented fallback)
    A = g.cov_gen(ctx, loc, w.n, dict(params, nugget=0.0), w.nb, amp=1, tol=1e-8, diag_add=diag_add)
    mp_info = g.potrf_mp(ctx, A)
    A.close()
    jitter = 0.0 if mp_info == 0 else 1e-4 * w.sigma2
    diag_mp = f64(np.r_[np.full(n_p, jitter), np.full(n_o, w.tau2)])
    for i in range(args.warmup):
        log("warmup", i, {k: round(v, 2) for k, v in step().items() if k in keys})
    recs, recs_mp = [], []
    for i in range(args.steps):
        r = step()
        recs.append(r)
        log("step", i, {k: round(v, 2) for k, v in r.items() if k in keys})
        r2 = step(amp=1, tol=1e-8, dadd=diag_mp)
        recs_mp.append(r2)
        log("step mixed", i, {k: round(v, 2) for k, v in r2.items() if k in keys}, r2["tiles"])
    med = {k: statistics.median(r[k] for r in recs) for k in keys}
    med_mp = {k: statistics.median(r[k] for r in recs_mp) for k in keys}
    d_in = float((recs_mp[-1]["cin_mask"] != recs[-1]["cin_mask"]).double().mean())
    d_out = float((recs_mp[-1]["cout_mask"] != recs[-1]["cout_mask"]).double().mean())
    cond_flops = 2.0 * n_p * w.nsim * n_o
    krige_flops = n_o ** 3 / 3.0 + 2.0 * n_o ** 2 * n_p
    print(json.dumps({
        "metric": "conditional simulations / s, kriging workload (nsim / (T_trmm + T_cond+scan))",
        "value": round(w.nsim / ((med["trmm"] + med["cond_scan_regions"]) * 1e-3), 1), "unit": "simulations/s",
        "config": {"workload": "krige20k: 20,000 prediction + 20,000 observation locations, Matern nu=1.5 range=0.1, "
                               "trend (0.5, 1, -1), tau2 0.01, FP64 tiles, tile 512, nsim 1000, u 1, level 0.9"},
        "steps": args.steps, "warmup": args.warmup, "phase_ms_median": {k: round(v, 2) for k, v in med.items()},
        "krige_fp64_tflops": round(krige_flops / (med["krige"] * 1e-3) / 1e12, 1),
        "joint_potrf_fp64_tflops": round(w.n ** 3 / 3.0 / (med["potrf"] * 1e-3) / 1e12, 1),
        "conditioning_fp64_tflops_lower_bound": round(cond_flops / (med["cond_scan_regions"] * 1e-3) / 1e12, 1),
        "regions_cells": {"cin": recs[-1]["cin"], "cout": recs[-1]["cout"]},
        "mixed_precision": {
            "joint_factor": "tolerance 1e-8 (tile-count-scaled rule), FP16 simulation product; kriging FP64",
            "prediction_row_jitter": jitter,
            "jitter_reason": (f"without it the mixed-precision factor stops at column {mp_info} (non-positive pivot)"
                              if mp_info else "none needed"),
            "tiles_fp64_fp32_fp16": recs_mp[-1]["tiles"],
            "value": round(w.nsim / ((med_mp["trmm"] + med_mp["cond_scan_regions"]) * 1e-3), 1),
            "unit": "simulations/s", "phase_ms_median": {k: round(v, 2) for k, v in med_mp.items()},
            "joint_potrf_fp64_equiv_tflops": round(w.n ** 3 / 3.0 / (med_mp["potrf"] * 1e-3) / 1e12, 1),
            "regions_cells": {"cin": recs_mp[-1]["cin"], "cout": recs_mp[-1]["cout"]},
            "cells_differing_from_fp64": {"inner": d_in, "outer": d_out}},
    }), flush=True)


STUDY_RANGES = (("weak", 0.033), ("medium", 0.1), ("strong", 0.234))
# (label, amp, fixedacc, FP16 destination between TRMM k-tasks)
STUDY_LEVELS = (("DP", 0, 0.0, False),) + tuple((f"1e-{e}", 1, 10.0 ** -e, False) for e in range(4, 15)) + \
    (("1e-4 fp16-dest", 1, 1e-4, True),)


def study(args):
    """The pages' simulation study on one GPU ("Mixed-Precision GPU Acceleration for Confidence
    Regions of Spatial Excursion Sets", Sec. VI-B; Fig. 3 coverage, the DP-vs-fixedacc = 1e-4 cell
    differences, Fig. 5 FP16 tile shares).  Per correlation level (range 0.033 / 0.1 / 0.234):
    3,200 uniform observation locations and a 120 x 120 prediction grid (n = 17,600, prediction
    rows first, each block in Morton order), exponential covariance (Matern 1/2, sigma^2 = 1),
    trend (0, 15, 10) on (1, x, y), u = 10, tau^2 = 0.01 on the observation block, 80,000
    conditional simulations, level 0.9.  Every replicate draws the truth (Z_p, Y_o) = X b + L_V eta
    from the library's FP64 factor of the joint covariance, kriges, and for every precision level
    simulates (same seed), conditions and calibrates; coverage is the share of replicates whose
    C_in lies inside the true excursion set (inner) and whose true set lies inside C_out (outer).
    Levels: all-FP64, fixedacc 1e-4 ... 1e-14 at every decade (Fig. 3's axis), and 1e-4 with the
    FP16 destination of Algorithm 1; levels whose factor coincides (same tile map, scale and
    destination mode) are computed once and reported for each.  Tile 512 (the FP16-destination
    path needs a multiple of 128).  The FP16 shares of Fig. 5 come from the automatic tolerance
    selection on the pages' 34 x 34 tile grid (tile 528)."""
    import numpy as np
    import torch

    import gp_conditional_simulation_amd as g
    import gpex_synth as syn

    dev = torch.device("cuda:0")
    f64 = lambda a: torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device=dev)   # noqa: E731
    reps, nsim, nb, u, level, tau2 = args.study_reps, args.study_nsim, 512, 10.0, 0.9, 0.01
    ranges = [rg for rg in STUDY_RANGES if rg[0] in args.study_ranges.split(",")]
    want = args.study_levels.split(",") if args.study_levels != "all" else [lv[0] for lv in STUDY_LEVELS]
    levels = [lv for lv in STUDY_LEVELS if lv[0] in want]
    if not levels or levels[0][0] != "DP":
        raise SystemExit("--study-levels must include DP (the reference of the cell differences)")
    xp, yp = syn.grid_centres(120)
    xo, yo = syn.uniform_locations(3200, 3005)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    n_p, n_o = len(xp), len(xo)
    n = n_p + n_o
    x, y = np.r_[xp, xo], np.r_[yp, yo]
    mean = f64(syn.trend_mean(x, y, (0.0, 15.0, 10.0)))
    diag_add = f64(np.r_[np.zeros(n_p), np.full(n_o, tau2)])
    loc, loc_o, loc_p = f64(np.r_[x, y]), f64(np.r_[xo, yo]), f64(np.r_[xp, yp])
    ctx = g.Context(0)
    out = {"design": {"n_p": n_p, "n_o": n_o, "nsim": nsim, "reps": reps, "u": u, "level": level, "tau2": tau2,
                      "nb": nb, "trend": [0.0, 15.0, 10.0], "nu": 0.5, "levels": [lv[0] for lv in levels]},
           "ranges": []}
    t_start = time.time()
    M = g.colmajor(n, nsim, ctx)
    for name, beta in ranges:
        params = {"kind": 0, "sigma2": 1.0, "range": beta, "nu": 0.5, "nugget": 0.0}
        # Fig. 5: FP16 share after the automatic tolerance selection, on 34 x 34 tiles
        A = g.cov_gen(ctx, loc, n, params, 528, amp=1, auto_tol=True, diag_add=diag_add)
        auto = {"nt": A.info()["nt"], "tiles_fp64_fp32_fp16": A.diag["tiles"], "tol": A.diag["tol"],
                "reductions": A.diag["tol_reductions"],
                "fp16_share": A.diag["tiles"][2] / sum(A.diag["tiles"])}
        A.close()
        # truths: the FP64 factor of the joint covariance times seeded N(0, 1) columns
        AV = g.cov_gen(ctx, loc, n, params, nb, amp=0, diag_add=diag_add)
        if g.potrf_mp(ctx, AV) != 0:
            raise RuntimeError("joint covariance not positive definite")
        T, _ = g.trmm_sim(ctx, AV, reps, seed=777000 + int(beta * 1000), want_diag=False)
        T = T + mean[:, None]
        AV.close()
        facs, rows, seen = {}, [], {}
        for label, amp, tol, emu in levels:
            A = g.cov_gen(ctx, loc, n, params, nb, amp=amp, tol=tol, diag_add=diag_add, fp16_dest=emu)
            rec = {"level": label, "tiles_fp64_fp32_fp16": A.diag["tiles"], "s": A.diag["s"],
                   "eq10_pass": A.diag["eq10_pass"], "eq11_pass": A.diag["eq11_pass"],
                   "inner": 0, "outer": 0, "joint": 0, "diff_in": 0.0, "diff_out": 0.0}
            # levels whose tile map, scale and destination mode coincide give the same factor and
            # simulations: computed once
            key = (amp, emu, A.diag["s"], A.info()["map"].tobytes())
            if key in seen:
                A.close()
                rec["same_as"] = seen[key]
                rows.append(rec)
                continue
            seen[key] = label
            info = g.potrf_mp(ctx, A)
            rec["potrf_info"] = info
            if info != 0:
                A.close()
                rec["skipped"] = "factorization lost positive definiteness"
            else:
                facs[label] = A
            rows.append(rec)
        live = [r for r in rows if "skipped" not in r and "same_as" not in r]
        t0 = time.time()
        for r in range(reps):
            field = T[:, r]
            z_p, y_o = field[:n_p], field[n_p:].contiguous()
            truth = z_p >= u
            W, zhat, v, info = g.krige(ctx, loc_o, n_o, loc_p, n_p, y_o, 3, params, tau2, nb)
            if info != 0:
                raise RuntimeError("kriging failed")
            ref = None
            for rec in live:
                g.trmm_sim(ctx, facs[rec["level"]], nsim, seed=4000 + r, M=M, want_diag=False)
                o = g.excursion_regions(ctx, M, n_p, n_o, nsim, u, level, W=W, y_o=y_o, zhat=zhat, v=v)
                if o["status"] != 0:
                    raise RuntimeError(f"calibration failed: status {o['status']}")
                cin, cout = o["cin"].bool(), o["cout"].bool()
                ok_in = not bool((cin & ~truth).any())
                ok_out = not bool((truth & ~cout).any())
                rec["inner"] += ok_in
                rec["outer"] += ok_out
                rec["joint"] += ok_in and ok_out
                if ref is None:
                    ref = (cin, cout)
                rec["diff_in"] += float((cin != ref[0]).double().mean())
                rec["diff_out"] += float((cout != ref[1]).double().mean())
            if (r + 1) % 25 == 0:
                log(f"{name} replicate {r + 1}/{reps}: " + ", ".join(
                    f"{rec['level']} {rec['inner'] / (r + 1):.3f}/{rec['outer'] / (r + 1):.3f}" for rec in live) +
                    f"  ({time.time() - t0:.0f} s)")
        for rec in rows:
            if "same_as" in rec:
                src_rec = next(r for r in rows if r["level"] == rec["same_as"])
                for k in ("inner", "outer", "joint", "diff_in", "diff_out"):
                    rec[k] = src_rec[k]
                continue
            for k in ("inner", "outer", "joint", "diff_in", "diff_out"):
                rec[k] = rec[k] / reps
        for A in facs.values():
            A.close()
        out["ranges"].append({"correlation": name, "range": beta, "auto_tolerance_plan": auto, "levels": rows,
                              "seconds": round(time.time() - t0, 1)})
    out["seconds"] = round(time.time() - t_start, 1)
    out["binomial_se_at_0.9"] = float(np.sqrt(0.09 / reps))
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="unif100k_tol1e-8")
    ap.add_argument("--nb", type=int, default=0, help="tile size override for --workload / --krige (0: the recipe's)")
    ap.add_argument("--cpu-rows", type=int, default=10240)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mp", action="store_true", help="skip the mixed-precision N = 100k workloads")
    ap.add_argument("--mp-steps", type=int, default=2)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    ap.add_argument("--trmm-sweep", action="store_true",
                    help="TRMM throughput against N at three correlation levels instead of the step benchmark")
    ap.add_argument("--krige", action="store_true",
                    help="the kriging workload's conditional path instead of the step benchmark")
    ap.add_argument("--study", action="store_true",
                    help="the pages' simulation study (coverage and region differences per tolerance level)")
    ap.add_argument("--study-reps", type=int, default=200)
    ap.add_argument("--study-nsim", type=int, default=80000)
    ap.add_argument("--study-ranges", default="weak,medium,strong")
    ap.add_argument("--study-levels", default="all",
                    help="comma-separated level labels (DP, 1e-4 ... 1e-14, '1e-4 fp16-dest'), or all")
    ap.add_argument("--sweep-nsim", type=int, default=2048)
    ap.add_argument("--sweep-max-n", type=int, default=131072)
    ap.add_argument("--sweep-n", default="", help="comma-separated sizes instead of the sweep's list (multiples of 1024)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library's path is single-device (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if args.trmm_sweep:
        trmm_sweep(args)
        return
    if args.krige:
        krige_bench(args)
        return
    if args.study:
        study(args)
        return

    import numpy as np
    import torch

    import gp_conditional_simulation_amd as g
    import gpex_synth as syn

    w = syn.workload(args.workload)
    if args.nb:
        w = dataclasses.replace(w, nb=args.nb)
    if w.n_obs:
        raise SystemExit("the benchmark workload is an unconditional one")
    x, y = w.locations()
    dev = torch.device("cuda:0")
    loc = torch.tensor(np.r_[x, y], dtype=torch.float64, device=dev)
    params = {"kind": w.kind, "sigma2": w.sigma2, "range": w.beta, "nu": w.nu, "nugget": w.nugget}
    ctx = g.Context(0)
    ctx.set_timing(True)
    M = g.colmajor(w.n, w.nsim, ctx)
    counts_buf = torch.empty(w.n, dtype=torch.int64, device=dev)      # outputs of the scan, reused
    sizes_buf = torch.empty(w.nsim, dtype=torch.int32, device=dev)
    if args.copy_calibration_mib:
        src = torch.ones(args.copy_calibration_mib * 2 ** 20 // 8, dtype=torch.float64, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)          # reads and writes exactly copy_calibration_mib MiB
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()

    def step():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record()
        A = g.cov_gen(ctx, loc, w.n, params, w.nb, amp=w.amp, tol=w.tol)
        ev[1].record()
        info = g.potrf_mp(ctx, A)
        if info != 0:
            raise RuntimeError(f"factorisation failed at column {info}")
        ev[2].record()
        _, d = g.trmm_sim(ctx, A, w.nsim, seed=w.seed_sim, M=M)
        ev[3].record()
        out = g.excursion_regions(ctx, M, w.n, 0, w.nsim, w.u, counts=counts_buf, sizes=sizes_buf)
        ev[4].record()
        torch.cuda.synchronize()
        ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
        tm = ctx.timings()
        inf = A.info()
        A.close()
        return {"gen": ms[0], "potrf": ms[1], "trmm": ms[2], "scan": ms[3], "lib": tm, "diag": d, "info": inf,
                "counts_sum": int(out["counts"].sum().item())}

    for i in range(args.warmup):
        r = step()
        log(f"warmup {i}: gen {r['gen']:.1f} ms potrf {r['potrf']:.1f} ms trmm {r['trmm']:.1f} ms scan {r['scan']:.1f} ms")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = []
    for i in range(args.steps):
        r = step()
        recs.append(r)
        log(f"step {i}: gen {r['gen']:.1f} ms potrf {r['potrf']:.1f} ms trmm {r['trmm']:.1f} ms scan {r['scan']:.1f} ms")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    med = lambda k: statistics.median(r[k] for r in recs)   # noqa: E731
    lo = lambda k: min(r[k] for r in recs)                   # noqa: E731
    hi = lambda k: max(r[k] for r in recs)                   # noqa: E731
    T_potrf, T_trmm, T_scan, T_gen = med("potrf"), med("trmm"), med("scan"), med("gen")
    N, nsim = w.n, w.nsim
    flops = N ** 3 / 3.0 + float(N) ** 2 * nsim
    value = flops / ((T_potrf + T_trmm) * 1e-3) / 1e12
    last = recs[-1]
    info = last["info"]
    lib = last["lib"]
    # dominant kernel: the trailing-update launches of the precision that takes the most time.
    # Flops are counted on the tiles' true sizes (the padded last tile row is not work), divided
    # by the average launch duration (HIP events around each launch on its own stream).  The
    # launches of the two factorization streams overlap, so the busy time (union of the launch
    # intervals) is reported beside it.
    prec = max(("fp64", "fp32", "fp16"), key=lambda p: lib["update_ms"][p])
    launches = lib["update_launches"][prec]
    upd_ms = statistics.median(r["lib"]["update_ms"][prec] for r in recs)
    busy_ms = statistics.median(r["lib"]["update_busy_ms"][prec] for r in recs)
    per_launch_ms = upd_ms / launches
    per_launch_flops = lib["update_flops_exact"][prec] / launches
    achieved = per_launch_flops / (per_launch_ms * 1e-3) / 1e12
    busy_rate = lib["update_flops_exact"][prec] / (busy_ms * 1e-3) / 1e12
    with_diag = all(r["lib"]["trmm_rows_with_diagonal"] for r in recs)
    tf = tile_flops(info["map"], info["nt"], info["nb"], nsim, w.amp, diag16=with_diag)
    t_ideal = sum(tf[p] / (PEAK_TF[p] * 1e12) for p in tf)
    tiles = last["diag"]["tiles"]
    fac = "+".join(p for p, c in zip(("f64", "f32", "f16"), tiles) if c) or "f64"
    trmm_kind = ("f16 TRMM (diagonal as two f16 parts, f32 accumulation)" if with_diag else
                 "f16 TRMM (f32 diagonal, f32 accumulation)") if w.amp else "f64 TRMM"
    dtype = f"{fac} factor tiles + {trmm_kind}"
    trmm_rows_ms = statistics.median(r["lib"]["trmm_rows_ms"] for r in recs)
    nt_, nb_ = info["nt"], info["nb"]
    # algorithmic flops of the launch on the padded columns: 2 nb^2 per off-diagonal tile and
    # column, nb^2 per (triangular) diagonal tile when the launch applies those too
    cols_ = ((nsim + 127) // 128) * 128
    rows_flops = (2.0 * (nt_ * (nt_ - 1) / 2) + (nt_ if with_diag else 0)) * nb_ * nb_ * cols_
    res = {
        "metric": "POTRF+TRMM FP64-equiv Tflop/s and conditional sims/sec at N=100k, 1 MI355X",
        "value": round(value, 3),
        "unit": "Tflop/s (FP64-equivalent, (N^3/3 + N^2 nsim) / (T_potrf + T_trmm))",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N} uniform [0,1]^2 Morton-ordered, Matern nu={w.nu} sigma2={w.sigma2} "
                               f"range={w.beta} nugget={w.nugget}, tile {w.nb}, tol {w.tol}, nsim {nsim}, u {w.u}",
                   "n": N, "nb": w.nb, "nsim": nsim, "tol": w.tol, "tiles_fp64_fp32_fp16": last["diag"]["tiles"],
                   "scale_s": last["diag"]["s"]},
        "sims_per_s": round(nsim / ((T_trmm + T_scan) * 1e-3), 1),
        "sims_per_s_kind": "unconditional simulations per second given the factor: nsim / (T_trmm + T_scan); "
                           "this workload has no observations (the kriging workload's conditional rate is bench.py --krige)",
        "sims_per_s_end_to_end": round(nsim / (ms_per_step * 1e-3), 1),
        "phase_ms_median": {"cov_gen": round(T_gen, 2), "potrf": round(T_potrf, 2), "trmm": round(T_trmm, 2),
                            "scan": round(T_scan, 2)},
        "phase_ms_min": {k: round(lo(r), 2) for k, r in (("cov_gen", "gen"), ("potrf", "potrf"), ("trmm", "trmm"),
                                                         ("scan", "scan"))},
        "phase_ms_max": {k: round(hi(r), 2) for k, r in (("cov_gen", "gen"), ("potrf", "potrf"), ("trmm", "trmm"),
                                                         ("scan", "scan"))},
        "hbm_phase_rates": hbm_rates(info, N, nsim, T_gen, T_scan),
        "precision_weighted_roofline": {"ideal_ms": round(t_ideal * 1e3, 2),
                                        "frac": round(t_ideal / ((T_potrf + T_trmm) * 1e-3), 4),
                                        "flops": {k: float(f"{v:.4e}") for k, v in tf.items()}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TF[prec], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TF[prec], 4), "traffic": traffic_per_launch(prec),
                     "kernel": "gpex::k_gemm_t<{0}, {0}, {0}, {0}, 0, 1, false, 1, 2, 2, 4, 1> (trailing tile update, {1})".format(
                         {"fp64": "double", "fp32": "float", "fp16": "_Float16"}[prec], prec),
                     "launches": launches, "avg_launch_ms": round(per_launch_ms, 4),
                     "flops_per_launch": float(f"{per_launch_flops:.4e}"),
                     "flops_counted": "2 r_i r_j r_k per off-diagonal tile task, r_i^2 r_k per diagonal one, r = true "
                                      "tile rows (unpadded)",
                     "busy_ms": round(busy_ms, 2), "busy_rate_tflops": round(busy_rate, 2),
                     "busy_frac": round(busy_rate / PEAK_TF[prec], 4)},
        "simulation_product": {"kernel": "FP16 row-panel launch of the TRMM (off-diagonal tiles"
                                         + (" and the diagonal tiles' two FP16 parts)" if with_diag else ")"),
                               "ms": round(trmm_rows_ms, 3), "flops": float(f"{rows_flops:.4e}"),
                               "tflops": round(rows_flops / (trmm_rows_ms * 1e-3) / 1e12, 1) if trmm_rows_ms else None,
                               "frac_fp16_peak": round(rows_flops / (trmm_rows_ms * 1e-3) / 1e12 / PEAK_TF["fp16"], 4)
                               if trmm_rows_ms else None},
        "counts_sum": last["counts_sum"],
    }
    if not args.no_mp and args.workload == "unif100k_tol1e-8":
        res["mixed_precision_workloads"] = [mp_workload(args, name, ctx, loc, M) for name in MP_WORKLOADS]
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(res), flush=True)


# Same locations and tolerance as the headline workload at medium and weak correlation, where the
# precision map holds FP32 (and FP16) tiles; measured after the headline, reported beside it.
MP_WORKLOADS = ("unif100k_b0.1_tol1e-8", "unif100k_b0.03_tol1e-8")


def mp_workload(args, name, ctx, loc, M):
    """Factorization + simulation product of a mixed-precision N = 100k workload: args.mp_steps
    measured steps after one warm-up, medians; per-precision trailing-update rates over their
    launches (flops on true tile sizes / summed launch time, and over the busy time)."""
    import torch

    import gp_conditional_simulation_amd as g
    import gpex_synth as syn

    w = syn.workload(name)
    params = {"kind": w.kind, "sigma2": w.sigma2, "range": w.beta, "nu": w.nu, "nugget": w.nugget}
    recs = []
    for i in range(1 + args.mp_steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        A = g.cov_gen(ctx, loc, w.n, params, w.nb, amp=w.amp, tol=w.tol)
        ev[0].record()
        info = g.potrf_mp(ctx, A)
        if info != 0:
            raise RuntimeError(f"{name}: factorisation failed at column {info}")
        ev[1].record()
        g.trmm_sim(ctx, A, w.nsim, seed=w.seed_sim, M=M, want_diag=False)
        ev[2].record()
        torch.cuda.synchronize()
        r = {"potrf": ev[0].elapsed_time(ev[1]), "trmm": ev[1].elapsed_time(ev[2]), "lib": ctx.timings(),
             "diag": dict(A.diag), "info": A.info()}
        A.close()
        log(f"{name} {'warmup' if i == 0 else 'step'}: potrf {r['potrf']:.1f} ms trmm {r['trmm']:.1f} ms")
        if i:
            recs.append(r)
    T_potrf = statistics.median(r["potrf"] for r in recs)
    T_trmm = statistics.median(r["trmm"] for r in recs)
    last = recs[-1]
    tf = tile_flops(last["info"]["map"], last["info"]["nt"], last["info"]["nb"], w.nsim, w.amp,
                    diag16=all(r["lib"]["trmm_rows_with_diagonal"] for r in recs))
    t_ideal = sum(tf[p] / (PEAK_TF[p] * 1e12) for p in tf)
    upd = {}
    for p in ("fp64", "fp32", "fp16"):
        n_l = last["lib"]["update_launches"][p]
        if not n_l:
            continue
        ms = statistics.median(r["lib"]["update_ms"][p] for r in recs)
        busy = statistics.median(r["lib"]["update_busy_ms"][p] for r in recs)
        fl = last["lib"]["update_flops_exact"][p]
        upd[p] = {"launches": n_l, "flops": float(f"{fl:.4e}"), "summed_launch_ms": round(ms, 2),
                  "busy_ms": round(busy, 2), "tflops_per_launch_time": round(fl / (ms * 1e-3) / 1e12, 2),
                  "tflops_busy": round(fl / (busy * 1e-3) / 1e12, 2),
                  "frac_of_peak_busy": round(fl / (busy * 1e-3) / 1e12 / PEAK_TF[p], 4)}
    d = last["diag"]
    N = w.n
    return {"workload": f"{w.name}: N={N}, Matern nu={w.nu} range={w.beta} nugget={w.nugget}, tile {w.nb}, "
                        f"tol {w.tol} (tile-count-scaled rule), nsim {w.nsim}",
            "tiles_fp64_fp32_fp16": d["tiles"], "scale_s": d["s"], "eq10_pass": d["eq10_pass"],
            "eq11_pass": d["eq11_pass"], "steps": args.mp_steps,
            "potrf_ms": round(T_potrf, 2), "trmm_ms": round(T_trmm, 2),
            "value_fp64_equiv_tflops": round((N ** 3 / 3.0 + float(N) ** 2 * w.nsim) / ((T_potrf + T_trmm) * 1e-3) / 1e12,
                                             3),
            "precision_weighted_roofline": {"ideal_ms": round(t_ideal * 1e3, 2),
                                            "frac": round(t_ideal / ((T_potrf + T_trmm) * 1e-3), 4),
                                            "flops": {k: float(f"{v:.4e}") for k, v in tf.items()}},
            "trailing_updates": upd}


if __name__ == "__main__":
    main()

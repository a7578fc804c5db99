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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
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


def tile_flops(pmap, nt, nb, nsim, amp):
    """Algorithmic flops per compute precision of the tiled Cholesky + TRMM (tiles of nb)."""
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
        f["fp32"] += nt * nb2s                                   # diagonal TRMM tiles in FP32
        f["fp16"] += nt * (nt - 1) / 2 * 2.0 * nb2s              # off-diagonal tiles in FP16
    else:
        f["fp64"] += nt * nb2s + nt * (nt - 1) * nb2s
    return f


def traffic_per_launch(prec):
    """HBM bytes per trailing-update launch from the committed counter summary, if it was taken
    on the current GEMM source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"potrf_update_{prec}_unif100k_traffic.json")
    src = os.path.join(ROOT, "gp_conditional_simulation_amd", "csrc", "gemm.hip")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="unif100k_tol1e-8")
    ap.add_argument("--cpu-rows", type=int, default=10240)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library's path is single-device (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gp_conditional_simulation_amd as g
    import gpex_synth as syn

    w = syn.workload(args.workload)
    if w.n_obs:
        raise SystemExit("the benchmark workload is an unconditional one")
    x, y = w.locations()
    dev = torch.device("cuda:0")
    loc = torch.tensor(np.r_[x, y], dtype=torch.float64, device=dev)
    params = {"kind": w.kind, "sigma2": w.sigma2, "range": w.beta, "nu": w.nu, "nugget": w.nugget}
    ctx = g.Context(0)
    ctx.set_timing(True)
    M = g.colmajor(w.n, w.nsim, ctx)
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
        out = g.excursion_regions(ctx, M, w.n, 0, w.nsim, w.u)
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
    T_potrf, T_trmm, T_scan, T_gen = med("potrf"), med("trmm"), med("scan"), med("gen")
    N, nsim = w.n, w.nsim
    flops = N ** 3 / 3.0 + float(N) ** 2 * nsim
    value = flops / ((T_potrf + T_trmm) * 1e-3) / 1e12
    last = recs[-1]
    info = last["info"]
    lib = last["lib"]
    # dominant kernel: the trailing-update launches of the precision that takes the most time
    prec = max(("fp64", "fp32", "fp16"), key=lambda p: lib["update_ms"][p])
    launches = lib["update_launches"][prec]
    upd_ms = statistics.median(r["lib"]["update_ms"][prec] for r in recs)
    per_launch_ms = upd_ms / launches
    per_launch_flops = lib["update_flops"][prec] / launches
    achieved = per_launch_flops / (per_launch_ms * 1e-3) / 1e12
    tf = tile_flops(info["map"], info["nt"], info["nb"], nsim, w.amp)
    t_ideal = sum(tf[p] / (PEAK_TF[p] * 1e12) for p in tf)
    res = {
        "metric": "POTRF+TRMM FP64-equiv Tflop/s and conditional sims/sec at N=100k, 1 MI355X",
        "value": round(value, 3),
        "unit": "Tflop/s (FP64-equivalent, (N^3/3 + N^2 nsim) / (T_potrf + T_trmm))",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64+f32+f16 (per-tile adaptive)", "data": "synthetic",
        "config": {"workload": f"{w.name}: N={N} uniform [0,1]^2 Morton-ordered, Matern nu={w.nu} sigma2={w.sigma2} "
                               f"range={w.beta} nugget={w.nugget}, tile {w.nb}, tol {w.tol}, nsim {nsim}, u {w.u}",
                   "n": N, "nb": w.nb, "nsim": nsim, "tol": w.tol, "tiles_fp64_fp32_fp16": last["diag"]["tiles"],
                   "scale_s": last["diag"]["s"]},
        "sims_per_s": round(nsim / ((T_trmm + T_scan) * 1e-3), 1),
        "sims_per_s_end_to_end": round(nsim / (ms_per_step * 1e-3), 1),
        "phase_ms_median": {"cov_gen": round(T_gen, 2), "potrf": round(T_potrf, 2), "trmm": round(T_trmm, 2),
                            "scan": round(T_scan, 2)},
        "precision_weighted_roofline": {"ideal_ms": round(t_ideal * 1e3, 2),
                                        "frac": round(t_ideal / ((T_potrf + T_trmm) * 1e-3), 4),
                                        "flops": {k: float(f"{v:.4e}") for k, v in tf.items()}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TF[prec], "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_TF[prec], 4), "traffic": traffic_per_launch(prec),
                     "kernel": "gpex::k_gemm_t<{0}, {0}, {0}, {0}, 0, 1, false, 1> (trailing tile update, {1})".format(
                         {"fp64": "double", "fp32": "float", "fp16": "_Float16"}[prec], prec),
                     "launches": launches, "avg_launch_ms": round(per_launch_ms, 4),
                     "flops_per_launch": float(f"{per_launch_flops:.4e}")},
        "counts_sum": last["counts_sum"],
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

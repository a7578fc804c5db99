"""Reduced run of the pages' simulation study: coverage of the inner and outer regions against the
tile-precision tolerance, and how far the regions move from their all-FP64 counterparts.

Design of "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets",
Sec. VI-B: 3,200 uniform observation locations and a 120 x 120 prediction grid (n = 17,600,
prediction rows first), exponential covariance (Matern nu = 1/2, sigma^2 = 1) with range 0.1
(the medium-correlation setting), trend (0, 15, 10) on (1, x, y), threshold u = 10,
80,000 conditional simulations, nominal level 0.9.  Each replicate draws a new truth
(Z_p, Y_o) = X b + L_V eta from the joint covariance (tau^2 = 0.01 on the observation block, the
same reading as the kriging workload), kriges, simulates, conditions and calibrates once per
tolerance level with the same normals, and records whether C_in is inside the true excursion set
and the true set inside C_out (Sec. VI-B), plus the share of prediction cells whose membership
differs from the all-FP64 regions (the comparison the pages make against fixedacc = 1e-4).

The pages use 1,000 replicates per setting; this run takes GPEX_STUDY_REPS (default 200), so the
binomial standard error of a 0.9 rate is 0.021.  It is an experiment rather than a parity gate:
it runs only with GPEX_STUDY=1 and writes its table to GPEX_STUDY_OUT (default
gpurun_out/study.json) when set.
"""
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpex_synth as syn
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)
if os.environ.get("GPEX_STUDY") != "1":  # pragma: no cover
    pytest.skip("the simulation study runs only with GPEX_STUDY=1 (several minutes)", allow_module_level=True)

import gp_conditional_simulation_amd as g  # noqa: E402

M_GRID, N_O, NB, NSIM = 120, 3200, 512, 80000
BETA, U, LEVEL, TAU2 = 0.1, 10.0, 0.9, 0.01
TREND = (0.0, 15.0, 10.0)
REPS = int(os.environ.get("GPEX_STUDY_REPS", "200"))
# (label, amp, tol): all-FP64, then fixedacc from tight to loose (tile-count-scaled rule)
LEVELS = [("DP", 0, 0.0), ("1e-14", 1, 1e-14), ("1e-10", 1, 1e-10), ("1e-8", 1, 1e-8), ("1e-6", 1, 1e-6),
          ("1e-4", 1, 1e-4)]


def dev(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device="cuda:0")


def test_coverage_against_tolerance():
    xp, yp = syn.grid_centres(M_GRID)
    xo, yo = syn.uniform_locations(N_O, 3005)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    n_p = len(xp)
    x, y = np.r_[xp, xo], np.r_[yp, yo]
    n = len(x)
    diag_add = np.r_[np.zeros(n_p), np.full(N_O, TAU2)]
    # truth generator: the oracle's joint covariance, factored by LAPACK
    V = oracle.cov_matrix(x, y, 0, 1.0, BETA, 0.5, diag_add=diag_add)
    LV = np.linalg.cholesky(V)
    del V
    mean = syn.trend_mean(x, y, TREND)
    print(f"\nstudy: n_p {n_p} n_o {N_O} nsim {NSIM} range {BETA} reps {REPS}", flush=True)

    ctx = g.Context(0)
    params = {"kind": 0, "sigma2": 1.0, "range": BETA, "nu": 0.5}
    loc = dev(np.r_[x, y])
    facs = {}
    levels = []
    for label, amp, tol in LEVELS:
        A = g.cov_gen(ctx, loc, n, dict(params, nugget=0.0), NB, amp=amp, tol=tol, diag_add=dev(diag_add))
        info = g.potrf_mp(ctx, A)
        print(f"  {label}: tiles fp64/fp32/fp16 {A.diag['tiles']}, eq10 {A.diag['eq10_pass']}, "
              f"eq11 {A.diag['eq11_pass']}, s {A.diag['s']:.6g}, factorisation info {info}", flush=True)
        if info != 0:   # the level's factor is not usable (loss of positive definiteness)
            A.close()
            continue
        facs[label] = A
        levels.append((label, amp, tol))
    assert levels and levels[0][0] == "DP"
    loc_o, loc_p = dev(np.r_[xo, yo]), dev(np.r_[xp, yp])
    M = g.colmajor(n, NSIM, ctx)
    rec = {lb: {"inner": 0, "outer": 0, "joint": 0, "diff_in": 0.0, "diff_out": 0.0} for lb, _, _ in levels}
    for r in range(REPS):
        eta = np.random.default_rng(20_000_000 + r).standard_normal(n)
        field = mean + LV @ eta
        z_p, y_o = field[:n_p], field[n_p:]
        truth = z_p >= U
        W, zhat, v, info = g.krige(ctx, loc_o, N_O, loc_p, n_p, dev(y_o), 3, params, TAU2, NB)
        assert info == 0
        ref = None
        for label, amp, tol in levels:
            g.trmm_sim(ctx, facs[label], NSIM, seed=4000 + r, M=M, want_diag=False)
            out = g.excursion_regions(ctx, M, n_p, N_O, NSIM, U, LEVEL, W=W, y_o=dev(y_o), zhat=zhat, v=v)
            assert out["status"] == 0
            cin = out["cin"].cpu().numpy().astype(bool)
            cout = out["cout"].cpu().numpy().astype(bool)
            ok_in = not np.any(cin & ~truth)
            ok_out = not np.any(truth & ~cout)
            e = rec[label]
            e["inner"] += ok_in
            e["outer"] += ok_out
            e["joint"] += ok_in and ok_out
            if ref is None:
                ref = (cin, cout)
            e["diff_in"] += np.mean(cin != ref[0])
            e["diff_out"] += np.mean(cout != ref[1])
        if (r + 1) % 20 == 0:
            print(f"  replicate {r + 1}: " + ", ".join(
                f"{lb} {rec[lb]['inner'] / (r + 1):.3f}/{rec[lb]['outer'] / (r + 1):.3f}" for lb, _, _ in levels),
                flush=True)
    table = []
    for label, amp, tol in levels:
        e = rec[label]
        row = {"level": label, "tiles_fp64_fp32_fp16": facs[label].diag["tiles"],
               "inner": e["inner"] / REPS, "outer": e["outer"] / REPS, "joint": e["joint"] / REPS,
               "cells_differing_from_DP_inner": e["diff_in"] / REPS,
               "cells_differing_from_DP_outer": e["diff_out"] / REPS}
        table.append(row)
        print(f"  {label:>6}: inner {row['inner']:.3f} outer {row['outer']:.3f} joint {row['joint']:.3f}  "
              f"differs from DP: inner {100 * row['cells_differing_from_DP_inner']:.3f}% "
              f"outer {100 * row['cells_differing_from_DP_outer']:.3f}%", flush=True)
    out_path = os.environ.get("GPEX_STUDY_OUT", os.path.join("gpurun_out", "study.json"))
    os.makedirs(os.path.dirname(out_path) or ".", exist_ok=True)
    json.dump({"design": {"n_p": n_p, "n_o": N_O, "nsim": NSIM, "range": BETA, "reps": REPS, "u": U,
                          "level": LEVEL, "tau2": TAU2, "nb": NB}, "levels": table}, open(out_path, "w"), indent=1)
    for A in facs.values():
        A.close()
    ctx.close()
    se = np.sqrt(0.9 * 0.1 / REPS)
    for row in table:
        if row["level"] in ("DP", "1e-14", "1e-10", "1e-8"):
            assert abs(row["inner"] - 0.9) <= 4 * se and abs(row["outer"] - 0.9) <= 4 * se, row

"""Reduced run of the pages' simulation study: coverage of the inner and outer regions and how far
the regions move from their all-FP64 counterparts as the tile-precision tolerance loosens.

Design of "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets",
Sec. VI-B, at the medium correlation level: 3,200 uniform observation locations and a 120 x 120
prediction grid (n = 17,600, prediction rows first), exponential covariance (Matern 1/2,
sigma^2 = 1, range 0.1), trend (0, 15, 10) on (1, x, y), u = 10, level 0.9, tau^2 = 0.01 on the
observation block.  Each replicate draws a truth (Z_p, Y_o) = X b + L_V eta from the oracle's
joint covariance (factored by the GPU's LAPACK-style Cholesky in torch, independent of the
library), kriges, simulates with the same seed at every level, conditions and calibrates.

Reduced for the test budget: 100 replicates (binomial standard error of a 0.9 rate: 0.03) and
20,000 simulations instead of 1,000 and 80,000; levels all-FP64, fixedacc 1e-8 and 1e-4 with the
FP16 destination of Algorithm 1.  The full study (three correlation levels, more replicates,
80,000 simulations, FP16 destination on and off) is bench.py --study.  Asserted: coverage of
every level within 3 standard errors of 0.9, fewer than 1% of the cells differing from the
all-FP64 regions (the pages report at most 0.54%), and that the 1e-4 level holds FP16 tiles.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpex_synth as syn
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import gp_conditional_simulation_amd as g  # noqa: E402

M_GRID, N_O, NB, NSIM, REPS = 120, 3200, 512, 20000, 100
BETA, U, LEVEL, TAU2 = 0.1, 10.0, 0.9, 0.01
TREND = (0.0, 15.0, 10.0)
LEVELS = [("DP", 0, 0.0, False), ("1e-8", 1, 1e-8, False), ("1e-4 fp16-dest", 1, 1e-4, True)]


def dev(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device="cuda:0")


def test_coverage_and_region_differences_against_tolerance():
    xp, yp = syn.grid_centres(M_GRID)
    xo, yo = syn.uniform_locations(N_O, 3005)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    n_p = len(xp)
    x, y = np.r_[xp, xo], np.r_[yp, yo]
    n = len(x)
    diag_add = np.r_[np.zeros(n_p), np.full(N_O, TAU2)]
    V = dev(oracle.cov_matrix(x, y, 0, 1.0, BETA, 0.5, diag_add=diag_add))
    LV = torch.linalg.cholesky(V)
    del V
    eta = torch.tensor(np.random.default_rng(20_000_000).standard_normal((n, REPS)), dtype=torch.float64,
                       device="cuda:0")
    truths = LV @ eta + dev(syn.trend_mean(x, y, TREND))[:, None]
    del LV, eta
    ctx = g.Context(0)
    params = {"kind": 0, "sigma2": 1.0, "range": BETA, "nu": 0.5}
    loc = dev(np.r_[x, y])
    facs, recs = {}, {}
    for label, amp, tol, emu in LEVELS:
        A = g.cov_gen(ctx, loc, n, dict(params, nugget=0.0), NB, amp=amp, tol=tol, diag_add=dev(diag_add),
                      fp16_dest=emu)
        assert g.potrf_mp(ctx, A) == 0
        facs[label] = A
        recs[label] = {"inner": 0, "outer": 0, "diff_in": 0.0, "diff_out": 0.0, "tiles": A.diag["tiles"]}
        print(f"  {label}: tiles {A.diag['tiles']} s {A.diag['s']:.6g}", flush=True)
    assert recs["1e-4 fp16-dest"]["tiles"][2] > 0
    loc_o, loc_p = dev(np.r_[xo, yo]), dev(np.r_[xp, yp])
    M = g.colmajor(n, NSIM, ctx)
    for r in range(REPS):
        field = truths[:, r]
        z_p, y_o = field[:n_p], field[n_p:].contiguous()
        truth = z_p >= U
        W, zhat, v, info = g.krige(ctx, loc_o, N_O, loc_p, n_p, y_o, 3, params, TAU2, NB)
        assert info == 0
        ref = None
        for label, _, _, _ in LEVELS:
            g.trmm_sim(ctx, facs[label], NSIM, seed=4000 + r, M=M, want_diag=False)
            out = g.excursion_regions(ctx, M, n_p, N_O, NSIM, U, LEVEL, W=W, y_o=y_o, zhat=zhat, v=v)
            assert out["status"] == 0
            cin, cout = out["cin"].bool(), out["cout"].bool()
            e = recs[label]
            e["inner"] += not bool((cin & ~truth).any())
            e["outer"] += not bool((truth & ~cout).any())
            if ref is None:
                ref = (cin, cout)
            e["diff_in"] += float((cin != ref[0]).double().mean())
            e["diff_out"] += float((cout != ref[1]).double().mean())
    for A in facs.values():
        A.close()
    ctx.close()
    se = np.sqrt(0.9 * 0.1 / REPS)
    for label, e in recs.items():
        inner, outer = e["inner"] / REPS, e["outer"] / REPS
        di, do = e["diff_in"] / REPS, e["diff_out"] / REPS
        print(f"  {label:>15}: inner {inner:.3f} outer {outer:.3f}  cells differing from DP: inner {100 * di:.3f}% "
              f"outer {100 * do:.3f}%", flush=True)
        assert abs(inner - 0.9) <= 3 * se and abs(outer - 0.9) <= 3 * se, (label, inner, outer)
        assert di < 0.01 and do < 0.01, (label, di, do)

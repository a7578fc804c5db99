"""Empirical coverage of the inner and outer confidence regions.

Protocol of "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets",
Sec. VI-B: locations fixed, every replicate draws a new truth (Z_p, Y_o) = X beta + L_V eta from
the joint covariance (tau^2 on the observation block), krige, simulate conditionally, calibrate;
the inner region succeeds when C_in is inside the true excursion set A+_u(Z) on the prediction
locations, the outer region when A+_u(Z) is inside C_out.  Nominal level 0.90.

Shape: the kriging workload's recipe (uniform prediction and observation locations, Matern 3/2,
range 0.1, trend (0.5, 1, -1), tau^2 = 0.01, u = 1, c = 0.9, 1,000 simulations) at 1,024 + 1,024
locations, so that the oracle can factor the joint covariance that generates the truths.
2,000 replicates: the binomial standard error of a 0.9 rate is 0.0067, the +-0.02 band is 3 of them.
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

N_P, N_O, NB, NSIM, REPS = 1024, 1024, 256, 1000, 2000


def dev(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device="cuda:0")


@pytest.fixture(scope="module")
def setup():
    w = syn.workload("krige20k")
    xp, yp = syn.uniform_locations(N_P, w.seed_loc)
    xo, yo = syn.uniform_locations(N_O, w.seed_obs)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    x, y = np.r_[xp, xo], np.r_[yp, yo]
    diag_add = np.r_[np.zeros(N_P), np.full(N_O, w.tau2)]
    # truth generator: the oracle's FP64 factor of the joint covariance
    V = oracle.cov_matrix(x, y, w.kind, w.sigma2, w.beta, w.nu, diag_add=diag_add)
    LV, info = oracle.potrf(V)
    assert info == 0
    mean = syn.trend_mean(x, y, w.trend)
    return w, x, y, xp, yp, xo, yo, diag_add, LV, mean


@pytest.mark.parametrize("amp", [0, 1], ids=["fp64", "mixed"])
def test_region_coverage(setup, amp):
    w, x, y, xp, yp, xo, yo, diag_add, LV, mean = setup
    ctx = g.Context(0)
    params = {"kind": w.kind, "sigma2": w.sigma2, "range": w.beta, "nu": w.nu}
    n = N_P + N_O
    # mixed: tol 1e-8 with the unscaled rule, so that the joint factor holds FP32 tiles (on this
    # 8 x 8 tile shape the tile-count-scaled rule keeps every tile FP64)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, dict(params, nugget=0.0), NB, amp=amp, tol=w.tol,
                  diag_add=dev(diag_add), nt_rule=not amp)
    if amp:
        assert A.diag["tiles"][1] + A.diag["tiles"][2] > 0, "the mixed case must hold reduced-precision tiles"
        print(f"mixed joint factor: tiles {A.diag['tiles']}", flush=True)
    assert g.potrf_mp(ctx, A) == 0
    loc_o, loc_p = dev(np.r_[xo, yo]), dev(np.r_[xp, yp])
    inner = outer = joint = 0
    for r in range(REPS):
        eta = np.random.default_rng(10_000_000 + r).standard_normal(n)
        field = mean + LV @ eta
        z_p, y_o = field[:N_P], field[N_P:]
        W, zhat, v, info = g.krige(ctx, loc_o, N_O, loc_p, N_P, dev(y_o), 3, params, w.tau2, NB)
        assert info == 0
        M, _ = g.trmm_sim(ctx, A, NSIM, seed=w.seed_sim + r, want_diag=False)
        out = g.excursion_regions(ctx, M, N_P, N_O, NSIM, w.u, w.level, W=W, y_o=dev(y_o), zhat=zhat, v=v)
        assert out["status"] == 0
        truth = z_p >= w.u
        cin = out["cin"].cpu().numpy().astype(bool)
        cout = out["cout"].cpu().numpy().astype(bool)
        ok_in = not np.any(cin & ~truth)
        ok_out = not np.any(truth & ~cout)
        inner += ok_in
        outer += ok_out
        joint += ok_in and ok_out
        if (r + 1) % 250 == 0:
            print(f"  replicate {r + 1}: inner {inner / (r + 1):.4f} outer {outer / (r + 1):.4f}", flush=True)
    A.close()
    ctx.close()
    ri, ro, rj = inner / REPS, outer / REPS, joint / REPS
    print(f"coverage ({'mixed' if amp else 'fp64'}): inner {ri:.4f} outer {ro:.4f} joint {rj:.4f} over {REPS}",
          flush=True)
    assert abs(ri - 0.90) <= 0.02
    assert abs(ro - 0.90) <= 0.02

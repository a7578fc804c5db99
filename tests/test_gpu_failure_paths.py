"""Failure paths the pages name, driven through real computations on the GPU.

"Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets":
  * Sec. V-C: positive MSPEs are required.  With tau^2 = 0 and a prediction location equal to an
    observation location, kriging interpolates: zhat = y and v = 0 in exact arithmetic, so the
    computed v is within rounding of 0 and the calibration must reject it exactly when v <= 0.
  * Eq. 4: the latent block of the joint covariance has no error variance; duplicated prediction
    locations make it singular, the factorization reports the failing column, and the documented
    fallback (1e-8 sigma^2 on the prediction rows) factors.
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


def dev(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device="cuda:0")


def dev_cm(a):
    return torch.tensor(np.ascontiguousarray(np.asarray(a).T), dtype=torch.float64, device="cuda:0").T


@pytest.fixture(scope="module")
def ctx():
    c = g.Context(0)
    yield c
    c.close()


@pytest.mark.parametrize("k_trend", [0, 3])
def test_interpolation_point_mspe(ctx, k_trend):
    n_o, n_p, nsim = 300, 40, 64
    xo, yo = syn.uniform_locations(n_o, 5)
    xp, yp = syn.uniform_locations(n_p, 6)
    xp[7], yp[7] = xo[20], yo[20]          # prediction location 7 is observation location 20
    y_obs = syn.trend_mean(xo, yo, (0.5, 1.0, -1.0)) + np.random.default_rng(7).standard_normal(n_o)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), k_trend, params,
                               0.0, 64)
    assert info == 0
    vg, zg = v.cpu().numpy(), zhat.cpu().numpy()
    ro = oracle.krige(xo, yo, xp, yp, y_obs, k_trend, 0, 1.0, 0.1, 1.5, 0.0)
    assert abs(vg[7]) <= 1e-9 and abs(ro["v"][7]) <= 1e-9          # v = 0 up to rounding
    assert zg[7] == pytest.approx(y_obs[20], abs=1e-7)              # zhat = y at the data point
    assert np.all(np.delete(vg, 7) > 0)
    M = dev_cm(syn.explicit_normals(n_p + n_o, nsim, 8))
    out = g.excursion_regions(ctx, M, n_p, n_o, nsim, 0.5, 0.9, W=W, y_o=dev(y_obs), zhat=zhat, v=v)
    expect = g.ERR_MSPE_NONPOS if vg.min() <= 0 else g.OK
    assert out["status"] == expect, (vg[7], out["status"])
    # the rejection itself, with the computed MSPE at the data point set to its exact value 0
    v0 = v.clone()
    v0[7] = 0.0
    out0 = g.excursion_regions(ctx, M, n_p, n_o, nsim, 0.5, 0.9, W=W, y_o=dev(y_obs), zhat=zhat, v=v0)
    assert out0["status"] == g.ERR_MSPE_NONPOS


def test_singular_latent_block_and_documented_fallback(ctx):
    # 24 prediction locations given twice (a prediction grid that repeats cells) and no latent nugget
    n_p, n_o = 600, 400
    xp, yp = syn.uniform_locations(n_p, 11)
    xp[300:324], yp[300:324] = xp[100:124], yp[100:124]
    xo, yo = syn.uniform_locations(n_o, 12)
    x, y = np.r_[xp, xo], np.r_[yp, yo]
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5, "nugget": 0.0}
    diag_add = np.r_[np.zeros(n_p), np.full(n_o, 0.01)]
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n_p + n_o, params, 128, amp=0, diag_add=dev(diag_add))
    info = g.potrf_mp(ctx, A)
    A.close()
    assert info > 0, "exact duplicates must make the latent block singular"
    diag_add[:n_p] = 1e-8 * params["sigma2"]
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n_p + n_o, params, 128, amp=0, diag_add=dev(diag_add))
    assert g.potrf_mp(ctx, A) == 0
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 1.5, diag_add=diag_add)
    Lo, io = oracle.potrf(V)
    assert io == 0
    L = A.to_dense().cpu().numpy()
    # the factor of a matrix this ill-conditioned (kappa ~ 1e8 n) is checked by its backward error
    assert np.linalg.norm(L @ L.T - V) / np.linalg.norm(V) <= 1e-12
    A.close()

"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Tolerances: all-FP64 path relative Frobenius 1e-10 and bit-exact integer exceedance counts;
mixed-precision path 5e-3 for the factor and 1e-2 for simulated fields (relative Frobenius).
Sizes span several tiles with a ragged last tile.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpex_synth as syn
import oracle

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU but skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gp_conditional_simulation_amd as g  # noqa: E402


@pytest.fixture(scope="module")
def ctx():
    c = g.Context(0)
    yield c
    c.close()


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / np.linalg.norm(np.asarray(b)))


def dev(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device="cuda:0")


def dev_cm(a):
    """Column-major device copy of a 2-D numpy array (view n x m)."""
    return torch.tensor(np.ascontiguousarray(np.asarray(a).T), dtype=torch.float64, device="cuda:0").T


def setup_case(n, nb, nu, beta, seed, nugget=1e-4, grid=0):
    if grid:
        x, y = syn.grid_centres(grid)
    else:
        x, y = syn.uniform_locations(n, seed)
    x, y, _ = syn.ordered_locations(x, y)
    params = {"kind": 0, "sigma2": 1.0, "range": beta, "nu": nu, "nugget": nugget}
    return x, y, params


CASES_FP64 = [
    # (n, nb, nu, beta, seed, grid): several tiles, ragged last tile, the 40 x 40 grid workload
    (1600, 160, 0.5, 0.1, 0, 40),
    (1000, 160, 1.5, 0.1, 3, 0),
    (777, 128, 2.5, 0.05, 4, 0),
    (2500, 256, 1.5, 0.3, 5, 0),
]


@pytest.mark.parametrize("case", CASES_FP64, ids=lambda c: f"n{c[0]}_nb{c[1]}_nu{c[2]}")
def test_cov_gen_stats_and_values(ctx, case):
    n, nb, nu, beta, seed, grid = case
    x, y, params = setup_case(n, nb, nu, beta, seed, grid=grid)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    Vg = A.to_dense().cpu().numpy()
    np.testing.assert_allclose(np.tril(Vg), np.tril(V), rtol=1e-13, atol=1e-300)
    st_g = A.stats()
    st_o = oracle.tile_stats(V, nb)
    np.testing.assert_allclose(st_g[:, 0], st_o[:, 0], rtol=1e-12)
    np.testing.assert_allclose(st_g[:, 1:], st_o[:, 1:], rtol=1e-13)
    A.close()


@pytest.mark.parametrize("kind,nu", [(0, 0.5), (0, 1.5), (0, 2.5), (1, 0.5)], ids=["m12", "m32", "m52", "gauss"])
@pytest.mark.parametrize("beta", [1e-7, 1.6e-3, 40.0])
def test_cov_gen_extreme_ranges(ctx, kind, nu, beta):
    """Ranges at the ends of the exponent: 1e-7 (Matern: every off-diagonal entry is an exact zero;
    most exponents are clamped before their integer part is taken), 1.6e-3 (entries from sigma^2
    down through the subnormal range to zero) and 40 (every entry near sigma^2).  The exponent's argument x (r for
    the Matern models, d^2 / range for the Gaussian) carries a few ulps of rounding on either side,
    so an entry may differ by about x ulps relative; subnormal entries by their spacing."""
    n, nb, sigma2 = 700, 128, 2.5
    x, y = syn.uniform_locations(n, 21)
    x, y, _ = syn.ordered_locations(x, y)
    params = {"kind": kind, "sigma2": sigma2, "range": beta, "nu": nu, "nugget": 1e-4}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    V = oracle.cov_matrix(x, y, kind, sigma2, beta, nu, nugget=1e-4)
    Vg = A.to_dense().cpu().numpy()
    A.close()
    low = np.tril_indices(n)
    d2 = (x[:, None] - x[None, :]) ** 2 + (y[:, None] - y[None, :]) ** 2
    arg = d2 / beta if kind == 1 else np.sqrt(d2) / beta
    err = np.abs(Vg[low] - V[low])
    bound = 1e-300 + (1e-14 + 8 * np.finfo(float).eps * arg[low]) * np.abs(V[low])
    assert np.all(err <= bound), float(np.max(err / bound))
    if beta == 1e-7 and kind == 0:
        off = np.tril_indices(n, -1)
        assert np.all(Vg[off] == 0.0) and np.all(np.diag(Vg) == sigma2 + 1e-4)
    if beta == 1.6e-3:
        tiny = V[low][(V[low] > 0) & (V[low] < np.finfo(float).tiny)]
        assert tiny.size > 0   # the case reaches subnormal entries


@pytest.mark.parametrize("nu", [0.3, 0.75, 1.0, 2.2, 6.0])
@pytest.mark.parametrize("beta", [0.1, 0.01])
def test_cov_gen_general_matern_order(ctx, nu, beta):
    """Matern of an order without a closed form (the trapezoidal K_nu of the generator) against the
    oracle's scipy-based 2^(1-nu)/Gamma(nu) r^nu K_nu(r): both carry a few ulps of rounding in r and
    in exp's argument (about r + nu |ln r| ulps) and scipy's K_nu about 1e-14."""
    n, nb, sigma2 = 700, 128, 1.7
    x, y = syn.uniform_locations(n, 31)
    x, y, _ = syn.ordered_locations(x, y)
    params = {"kind": 0, "sigma2": sigma2, "range": beta, "nu": nu, "nugget": 1e-4}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    V = oracle.cov_matrix(x, y, 0, sigma2, beta, nu, nugget=1e-4)
    Vg = A.to_dense().cpu().numpy()
    st_g = A.stats()
    A.close()
    low = np.tril_indices(n)
    r = np.hypot(x[:, None] - x[None, :], y[:, None] - y[None, :])[low] / beta
    lr = np.abs(np.log(np.where(r > 0, r, 1.0)))
    err = np.abs(Vg[low] - V[low])
    bound = 1e-300 + (1e-13 + 8 * np.finfo(float).eps * (r + nu * lr)) * np.abs(V[low])
    assert np.all(err <= bound), float(np.max(err / bound))
    np.testing.assert_allclose(st_g[:, 0], oracle.tile_stats(V, nb)[:, 0], rtol=1e-12)


def test_general_matern_order_factor_simulation_and_kriging(ctx):
    """nu = 0.8 through the rest of the path: the FP64 factor and M = L Z against the oracle's, and
    universal kriging against the oracle's (its covariances from scipy, its algebra the same C code
    as for the closed forms).  The matrices agree to about 1e-14, so the factor and the kriging
    weights agree to that times the conditioning (nugget 1e-4)."""
    n, nb, nsim, nu = 1100, 128, 40, 0.8
    x, y = syn.uniform_locations(n, 33)
    x, y, _ = syn.ordered_locations(x, y)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.15, "nu": nu, "nugget": 1e-4}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    assert g.potrf_mp(ctx, A) == 0
    Z = syn.explicit_normals(n, nsim, 2021)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    Lo, info = oracle.potrf(oracle.cov_matrix(x, y, 0, 1.0, 0.15, nu, nugget=1e-4))
    assert info == 0
    assert rel(A.to_dense().cpu().numpy(), Lo) <= 1e-8
    assert rel(M.cpu().numpy(), oracle.trmm(Lo, Z)) <= 1e-8
    A.close()
    xo, yo, xp, yp, y_obs = _krige_case(900, 300, 8)
    kp = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": nu}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), 900, dev(np.r_[xp, yp]), 300, dev(y_obs), 3, kp, 0.01, 128)
    assert info == 0
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, nu, 0.01)
    assert r["info"] == 0
    assert rel(W.cpu().numpy(), r["W"]) <= 1e-8
    assert rel(zhat.cpu().numpy(), r["zhat"]) <= 1e-8
    assert rel(v.cpu().numpy(), r["v"]) <= 1e-8


@pytest.mark.parametrize("tol", [1e-9, 1e-6, 1e-3])
def test_plan_from_device_stats_matches_oracle_plan(ctx, tol):
    n, nb = 3000, 160
    x, y, params = setup_case(n, nb, 1.5, 0.03, 12)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=tol)
    info = A.info()
    r = oracle.plan(A.stats(), info["nt"], tol, nt_rule=True)
    low = np.tril_indices(info["nt"])
    assert np.array_equal(info["map"][low], r.pmap[low])
    assert info["s"] == r.s and A.diag["s"] == r.s
    assert list(A.diag["tiles"]) == list(r.tiles)
    # stored values: each tile within its precision's rounding of s^2 V (then unscaled)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.03, 1.5, nugget=1e-4)
    Vg = A.to_dense().cpu().numpy()
    nt = info["nt"]
    for i in range(nt):
        for j in range(i + 1):
            a = Vg[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb]
            b = V[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb]
            p = info["map"][i, j]
            eps = {0: 3e-14, 1: 2.0 ** -24 + 3e-14, 2: 2.0 ** -11 + 3e-14}[p]  # exp(-d/beta) amplifies a 1-ulp distance change by d/beta (<= 47 here)
            floor = {0: 0.0, 1: 0.0, 2: 2.0 ** -24 / r.s ** 2}[p]
            assert np.all(np.abs(a - b) <= eps * np.abs(b) * 1.0001 + floor * 0.5001 + 1e-300), (i, j, p)
    A.close()


@pytest.mark.parametrize("case", CASES_FP64, ids=lambda c: f"n{c[0]}_nb{c[1]}_nu{c[2]}")
def test_potrf_fp64(ctx, case):
    n, nb, nu, beta, seed, grid = case
    x, y, params = setup_case(n, nb, nu, beta, seed, grid=grid)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    assert g.potrf_mp(ctx, A) == 0
    L = A.to_dense().cpu().numpy()
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    Lo, info = oracle.potrf(V)
    assert info == 0
    assert np.all(np.triu(L, 1) == 0)
    assert rel(L, Lo) <= 1e-10, rel(L, Lo)
    assert rel(L @ L.T, V) <= 1e-12
    A.close()


def test_tiled_block_matches_dense(ctx):
    n, nb = 700, 128
    x, y, params = setup_case(n, nb, 1.5, 0.1, 8)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    D = A.to_dense().cpu().numpy()
    for (r0, c0, nr, nc) in [(0, 0, 700, 700), (100, 37, 300, 250), (640, 0, 60, 700), (5, 600, 20, 100)]:
        B = A.block(r0, c0, nr, nc).cpu().numpy()
        ref = D[r0:r0 + nr, c0:c0 + nc].copy()
        # above the diagonal tiles the block reads 0; inside diagonal tiles the stored symmetric part
        for i in range(nr):
            for j in range(nc):
                if (c0 + j) // nb > (r0 + i) // nb:
                    ref[i, j] = 0.0
        np.testing.assert_array_equal(B, ref)
    assert g.potrf_mp(ctx, A) == 0
    L = A.to_dense().cpu().numpy()
    np.testing.assert_array_equal(A.block(300, 0, 100, 400).cpu().numpy(), L[300:400, :400])
    A.close()


def test_potrf_reports_non_spd(ctx):
    # a negative diagonal entry at location 150 makes the pivot of column 151 negative
    n, nb = 300, 64
    x, y = syn.uniform_locations(n, 1)
    da = np.full(n, 1e-4)
    da[150] = -1.5
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 0.5, "nugget": 0.0},
                  nb, amp=0, diag_add=dev(da))
    info = g.potrf_mp(ctx, A)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 0.5, diag_add=da)
    _, info_o = oracle.potrf(V)
    assert info == info_o == 151
    A.close()


MP_CASES = [
    # (n, nb, nu, beta, seed, tol, tile-count-scaled rule)
    (3200, 320, 1.5, 0.03, 1002, 1e-9, False),
    (3200, 320, 1.5, 0.1, 1002, 1e-9, False),
    (3200, 320, 1.5, 0.3, 1002, 1e-7, False),
    (4000, 512, 2.5, 0.1, 1003, 1e-6, False),
    (4000, 512, 2.5, 0.1, 1003, 1e-8, False),
    (4000, 512, 2.5, 0.1, 1003, 1e-6, True),
    (3200, 320, 1.5, 0.03, 1002, 1e-7, True),
]


@pytest.mark.parametrize("case", MP_CASES, ids=lambda c: f"n{c[0]}_b{c[3]}_tol{c[5]:g}_{'nt' if c[6] else 'plain'}")
def test_potrf_and_trmm_mixed_precision(ctx, case):
    n, nb, nu, beta, seed, tol, nt_rule = case
    x, y, params = setup_case(n, nb, nu, beta, seed)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=tol, nt_rule=nt_rule)
    assert A.diag["tiles"][1] + A.diag["tiles"][2] > 0, "case must exercise reduced-precision tiles"
    assert g.potrf_mp(ctx, A) == 0
    L = A.to_dense().cpu().numpy()
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    Lo, _ = oracle.potrf(V)
    ef = rel(L, Lo)
    nsim = 200
    Z = syn.explicit_normals(n, nsim, seed + 1)
    M, d = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    Mo = oracle.trmm(Lo, Z)
    em = rel(M.cpu().numpy(), Mo)
    print(f"map {A.diag['tiles']} s {A.diag['s']} factor {ef:.3e} M {em:.3e} normB {d['norm_B']:.4e}")
    assert ef <= 5e-3
    assert em <= 1e-2
    assert d["norm_B"] == pytest.approx(np.linalg.norm(Z) / A.diag["s"], rel=1e-12)
    A.close()


def test_automatic_tolerance_from_device_stats(ctx):
    n, nb = 3000, 160
    x, y, params = setup_case(n, nb, 1.5, 0.03, 12)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, auto_tol=True)
    r = oracle.plan_auto(A.stats(), A.info()["nt"])
    low = np.tril_indices(A.info()["nt"])
    assert np.array_equal(A.info()["map"][low], r.pmap[low])
    assert A.diag["tol"] == r.tol and A.diag["tol_reductions"] == r.reductions
    assert A.status == g.OK and A.diag["eq10_pass"] and A.diag["eq11_pass"]
    assert g.potrf_mp(ctx, A) == 0
    A.close()


def test_loose_tolerance_reports_failed_checks(ctx):
    # tol 1e-4 sends even the tiles beside the diagonal to FP16: Eq. 11 fails and, with a user
    # tolerance, the failure is reported (Sec. V-D) while the factorisation still runs
    n, nb = 2000, 160
    x, y, params = setup_case(n, nb, 1.5, 0.03, 9)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-4, nt_rule=False)
    assert A.status == g.WARN_CHECKS_FAILED
    assert not A.diag["eq11_pass"]
    r = oracle.plan(A.stats(), A.info()["nt"], 1e-4, nt_rule=False)
    assert not r.eq11_pass and A.diag["tiles"] == list(r.tiles)
    assert g.potrf_mp(ctx, A) >= 0
    A.close()


@pytest.mark.parametrize("case", CASES_FP64, ids=lambda c: f"n{c[0]}_nb{c[1]}_nu{c[2]}")
def test_trmm_fp64_counts_bit_exact(ctx, case):
    n, nb, nu, beta, seed, grid = case
    x, y, params = setup_case(n, nb, nu, beta, seed, grid=grid)
    nsim, u = 100, 0.5
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    assert g.potrf_mp(ctx, A) == 0
    Z = syn.explicit_normals(n, nsim, 2001)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    Lo, _ = oracle.potrf(V)
    Mo = oracle.trmm(Lo, Z)
    Mg = M.cpu().numpy()
    assert rel(Mg, Mo) <= 1e-10
    out = g.excursion_regions(ctx, M, n, 0, nsim, u)
    so = oracle.scan(Mo, u)
    near = np.sum(np.abs(Mo - u) < 1e-9)
    assert near == 0, f"{near} near-ties |S-u| < 1e-9 (diagnostic)"
    assert np.array_equal(out["counts"].cpu().numpy(), so["counts"])
    assert np.array_equal(out["sizes"].cpu().numpy(), so["sizes"])
    A.close()


def test_seeded_normals_match_oracle_generator(ctx):
    n, nsim = 1001, 37
    Zg = g.normals(ctx, 2001, 0, n, nsim).cpu().numpy()
    Zo = oracle.normals(2001, 0, n, nsim)
    np.testing.assert_allclose(Zg, Zo, rtol=4e-15, atol=4e-15)
    Zg1 = g.normals(ctx, 77, 3, n, nsim).cpu().numpy()
    np.testing.assert_allclose(Zg1, oracle.normals(77, 3, n, nsim), rtol=4e-15, atol=4e-15)


def test_seeded_trmm_uses_the_seeded_stream(ctx):
    n, nb, nsim = 640, 160, 50
    x, y, params = setup_case(n, nb, 0.5, 0.1, 0)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    assert g.potrf_mp(ctx, A) == 0
    M, _ = g.trmm_sim(ctx, A, nsim, seed=2001)
    Lo, _ = oracle.potrf(oracle.cov_matrix(x, y, 0, 1.0, 0.1, 0.5, nugget=1e-4))
    Mo = oracle.trmm(Lo, oracle.normals(2001, 0, n, nsim))
    assert rel(M.cpu().numpy(), Mo) <= 1e-10
    A.close()


def _krige_case(n_o, n_p, seed, tau2=0.01, beta=0.1, nu=1.5):
    xo, yo = syn.uniform_locations(n_o, seed)
    xp, yp = syn.uniform_locations(n_p, seed + 100)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    rng = np.random.default_rng(seed)
    y_obs = syn.trend_mean(xo, yo, (0.5, 1.0, -1.0)) + rng.standard_normal(n_o)
    return xo, yo, xp, yp, y_obs


@pytest.mark.parametrize("k_trend", [3, 0])
@pytest.mark.parametrize("n_o,n_p,nb", [(1500, 700, 256), (1000, 1000, 160)])
def test_krige_fp64(ctx, k_trend, n_o, n_p, nb):
    xo, yo, xp, yp, y_obs = _krige_case(n_o, n_p, 4)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), k_trend, params,
                               0.01, nb)
    assert info == 0
    r = oracle.krige(xo, yo, xp, yp, y_obs, k_trend, 0, 1.0, 0.1, 1.5, 0.01)
    Wg = W.cpu().numpy()
    assert rel(Wg, r["W"]) <= 1e-10
    assert rel(zhat.cpu().numpy(), r["zhat"]) <= 1e-10
    assert rel(v.cpu().numpy(), r["v"]) <= 1e-10
    if k_trend:
        Xo, Xp = syn.design_matrix(xo, yo), syn.design_matrix(xp, yp)
        np.testing.assert_allclose(Xo.T @ Wg, Xp.T, atol=1e-9)


def test_conditioning_scan_and_regions(ctx):
    n_o, n_p, nb, nsim, u, c = 1200, 800, 256, 300, 1.0, 0.9
    xo, yo, xp, yp, y_obs = _krige_case(n_o, n_p, 21)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), 3, params, 0.01, nb)
    assert info == 0
    x = np.r_[xp, xo]; y = np.r_[yp, yo]
    diag_add = np.r_[np.zeros(n_p), np.full(n_o, 0.01)]
    n = n_p + n_o
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, dict(params, nugget=0.0), nb, amp=0, diag_add=dev(diag_add))
    assert g.potrf_mp(ctx, A) == 0
    Z = syn.explicit_normals(n, nsim, 2004)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    out = g.excursion_regions(ctx, M, n_p, n_o, nsim, u, c, W=W, y_o=dev(y_obs), zhat=zhat, v=v, want_S=True)
    assert out["status"] == 0
    # oracle chain
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.01)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 1.5, diag_add=diag_add)
    Lo, _ = oracle.potrf(V)
    So = oracle.condition(oracle.trmm(Lo, Z), n_p, r["W"], y_obs)
    assert rel(out["S"].cpu().numpy(), So) <= 1e-10
    t = (r["zhat"] - u) / np.sqrt(r["v"])
    sc = oracle.scan(So, u, t)
    assert np.sum(np.abs(So - u) < 1e-9) == 0
    assert np.array_equal(out["counts"].cpu().numpy(), sc["counts"])
    assert np.array_equal(out["sizes"].cpu().numpy(), sc["sizes"])
    np.testing.assert_allclose(out["psi"], sc["psi"], rtol=1e-9)
    np.testing.assert_allclose(out["phi"], sc["phi"], rtol=1e-9)
    cal = oracle.calibrate(sc["psi"], sc["phi"], t, c)
    assert out["n_psi"] == cal["n_psi"] and out["n_phi"] == cal["n_phi"]
    assert out["q_out"] == pytest.approx(cal["q_out"], rel=1e-9)
    assert out["q_in"] == pytest.approx(cal["q_in"], rel=1e-9)
    assert np.array_equal(out["cout"].cpu().numpy(), cal["cout"])
    assert np.array_equal(out["cin"].cpu().numpy(), cal["cin"])
    A.close()


def test_negative_excursion_set_by_sign_reversal(ctx):
    """The negative excursion set {Z <= u} ("Mixed-Precision GPU Acceleration for Confidence Regions
    of Spatial Excursion Sets", Sec. III: reverse the sign of the process and the threshold):
    counts and sizes are #{S <= u} counted directly; psi, phi, the quantiles and both regions are
    the oracle's scan and calibration of -S against -u with t = (u - zhat) / sqrt(v); and the call
    agrees bitwise with the positive-set call on -M, -y_o, -u and -zhat (negation is exact in every
    rounding of the conditioning)."""
    n_o, n_p, nb, nsim, u, c = 1200, 800, 256, 300, 0.5, 0.9
    xo, yo, xp, yp, y_obs = _krige_case(n_o, n_p, 21)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), 3, params, 0.01, nb)
    assert info == 0
    x = np.r_[xp, xo]; y = np.r_[yp, yo]
    diag_add = np.r_[np.zeros(n_p), np.full(n_o, 0.01)]
    n = n_p + n_o
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, dict(params, nugget=0.0), nb, amp=0, diag_add=dev(diag_add))
    assert g.potrf_mp(ctx, A) == 0
    Z = syn.explicit_normals(n, nsim, 2006)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    out = g.excursion_regions(ctx, M, n_p, n_o, nsim, u, c, W=W, y_o=dev(y_obs), zhat=zhat, v=v, want_S=True,
                              below=True)
    assert out["status"] == 0
    S = out["S"].cpu().numpy()
    assert np.array_equal(out["counts"].cpu().numpy(), np.sum(S <= u, axis=1))
    assert np.array_equal(out["sizes"].cpu().numpy(), np.sum(S <= u, axis=0))
    # oracle: the positive-set scan and calibration of the sign-reversed problem
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.01)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 1.5, diag_add=diag_add)
    Lo, _ = oracle.potrf(V)
    So = oracle.condition(oracle.trmm(Lo, Z), n_p, r["W"], y_obs)
    assert rel(S, So) <= 1e-10
    assert np.sum(np.abs(So - u) < 1e-9) == 0
    t = (u - r["zhat"]) / np.sqrt(r["v"])
    sc = oracle.scan(-So, -u, t)
    assert np.array_equal(out["counts"].cpu().numpy(), sc["counts"])
    np.testing.assert_allclose(out["psi"], sc["psi"], rtol=1e-9)
    np.testing.assert_allclose(out["phi"], sc["phi"], rtol=1e-9)
    cal = oracle.calibrate(sc["psi"], sc["phi"], t, c)
    assert out["n_psi"] == cal["n_psi"] and out["n_phi"] == cal["n_phi"]
    assert out["q_out"] == pytest.approx(cal["q_out"], rel=1e-9)
    assert out["q_in"] == pytest.approx(cal["q_in"], rel=1e-9)
    assert np.array_equal(out["cout"].cpu().numpy(), cal["cout"])
    assert np.array_equal(out["cin"].cpu().numpy(), cal["cin"])
    # bitwise against the positive-set call on the negated inputs
    neg = g.excursion_regions(ctx, -M, n_p, n_o, nsim, -u, c, W=W, y_o=dev(-y_obs), zhat=-zhat, v=v)
    assert neg["status"] == 0
    for key in ("counts", "sizes", "cin", "cout"):
        assert np.array_equal(neg[key].cpu().numpy(), out[key].cpu().numpy()), key
    assert np.array_equal(neg["psi"], out["psi"]) and np.array_equal(neg["phi"], out["phi"])
    assert neg["q_in"] == out["q_in"] and neg["q_out"] == out["q_out"]
    A.close()


def test_regions_error_paths(ctx):
    n_p, nsim = 50, 20
    M = dev_cm(np.full((n_p, nsim), -3.0))
    zhat = dev(np.zeros(n_p))
    v = dev(np.ones(n_p))
    out = g.excursion_regions(ctx, M, n_p, 0, nsim, 0.0, 0.9, zhat=zhat, v=v)
    assert out["status"] == g.ERR_EMPTY_SAMPLE and out["n_psi"] == 0
    assert np.all(out["psi"] == np.inf)
    v2 = dev(np.r_[np.ones(n_p - 1), 0.0])
    out = g.excursion_regions(ctx, M, n_p, 0, nsim, -5.0, 0.9, zhat=zhat, v=v2)
    assert out["status"] == g.ERR_MSPE_NONPOS


# ---- edge cases: a single padded tile, n = 1, one and ragged simulation columns, kriging with
# ---- fewer observations than a tile and a single prediction location

@pytest.mark.parametrize("n,nb,nsim", [(1, 16, 1), (37, 64, 1), (100, 128, 129), (160, 160, 3), (161, 160, 257)],
                         ids=lambda v: str(v))
def test_small_and_ragged_fp64(ctx, n, nb, nsim):
    x, y, params = setup_case(n, nb, 1.5, 0.2, 7)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    assert g.potrf_mp(ctx, A) == 0
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.2, 1.5, nugget=1e-4)
    Lo, info = oracle.potrf(V)
    assert info == 0
    Ld = A.to_dense().cpu().numpy()
    assert rel(np.tril(Ld), Lo) <= 1e-12
    assert np.all(np.triu(Ld, 1) == 0.0)
    Z = syn.explicit_normals(n, nsim, 2001)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    Mo = oracle.trmm(Lo, Z)
    assert rel(M.cpu().numpy(), Mo) <= 1e-12
    out = g.excursion_regions(ctx, M, n, 0, nsim, 0.0)
    so = oracle.scan(Mo, 0.0)
    assert np.array_equal(out["counts"].cpu().numpy(), so["counts"])
    assert np.array_equal(out["sizes"].cpu().numpy(), so["sizes"])
    A.close()


@pytest.mark.parametrize("amp,nb", [(0, 256), (1, 256), (0, 320), (1, 320)],
                         ids=["fp64-nb256", "mixed-nb256", "fp64-nb320", "mixed-nb320"])
def test_trmm_writes_only_the_callers_part_of_m(ctx, amp, nb):
    """The simulation product stores rows [0, n) and columns [0, nsim) of M through the caller's
    leading dimension and nothing else: a larger buffer keeps its sentinels outside that part,
    and the part is bitwise the result of a call with ldm = n (ragged last tile and column block;
    tile 320 also takes the bounds-checked kernels of ragged 128-blocks)."""
    import ctypes
    n, nsim, extra_rows = 1000, 300, 37
    x, y, params = setup_case(n, nb, 1.5, 0.1, 11)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=amp, tol=1e-7)
    assert g.potrf_mp(ctx, A) == 0
    Z = dev_cm(syn.explicit_normals(n, nsim, 2011))
    M_ref, _ = g.trmm_sim(ctx, A, nsim, Z=Z)
    ldm = n + extra_rows
    sentinel = 12345.0
    buf = torch.full((nsim + 1, ldm), sentinel, dtype=torch.float64, device="cuda:0")   # column-major ldm x (nsim + 1)
    rc = g.lib().gpex_trmm_sim(ctx.h, A.h, nsim, 0, ctypes.c_void_p(Z.data_ptr()), ctypes.c_void_p(buf.data_ptr()),
                               ldm, None)
    ctx.check(rc, allow=(g.OK,))
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:nsim, :n], M_ref.T.cpu().numpy())
    assert np.all(got[:nsim, n:] == sentinel)
    assert np.all(got[nsim, :] == sentinel)
    A.close()


def test_trmm_256_blocks_rows_and_store_guard(ctx):
    """Row panels large enough for the 256 x 256 FP16 kernel (65 panels x 2 x 8 blocks): sampled
    rows of M, including rows of every 64-row wave group and of the ragged last tile row, equal
    the factor's row times the oracle's seeded normals (to FP16 accuracy), a call through a
    larger leading dimension stores exactly rows [0, n) and columns [0, nsim), bitwise as with
    ldm = n, and the general kernel (diagonal tiles in FP32 in a launch of their own) gives the same
    columns to FP32 rounding."""
    import ctypes
    n, nb, nsim, seed, extra_rows = 33500, 512, 2000, 2013, 37
    x, y, params = setup_case(n, nb, 1.5, 0.1, 13)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-8)
    assert g.potrf_mp(ctx, A) == 0
    M_ref, _ = g.trmm_sim(ctx, A, nsim, seed=seed)
    # tile row 1 (rows 512-1023): every 64-row wave group of both 256-row blocks; tile row 0 has
    # only its diagonal product; rows 33280-33499 are the ragged last tile row
    rows = [0, 512, 600, 700, 800, 900, 1023, 20000, 33279, 33280, 33499]
    Z = oracle.normals(seed, 0, n, nsim, rows=(0, max(rows) + 1))
    Mr = M_ref[rows].cpu().numpy()
    for k, r in enumerate(rows):
        lr = A.block(r, 0, 1, r + 1).cpu().numpy()[0]
        ref = lr @ Z[:r + 1]
        er = np.linalg.norm(Mr[k] - ref) / np.linalg.norm(ref)
        assert er <= 1e-2, (r, er)
    ldm = n + extra_rows
    sentinel = 12345.0
    buf = torch.full((nsim + 1, ldm), sentinel, dtype=torch.float64, device="cuda:0")   # column-major ldm x (nsim + 1)
    rc = g.lib().gpex_trmm_sim(ctx.h, A.h, nsim, seed, None, ctypes.c_void_p(buf.data_ptr()), ldm, None)
    ctx.check(rc, allow=(g.OK,))
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.array_equal(got[:nsim, :n], M_ref.T.cpu().numpy())
    assert np.all(got[:nsim, n:] == sentinel)
    assert np.all(got[nsim, :] == sentinel)
    # 1,920 columns (not a multiple of 256) take the general 128 x 256 kernel for the off-diagonal
    # tiles and an FP32 launch for the diagonal ones; column j of the seeded normals does not depend
    # on nsim, so the shared columns differ only by the diagonal's FP16 parts (about 2^-22 of each
    # entry) and FP32 rounding of the sums
    M_gen, _ = g.trmm_sim(ctx, A, 1920, seed=seed)
    Mg, Mp = M_gen.cpu().numpy(), M_ref[:, :1920].cpu().numpy()
    assert np.linalg.norm(Mg - Mp) / np.linalg.norm(Mp) <= 1e-5
    A.close()


def test_trmm_diagonal_fp16_parts(ctx):
    """The two FP16 parts of each diagonal tile that the row-panel kernel multiplies with:
    hi = cast16(L_kk) and lo = cast16(L_kk - hi) of the stored factor, exactly (numpy's
    float64 -> float16 conversion rounds to nearest even), zeros above the diagonal and outside
    the diagonal tiles; and rows of tile rows 0 and 1 of the product (16 row panels x 4 x 16
    blocks of 256 x 256, so the diagonal tiles join the row panels' launch) equal the factor's rows
    times the seeded normals to FP16 accuracy."""
    n, nb, nsim, seed = 16000, 1024, 4096, 2021
    x, y, params = setup_case(n, nb, 1.5, 0.1, 17)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-8)
    assert g.potrf_mp(ctx, A) == 0
    nt = (n + nb - 1) // nb
    for k in range(nt):
        r0, m = k * nb, min(nb, n - k * nb)
        t = np.tril(A.block_raw(r0, r0, m, m).cpu().numpy())
        P = A.block_raw(r0, 0, m, r0 + m, diag_parts=True).cpu().numpy()
        hi = t.astype(np.float16)
        lo = (t - hi.astype(np.float64)).astype(np.float16)
        assert np.array_equal(P[:, r0:], hi.astype(np.float64) + lo.astype(np.float64)), k
        assert np.all(np.abs(P[:, r0:] - t) <= 2.0 ** -22 * np.abs(t) + 2.0 ** -25), k
        assert not np.any(P[:, :r0]), k
    M, _ = g.trmm_sim(ctx, A, nsim, seed=seed)
    rows = [0, 1, 255, 256, 777, 1023, 1024, 1500, 2047]
    Z = oracle.normals(seed, 0, n, nsim, rows=(0, max(rows) + 1))
    Mr = M[rows].cpu().numpy()
    for k, r in enumerate(rows):
        lr = A.block(r, 0, 1, r + 1).cpu().numpy()[0]
        ref = lr @ Z[:r + 1]
        er = np.linalg.norm(Mr[k] - ref) / np.linalg.norm(ref)
        assert er <= 1e-2, (r, er)
    A.close()


@pytest.mark.parametrize("nb", [160, 320])
def test_diagonal_fp16_parts_small_tiles(ctx, nb):
    """The diagonal tiles' FP16 parts for tile orders that are not a multiple of 256: 160 (not a
    multiple of 64: one (hi, lo) pair as wide as the tile) and 320 (five pairs of 64), with a ragged
    last tile; hi + lo is exactly binary16(L) + binary16(L - binary16(L)) of the stored factor."""
    n = 1000
    x, y, params = setup_case(n, nb, 1.5, 0.05, 23)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-6)
    assert g.potrf_mp(ctx, A) == 0
    L = np.tril(A.block_raw(0, 0, n, n).cpu().numpy())
    P = A.block_raw(0, 0, n, n, diag_parts=True).cpu().numpy()
    for k in range((n + nb - 1) // nb):
        sl = slice(k * nb, min((k + 1) * nb, n))
        t = L[sl, sl]
        hi = t.astype(np.float16)
        lo = (t - hi.astype(np.float64)).astype(np.float16)
        assert np.array_equal(P[sl, sl], hi.astype(np.float64) + lo.astype(np.float64)), k
        P[sl, sl] = 0.0
    assert not np.any(P)
    A.close()


def test_trmm_whole_rows_against_emulation(ctx):
    """The whole-row launch (each diagonal tile as two FP16 parts inside its row's FP32 sum) against
    the oracle's emulation of that form: the leading 4 tile rows and 16 columns of an explicit-Z
    product large enough for the 256 x 256 row-panel kernel (16 row panels x 4 x 16 blocks).  Rows
    below 4 nb depend only on the leading block of the factor, so the emulation runs on that block;
    the two sides differ only in FP32 summation order."""
    n, nb, nsim, m, cols = 16000, 1024, 4096, 4096, 16
    x, y, params = setup_case(n, nb, 1.5, 0.1, 19)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-8)
    assert g.potrf_mp(ctx, A) == 0
    s = A.diag["s"]
    Z = syn.explicit_normals(n, nsim, 2031)
    ctx.set_timing(True)
    try:
        M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
        assert ctx.timings()["trmm_rows_with_diagonal"], "the row-panel kernel did not take the diagonal tiles"
    finally:
        ctx.set_timing(False)
    Ls = np.tril(A.block_raw(0, 0, m, m).cpu().numpy())
    Mg = M[:m, :cols].cpu().numpy()
    Me2 = oracle.trmm_mp_emul(Ls, nb, s, Z[:m, :cols], diag16=True)
    Me0 = oracle.trmm_mp_emul(Ls, nb, s, Z[:m, :cols])
    e2, e0 = rel(Mg, Me2), rel(Mg, Me0)
    print(f"map {A.diag['tiles']}: whole-row launch vs emulation {e2:.2e} (vs the FP32-diagonal emulation {e0:.2e})")
    assert e2 <= 1e-5
    A.close()


def test_single_tile_mixed_precision_simulation(ctx):
    """One tile (no off-diagonal work): the mixed-precision product is the FP32 diagonal alone,
    applied to B = Z / s rounded to FP16, with the scale s of Eq. 12 (no reduced-precision tile:
    u_s = min(65504, 65504 / sqrt(max V_ii)) with max V_ii = 1 + 1e-4, so s = 65499).  This is the
    per-step product path (there are no row panels)."""
    n, nb, nsim = 150, 160, 64
    x, y, params = setup_case(n, nb, 0.5, 0.1, 9)
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-8)
    assert g.potrf_mp(ctx, A) == 0
    assert A.diag["tiles"] == [1, 0, 0]
    Z = syn.explicit_normals(n, nsim, 2002)
    M, d = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    Lo, _ = oracle.potrf(oracle.cov_matrix(x, y, 0, 1.0, 0.1, 0.5, nugget=1e-4))
    Mo = oracle.trmm(Lo, Z)
    assert rel(M.cpu().numpy(), Mo) <= 1e-2
    s = A.diag["s"]
    assert s == math.floor(65504.0 / math.sqrt(1.0 + 1e-4)) - 1.0 == 65499.0
    assert d["norm_B"] == pytest.approx(np.linalg.norm(Z / s), rel=1e-12)   # of Z / s before rounding
    A.close()


@pytest.mark.parametrize("n_o,n_p,nb", [(40, 1, 64), (3, 5, 16), (200, 1, 160)], ids=lambda v: str(v))
def test_krige_small(ctx, n_o, n_p, nb):
    xo, yo, xp, yp, y_obs = _krige_case(n_o, n_p, 31)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), 3, params,
                               0.01, nb)
    assert info == 0
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.01)
    assert rel(W.cpu().numpy(), r["W"]) <= 1e-9
    assert rel(zhat.cpu().numpy(), r["zhat"]) <= 1e-9
    assert rel(v.cpu().numpy(), r["v"]) <= 1e-9


def test_bad_tile_sizes_are_rejected(ctx):
    x, y, params = setup_case(100, 64, 1.5, 0.2, 1)
    for nb in (8, 24, 4096):
        with pytest.raises(g.GpexError):
            g.cov_gen(ctx, dev(np.r_[x, y]), 100, params, nb, amp=0)

"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Every oracle function is checked here against something other than itself: closed forms,
library special cases (scipy / LAPACK routines the oracle does not use), invariants the pages
state, hand-worked fixtures under tests/golden/, and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg as sla
import scipy.special as sps
import scipy.stats as sst

import gpex_synth as syn
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _inf(v):
    return float(v) if not isinstance(v, str) else float(v.replace("inf", "inf"))


def matern_bessel(d, sigma2, beta, nu):
    """General Matern by the modified Bessel function: sigma2 2^(1-nu)/Gamma(nu) r^nu K_nu(r)."""
    r = np.asarray(d, float) / beta
    out = np.full(r.shape, sigma2)
    nz = r > 0
    out[nz] = sigma2 * 2.0 ** (1 - nu) / sps.gamma(nu) * r[nz] ** nu * sps.kv(nu, r[nz])
    return out


# ---------------------------------------------------------------- covariance
@pytest.mark.parametrize("nu", [0.5, 1.5, 2.5])
def test_matern_closed_forms_equal_bessel_definition(nu):
    rng = np.random.default_rng(7)
    d = np.concatenate([[0.0, 1e-9], rng.random(200) * 1.5])
    for beta, s2 in [(0.03, 1.0), (0.1, 2.5), (0.3, 0.7)]:
        got = np.array([oracle.cov(0, s2, beta, nu, x) for x in d])
        ref = matern_bessel(d, s2, beta, nu)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)
        assert got[0] == s2  # C(0) = sigma^2


def test_gaussian_correlation_special_values():
    # page 5: K(x, x') = exp(-||x - x'||^2 / theta); scaled by sigma^2
    theta, s2 = 0.2, 1.7
    assert oracle.cov(1, s2, theta, 0.0, 0.0) == s2
    assert oracle.cov(1, s2, theta, 0.0, math.sqrt(theta)) == pytest.approx(s2 / math.e, rel=1e-15)
    assert oracle.cov(1, s2, theta, 0.0, 2 * math.sqrt(theta)) == pytest.approx(s2 * math.exp(-4), rel=1e-14)
    assert math.isnan(oracle.lib().orc_cov(0, 1.0, 0.1, 0.75, 0.3))  # the C closed forms: half-integer nu only


@pytest.mark.parametrize("nu", [0.5, 1.5, 2.5])
def test_general_matern_equals_closed_forms(nu):
    # the general-order route (scipy kve) at the half-integer orders the C oracle has in closed form
    r = np.concatenate([[0.0, 1e-12, 1e-6], np.geomspace(1e-3, 700, 200)])
    got = oracle.matern_correlation(r, nu)
    ref = np.array([oracle.lib().orc_cov(0, 1.0, 1.0, nu, x) for x in r])
    # both sides round exp's argument (about r ulps at large r)
    assert np.all(np.abs(got - ref) <= (2e-14 + 8 * np.finfo(float).eps * r) * ref + 1e-300)


def test_general_matern_matches_high_precision_bessel():
    # against 30-digit mpmath values of 2^(1-nu)/Gamma(nu) r^nu K_nu(r) (an independent library)
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 30
    for nu in (0.05, 0.3, 0.75, 1.0, 2.2, 3.7, 6.0, 8.0):
        for r in (1e-7, 1e-3, 0.2, 1.0, 3.3, 17.0, 90.0, 400.0):
            ref = float(mp.mpf(2) ** (1 - nu) / mp.gamma(nu) * mp.mpf(r) ** nu * mp.besselk(nu, r))
            got = float(oracle.matern_correlation(np.array([r]), nu)[0])
            assert got == pytest.approx(ref, rel=1e-13 + 8 * np.finfo(float).eps * r), (nu, r)
    # limits: 1 at r = 0 and decreasing in r
    r = np.geomspace(1e-2, 50, 400)
    for nu in (0.3, 1.0, 4.0):
        c = oracle.matern_correlation(np.r_[0.0, 1e-9, r], nu)
        assert c[0] == 1.0 and abs(c[1] - 1.0) < 1e-4 and np.all(np.diff(c[2:]) < 0)


def test_krige_from_matrices_equals_krige():
    # the kriging algebra on given Sigma_y and V_op (the general-order route) is the same C code as
    # the location-based call: bitwise equal at a closed-form order
    rng = np.random.default_rng(5)
    xo, yo, xp, yp = rng.random(60), rng.random(60), rng.random(25), rng.random(25)
    y_obs = rng.standard_normal(60)
    ref = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.1, 0.2, 1.5, 0.02)
    Sy = oracle.cov_matrix(xo, yo, 0, 1.1, 0.2, 1.5, nugget=0.02)
    Vop = oracle.cov_cross(xo, yo, xp, yp, 0, 1.1, 0.2, 1.5)
    W = np.zeros((60, 25), order="F"); z = np.zeros(25); v = np.zeros(25)
    info = oracle.lib().orc_krige_mats(Sy, Vop, xo, yo, 60, xp, yp, 25, y_obs, 3, 1.1, W, z, v, None)
    assert info == 0
    assert np.array_equal(W, ref["W"]) and np.array_equal(z, ref["zhat"]) and np.array_equal(v, ref["v"])
    # a general order goes through it: unbiasedness X_o^T W = X_p^T holds
    g = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.1, 0.2, 0.8, 0.02)
    assert g["info"] == 0
    np.testing.assert_allclose(np.c_[np.ones(60), xo, yo].T @ g["W"], np.c_[np.ones(25), xp, yp].T, atol=1e-10)


def test_cov_matrix_matches_library_distance_and_bessel():
    rng = np.random.default_rng(3)
    x, y = rng.random(40), rng.random(40)
    from scipy.spatial.distance import cdist
    D = cdist(np.c_[x, y], np.c_[x, y])
    V = oracle.cov_matrix(x, y, 0, 1.3, 0.1, 1.5, nugget=1e-4)
    ref = matern_bessel(D, 1.3, 0.1, 1.5) + 1e-4 * np.eye(40)
    np.testing.assert_allclose(V, ref, rtol=1e-12)
    assert np.array_equal(V, V.T)
    da = rng.random(40)
    V2 = oracle.cov_matrix(x, y, 0, 1.3, 0.1, 1.5, nugget=5.0, diag_add=da)
    np.testing.assert_allclose(np.diag(V2), 1.3 + da, rtol=1e-15)
    C = oracle.cov_cross(x[:10], y[:10], x[10:], y[10:], 0, 1.3, 0.1, 1.5)
    np.testing.assert_array_equal(C, V[:10, 10:])


@pytest.mark.parametrize("n,nb", [(37, 8), (64, 16), (10, 3)])
def test_tile_stats_invariants(n, nb):
    rng = np.random.default_rng(n)
    x, y = rng.random(n), rng.random(n)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.2, 0.5, nugget=1e-4)
    st = oracle.tile_stats(V, nb)
    nt = (n + nb - 1) // nb
    tot = 0.0
    for i in range(nt):
        for j in range(i + 1):
            blk = V[i * nb:(i + 1) * nb, j * nb:(j + 1) * nb]
            t = st[i * (i + 1) // 2 + j]
            assert t[1] == blk.min() and t[2] == blk.max()
            np.testing.assert_allclose(t[0], (blk ** 2).sum(), rtol=1e-13)
            tot += t[0] * (1 if i == j else 2)
    np.testing.assert_allclose(tot, np.linalg.norm(V) ** 2, rtol=1e-12)


# ---------------------------------------------------------------- Cholesky
def test_potrf_2x2_closed_form():
    a, b, c = 4.0, 1.2, 3.0
    L, info = oracle.potrf(np.array([[a, b], [b, c]]))
    assert info == 0
    l11 = math.sqrt(a)
    l21 = b / l11
    np.testing.assert_allclose(L, [[l11, 0.0], [l21, math.sqrt(c - l21 ** 2)]], rtol=1e-15)


@pytest.mark.parametrize("n", [1, 5, 8, 200, 600])
def test_potrf_matches_lapack_and_reproduces_matrix(n):
    rng = np.random.default_rng(n)
    x, y = rng.random(n), rng.random(n)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 1.5, nugget=1e-4)
    L, info = oracle.potrf(V)
    assert info == 0
    ref = sla.cholesky(V, lower=True)
    assert np.linalg.norm(L - ref) / np.linalg.norm(ref) < 1e-10
    assert np.all(np.diag(L) > 0) and np.all(np.triu(L, 1) == 0)
    assert np.linalg.norm(L @ L.T - V) / np.linalg.norm(V) <= 10 * n * 2.0 ** -53


def test_potrf_leading_block_property_is_exact():
    rng = np.random.default_rng(11)
    x, y = rng.random(300), rng.random(300)
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.3, 1.5, nugget=1e-4)
    L, _ = oracle.potrf(V)
    Lm, _ = oracle.potrf(V[:97, :97])
    np.testing.assert_array_equal(L[:97, :97], Lm)


def test_potrf_reports_failing_column():
    A = np.diag([4.0, 1.0, -1.0, 2.0])
    assert oracle.potrf(A)[1] == 3
    assert oracle.potrf(np.array([[1.0, 2.0], [2.0, 1.0]]))[1] == 2
    # duplicated location without nugget: singular, the factor breaks down
    x = np.array([0.1, 0.5, 0.1, 0.9]); y = np.array([0.2, 0.5, 0.2, 0.1])
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 0.5, nugget=0.0)
    assert oracle.potrf(V)[1] == 3


# ---------------------------------------------------------------- TRMM, solves, products
def test_trmm_equals_dense_triangular_product():
    rng = np.random.default_rng(5)
    n, ns = 120, 17
    L = np.tril(rng.standard_normal((n, n)))
    A = L + np.triu(rng.standard_normal((n, n)), 1) * 7  # upper part must be ignored
    Z = rng.standard_normal((n, ns))
    M = oracle.trmm(A, Z)
    np.testing.assert_allclose(M, L @ Z, rtol=1e-12, atol=1e-12)
    # leading rows depend only on the leading block of L
    np.testing.assert_array_equal(oracle.trmm(A[:40, :40], Z[:40])[:40], M[:40])


def test_sample_covariance_identity():
    rng = np.random.default_rng(9)
    n, ns = 30, 50
    L = np.tril(rng.standard_normal((n, n)))
    Z = rng.standard_normal((n, ns))
    M = oracle.trmm(L, Z)
    np.testing.assert_allclose(M @ M.T / ns, L @ (Z @ Z.T / ns) @ L.T, rtol=1e-10, atol=1e-10)


def test_triangular_solves_and_gemm():
    rng = np.random.default_rng(2)
    n = 50
    L = np.tril(rng.standard_normal((n, n))) + 8 * np.eye(n)
    B = rng.standard_normal((n, 6))
    X = oracle.trsm_lower(L, B)
    np.testing.assert_allclose(L @ X, B, atol=1e-12)
    X2 = oracle.trsm_lower_trans(L, B)
    np.testing.assert_allclose(L.T @ X2, B, atol=1e-12)
    A = rng.standard_normal((7, 5)); Bm = rng.standard_normal((7, 4))
    np.testing.assert_allclose(oracle.gemm(A, Bm, transa=True), A.T @ Bm, rtol=1e-13)
    np.testing.assert_allclose(oracle.gemm(Bm.T, A.T, transb=True), Bm.T @ A, rtol=1e-13)


# ---------------------------------------------------------------- kriging
def _krige_setup(n_o=60, n_p=40, seed=4, tau2=0.01, nu=1.5, beta=0.1):
    rng = np.random.default_rng(seed)
    xo, yo = rng.random(n_o), rng.random(n_o)
    xp, yp = rng.random(n_p), rng.random(n_p)
    y_obs = rng.standard_normal(n_o) + 0.5 + xo - yo
    return xo, yo, xp, yp, y_obs


def test_krige_unbiasedness_constraint():
    xo, yo, xp, yp, y_obs = _krige_setup()
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.01)
    assert r["info"] == 0
    Xo, Xp = syn.design_matrix(xo, yo), syn.design_matrix(xp, yp)
    np.testing.assert_allclose(Xo.T @ r["W"], Xp.T, atol=1e-9)


def test_krige_explicit_inverse_form():
    # Eq. 5 with explicit inverses and Eq. 6 in its per-column form, at n <= 200
    xo, yo, xp, yp, y_obs = _krige_setup(90, 30, seed=8)
    tau2, s2 = 0.01, 1.0
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, s2, 0.1, 1.5, tau2)
    from scipy.spatial.distance import cdist
    Sy = matern_bessel(cdist(np.c_[xo, yo], np.c_[xo, yo]), s2, 0.1, 1.5) + tau2 * np.eye(90)
    Vop = matern_bessel(cdist(np.c_[xo, yo], np.c_[xp, yp]), s2, 0.1, 1.5)
    Xo, Xp = syn.design_matrix(xo, yo), syn.design_matrix(xp, yp)
    Si = np.linalg.inv(Sy)
    W = Si @ (Vop - Xo @ np.linalg.inv(Xo.T @ Si @ Xo) @ (Xo.T @ Si @ Vop - Xp.T))
    np.testing.assert_allclose(r["W"], W, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(r["zhat"], W.T @ y_obs, rtol=1e-8, atol=1e-10)
    v = np.array([s2 + W[:, i] @ Sy @ W[:, i] - 2 * W[:, i] @ Vop[:, i] for i in range(30)])
    np.testing.assert_allclose(r["v"], v, rtol=1e-7, atol=1e-10)
    assert np.all(r["v"] > 0)


def test_krige_mspe_two_routes_agree():
    # U = Sigma_y W (the page's route) versus the identity U = V_op - X_o H
    xo, yo, xp, yp, y_obs = _krige_setup(80, 25, seed=12)
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.01, want_H=True)
    Vop = oracle.cov_cross(xo, yo, xp, yp, 0, 1.0, 0.1, 1.5)
    Xo = syn.design_matrix(xo, yo)
    U2 = Vop - Xo @ r["H"]
    v2 = 1.0 + (r["W"] * U2).sum(0) - 2 * (Vop * r["W"]).sum(0)
    np.testing.assert_allclose(r["v"], v2, rtol=1e-8, atol=1e-10)


def test_krige_no_trend_is_gp_predictive_equations():
    # page 5 Eq. 1-2 without the psi/N scale: mu = k^T K^-1 Y, var = K(x,x) - k^T K^-1 k
    xo, yo, xp, yp, y_obs = _krige_setup(70, 20, seed=21)
    tau2 = 0.02
    r = oracle.krige(xo, yo, xp, yp, y_obs, 0, 1, 1.0, 0.05, 0.0, tau2)
    from scipy.spatial.distance import cdist
    K = np.exp(-cdist(np.c_[xo, yo], np.c_[xo, yo]) ** 2 / 0.05) + tau2 * np.eye(70)
    k = np.exp(-cdist(np.c_[xo, yo], np.c_[xp, yp]) ** 2 / 0.05)
    KinvK = sla.solve(K, k, assume_a="pos")
    np.testing.assert_allclose(r["zhat"], KinvK.T @ y_obs, rtol=1e-7, atol=1e-9)
    np.testing.assert_allclose(r["v"], 1.0 - (k * KinvK).sum(0), rtol=1e-6, atol=1e-9)


def test_krige_interpolates_with_zero_noise():
    xo, yo, xp, yp, y_obs = _krige_setup(50, 10, seed=31)
    xp[3], yp[3] = xo[17], yo[17]
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.0)
    assert r["info"] == 0
    assert r["zhat"][3] == pytest.approx(y_obs[17], abs=1e-7)
    assert abs(r["v"][3]) < 1e-7


def test_conditional_simulation_mean_and_variance():
    # Sec. V-B: in exact arithmetic E[S] = W^T y_o and diag Cov(S) = v
    n_p, n_o, ns = 12, 30, 60000
    xo, yo, xp, yp, y_obs = _krige_setup(n_o, n_p, seed=41)
    tau2 = 0.05
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.2, 1.5, tau2)
    x = np.r_[xp, xo]; y = np.r_[yp, yo]
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.2, 1.5, diag_add=np.r_[np.zeros(n_p), np.full(n_o, tau2)])
    L, info = oracle.potrf(V)
    assert info == 0
    Z = syn.explicit_normals(n_p + n_o, ns, 5)
    S = oracle.condition(oracle.trmm(L, Z), n_p, r["W"], y_obs)
    se_mean = np.sqrt(r["v"] / ns)
    assert np.all(np.abs(S.mean(1) - r["zhat"]) < 5 * se_mean)
    se_var = r["v"] * np.sqrt(2.0 / ns)
    assert np.all(np.abs(S.var(1) - r["v"]) < 5 * se_var)


# ---------------------------------------------------------------- scan, quantiles, regions
def test_scan_worked_example():
    g = _gold("scan_worked_example.json")
    S = np.array(g["S_rows_by_cols"])
    out = oracle.scan(S, g["u"], np.array(g["t"]))
    assert out["counts"].tolist() == g["counts"]
    assert out["sizes"].tolist() == g["sizes"]
    assert out["psi"].tolist() == [float(v) for v in g["psi"]]
    assert out["phi"].tolist() == [float(v) for v in g["phi"]]


def test_scan_counts_invariant_and_empty_sets():
    rng = np.random.default_rng(1)
    S = rng.standard_normal((9, 33))
    t = rng.standard_normal(9)
    out = oracle.scan(S, 0.3, t)
    assert out["counts"].sum() == out["sizes"].sum()
    S[:, 4] = -5.0
    S[:, 7] = 5.0
    out = oracle.scan(S, 0.3, t)
    assert out["psi"][4] == np.inf and out["sizes"][4] == 0
    assert out["phi"][7] == -np.inf and out["sizes"][7] == 9


def test_quantile_examples():
    g = _gold("quantile_examples.json")
    for c in g["cases"]:
        assert oracle.quantile_index(c["p"], c["n"]) == c["k"], c
    a = np.arange(1.0, 1001.0)[::-1]
    for p in (0.1, 0.5, 0.9, 0.95):
        assert oracle.empirical_quantile(a, p) == math.ceil(round(p * 1000, 6))


def test_regions_worked_example():
    g = _gold("quantile_examples.json")["regions"]
    out = oracle.calibrate([float(v) for v in g["psi"]], [float(v) for v in g["phi"]], g["t"], g["level"])
    for k in ("q_out", "q_in", "n_psi", "n_phi"):
        assert out[k] == g[k]
    assert out["cout"].tolist() == g["cout"] and out["cin"].tolist() == g["cin"]
    with pytest.raises(oracle.regions.EmptySample):
        oracle.calibrate([np.inf, np.inf], [0.0], [0.0], 0.9)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_regions_in_sample_containment(seed):
    # by construction of Eq. 9: at least (1-alpha) of the simulated excursion sets lie inside
    # C_out, and at least (1-alpha) of the simulated non-excursion sets avoid C_in
    rng = np.random.default_rng(seed)
    n, ns, u, c = 25, 400, 0.2, 0.9
    S = rng.standard_normal((n, ns)) + np.linspace(-1, 1, n)[:, None]
    t = np.linspace(-2, 2, n) + 0.01 * rng.standard_normal(n)
    sc = oracle.scan(S, u, t)
    cal = oracle.calibrate(sc["psi"], sc["phi"], t, c)
    cout, cin = cal["cout"].astype(bool), cal["cin"].astype(bool)
    inside = sum(1 for j in range(ns) if (S[:, j] >= u).any() and np.all(cout[S[:, j] >= u]))
    avoid = sum(1 for j in range(ns) if (S[:, j] <= u).any() and not np.any(cin[S[:, j] <= u]))
    assert inside >= (1 - (1 - c)) * cal["n_psi"] - 1e-9
    assert avoid >= (1 - (1 - c)) * cal["n_phi"] - 1e-9
    # brute force over every upper level set {t >= q}: C_out is the smallest one that holds at
    # least n_psi - k + 1 simulated excursion sets (k = ceil(alpha n_psi)); C_in is the largest
    # {t > q} avoided by at least k' = ceil((1 - alpha) n_phi) simulated non-excursion sets
    k = oracle.quantile_index(round(1 - c, 6), cal["n_psi"])
    k2 = oracle.quantile_index(c, cal["n_phi"])
    for q in np.r_[t, cal["q_out"], cal["q_in"]]:
        cnt = sum(1 for j in range(ns) if (S[:, j] >= u).any() and np.all(t[S[:, j] >= u] >= q))
        cnt2 = sum(1 for j in range(ns) if (S[:, j] <= u).any() and not np.any(t[S[:, j] <= u] > q))
        if q <= cal["q_out"]:
            assert cnt >= cal["n_psi"] - k + 1
        else:
            assert cnt <= cal["n_psi"] - k
        if q >= cal["q_in"]:
            assert cnt2 >= k2
        else:
            assert cnt2 <= k2 - 1


# ---------------------------------------------------------------- random numbers
def test_normals_are_standard_normal_and_independent():
    Z = oracle.normals(2005, 0, 1000, 200)
    z = Z.ravel(order="F")
    assert abs(z.mean()) < 5 / math.sqrt(z.size)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / z.size)
    assert sst.kstest(z, "norm").pvalue > 1e-3
    # lag-1 correlation along the generation order (pairs share a Box-Muller draw)
    assert abs(np.corrcoef(z[:-1], z[1:])[0, 1]) < 5 / math.sqrt(z.size)
    Z2 = oracle.normals(2006, 0, 1000, 200)
    Z3 = oracle.normals(2005, 1, 1000, 200)
    for other in (Z2, Z3):
        assert abs(np.corrcoef(z, other.ravel(order="F"))[0, 1]) < 5 / math.sqrt(z.size)


def test_normals_counter_based_blocks_and_box_muller_radius():
    Z = oracle.normals(77, 0, 101, 13)
    B = oracle.normals(77, 0, 101, 13, rows=(37, 90), cols=(3, 11))
    np.testing.assert_array_equal(B, Z[37:90, 3:11])
    # the two members of a pair share the radius sqrt(-2 ln u1) from words 0-1
    z = Z.ravel(order="F")
    for p in (0, 5, 300):
        w = oracle.philox4x32_10([p, 0, 0, 0], [77, 0])
        u1 = ((int(w[1]) << 32 | int(w[0])) >> 11) * 2.0 ** -53 + 2.0 ** -54
        assert z[2 * p] ** 2 + z[2 * p + 1] ** 2 == pytest.approx(-2 * math.log(u1), rel=1e-12)


def test_philox_uniform_words_and_key_sensitivity():
    ws = np.array([oracle.philox4x32_10([i, 0, 0, 0], [1, 2]) for i in range(4000)], dtype=np.uint64)
    bits = ((ws[:, :, None] >> np.arange(32, dtype=np.uint64)) & np.uint64(1)).astype(float)
    # every output bit is a fair coin
    assert np.all(np.abs(bits.mean(0) - 0.5) < 5 * 0.5 / math.sqrt(4000))
    # a one-bit change of key or counter flips about half of the output bits
    a = oracle.philox4x32_10([9, 0, 0, 0], [1, 2])
    b = oracle.philox4x32_10([9, 0, 0, 0], [1, 3])
    c = oracle.philox4x32_10([8, 0, 0, 0], [1, 2])
    for o in (b, c):
        flips = sum(bin(int(x) ^ int(y)).count("1") for x, y in zip(a, o))
        assert 30 < flips < 98


# ---------------------------------------------------------------- planner
def test_planner_printed_constants():
    assert oracle.planner.EQ10_LIMIT == pytest.approx(1.10e12, rel=5e-3)
    assert oracle.planner.EPS[oracle.planner.FP16] == 2.0 ** -10
    assert oracle.planner.X_MAX[oracle.planner.FP32] == np.finfo(np.float32).max
    assert oracle.planner.X_MIN_NORM[oracle.planner.FP16] == np.finfo(np.float16).tiny
    assert oracle.planner.X_MIN_SUB[oracle.planner.FP16] == np.finfo(np.float16).smallest_subnormal
    assert oracle.planner.X_MAX[oracle.planner.FP16] == np.finfo(np.float16).max


def test_planner_worked_example():
    g = _gold("planner_worked_example.json")
    r = oracle.plan(np.array(g["stats"]), g["nt"], g["tol"])
    for i, row in enumerate(g["pmap_lower"]):
        assert r.pmap[i, :i + 1].tolist() == row
    assert r.s == g["s"]
    assert r.l_bound == pytest.approx(g["l_bound_approx"], rel=1e-4)
    assert r.eq10_pass == g["eq10_pass"] and r.eq11_pass == g["eq11_pass"]
    assert list(r.tiles) == g["tiles"]


def test_planner_rule_variants_worked_example():
    g = _gold("planner_worked_example.json")
    rc = g["rule_cases"]
    st = np.array(g["stats"])
    ru = oracle.plan(st, g["nt"], rc["tol"], nt_rule=False)
    rs = oracle.plan(st, g["nt"], rc["tol"], nt_rule=True)
    for i in range(g["nt"]):
        assert ru.pmap[i, :i + 1].tolist() == rc["unscaled_pmap_lower"][i]
        assert rs.pmap[i, :i + 1].tolist() == rc["scaled_pmap_lower"][i]


def test_planner_automatic_refinement_worked_example():
    g = _gold("planner_auto_example.json")
    r = oracle.plan_auto(np.array(g["stats"]), g["nt"])
    assert r.reductions == g["reductions"]
    assert r.tol == pytest.approx(g["tol"], rel=1e-12)
    for i, row in enumerate(g["pmap_lower"]):
        assert r.pmap[i, :i + 1].tolist() == row
    assert r.eq10_pass and r.eq11_pass
    # one reduction fewer still fails Eq. 11
    r16 = oracle.plan(np.array(g["stats"]), g["nt"], 1e-4 * 0.9 ** 16)
    assert not r16.eq11_pass and r16.pmap[1, 0] == 2


def test_planner_automatic_refinement_stops_without_fp16():
    # a tile with a negative minimum fails Eq. 10 while it is FP16; the loop must run until the
    # tile leaves FP16: r = 1e-3/sqrt(200 + 2e-6) = 7.071e-5, r*2*2^-10 = 1.381e-7, so
    # 1e-4 * 0.9^k < 1.381e-7 first holds at k = 63
    st = np.array([[100.0, 0.5, 1.0], [1e-6, -1e-3, 1e-3], [100.0, 0.5, 1.0]])
    assert oracle.plan(st, 2, 1e-4).tiles[2] == 1
    r = oracle.plan_auto(st, 2)
    assert r.tiles[2] == 0 and r.reductions == 63
    assert oracle.plan(st, 2, r.tol / 0.9).tiles[2] == 1
    # no FP16 tile at the start: no reduction
    assert oracle.plan_auto(np.array([[100.0, 0.5, 1.0], [50.0, 0.2, 0.9], [100.0, 0.5, 1.0]]), 2).reductions == 0


def test_planner_edge_cases():
    st = np.array([[100.0, 0.5, 1.0], [50.0, 0.2, 0.9], [100.0, 0.5, 1.0]])
    r0 = oracle.plan(st, 2, 1e-8, amp=0)
    assert r0.s == 1.0 and r0.pmap[1, 0] == 0
    r1 = oracle.plan(st, 2, 1e-30)          # no reduced tile: cap applies, s = 65503
    assert r1.pmap[1, 0] == 0 and r1.s == 65503.0
    r2 = oracle.plan(st, 2, 1.0)            # everything allowed: FP16, u_16 = sqrt(65504/0.9)
    assert r2.pmap[1, 0] == 2
    assert r2.s == math.floor(math.sqrt(65504 / 0.9)) - 1
    assert not r2.eq11_pass                 # an FP16 tile as large as the diagonal fails Eq. 11
    r3 = oracle.plan(st, 2, 1.0, allow_fp16=False)
    assert r3.pmap[1, 0] == 1 and r3.s == 65503.0
    st_neg = st.copy(); st_neg[1, 1] = -1e-3
    assert not oracle.plan(st_neg, 2, 1.0).eq10_pass
    # smaller tolerance never lowers a tile's precision (monotonicity stated in Sec. V-D)
    rng = np.random.default_rng(0)
    nt = 6
    stv = np.abs(rng.standard_normal((nt * (nt + 1) // 2, 3))) * 10.0 ** rng.uniform(-12, 2, (nt * (nt + 1) // 2, 1))
    prev = None
    for tol in (1e-2, 1e-4, 1e-6, 1e-8, 1e-10):
        m = oracle.plan(stv, nt, tol).pmap
        if prev is not None:
            low = np.tril_indices(nt)
            assert np.all(m[low].astype(int) <= prev[low].astype(int))
        prev = m


# ---------------------------------------------------------------- synthetic inputs
def test_trend_contour_and_grid_centres():
    # Sec. VI-B: m(s) = 15x + 10y, the u = 10 contour is y = 1 - 1.5x; cell centres (2j+1)h/2
    xs = np.linspace(0, 0.66, 11)
    np.testing.assert_allclose(syn.trend_mean(xs, 1 - 1.5 * xs, (0, 15, 10)), 10.0, rtol=1e-14)
    x, y = syn.grid_centres(4)
    assert sorted(set(x.tolist())) == [0.125, 0.375, 0.625, 0.875]
    assert x[1] == 0.375 and y[1] == 0.125 and y[4] == 0.375
    p = syn.morton_order(np.array([0.9, 0.1, 0.6, 0.1]), np.array([0.9, 0.1, 0.1, 0.6]))
    assert p.tolist() == [1, 2, 3, 0]

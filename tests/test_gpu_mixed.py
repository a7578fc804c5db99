"""GPU checks of the mixed-precision path tile by tile, against the oracle's emulation.

"Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets", Sec. IV-B
(each tile stored and updated in its own precision), Algorithm 1 (FP16 copy of the factor, FP16
right-hand side, FP32 diagonal product, optional FP16 destination between k-tasks), Eq. 12 (scale).

Relative Frobenius error against the FP64 oracle cannot see the FP16 tiles (they hold a few 1e-6 of
||L||), so each precision class is checked on its own:
  * every stored value of an FP32 / FP16 tile is a binary32 / binary16 number (bitwise);
  * the FP16 copy the simulation product reads is binary16 rounding of the stored factor (bitwise);
  * every tile of L_s is within a per-precision bound of the emulated factorization (same storage
    rounding, FP32 accumulation inside reduced-precision tasks).  The bounds are about 15 times the
    spread between two emulations that differ only in their FP32 summation order, measured on these
    cases (FP64 tiles <= 6e-7, FP32 <= 8e-6, FP16 <= 1.1e-6): the cases are chosen well conditioned,
    since on ill-conditioned ones (e.g. range 0.03 at tol 1e-8 with the unscaled rule) that spread
    alone reaches 1e-3 in FP32 tiles and per-tile comparison means nothing there;
  * the simulation product is within 1e-4 of the emulated TRMM on the emulated factor.
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

TILE_TOL = {0: 1e-5, 1: 1e-4, 2: 2e-3}   # per-tile relative Frobenius bound vs the emulation


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
    return torch.tensor(np.ascontiguousarray(np.asarray(a).T), dtype=torch.float64, device="cuda:0").T


def locs(n, seed):
    x, y = syn.uniform_locations(n, seed)
    x, y, _ = syn.ordered_locations(x, y)
    return x, y


MIXED = [
    # (n, nb, nu, beta, seed, tol, tile-count-scaled rule): FP64, FP32 and FP16 tiles, ragged last tile
    (3200, 320, 1.5, 0.03, 1002, 1e-9, False),
    (3200, 320, 1.5, 0.03, 1002, 1e-7, True),
    (3100, 256, 0.5, 0.03, 3, 1e-8, True),
]


@pytest.mark.parametrize("case", MIXED, ids=lambda c: f"n{c[0]}_nb{c[1]}_tol{c[5]:g}_{'nt' if c[6] else 'plain'}")
def test_precision_classes_against_emulation(ctx, case):
    n, nb, nu, beta, seed, tol, nt_rule = case
    x, y = locs(n, seed)
    params = {"kind": 0, "sigma2": 1.0, "range": beta, "nu": nu, "nugget": 1e-4}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=tol, nt_rule=nt_rule)
    info = A.info()
    nt, s, pm = info["nt"], info["s"], info["map"]
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    r = oracle.plan(oracle.tile_stats(V, nb), nt, tol, nt_rule=nt_rule)
    low = np.tril_indices(nt)
    assert np.array_equal(pm[low], r.pmap[low]) and s == r.s
    assert A.diag["tiles"][1] > 0 and A.diag["tiles"][2] > 0, "case must hold FP32 and FP16 tiles"
    sl = lambda i: slice(i * nb, min((i + 1) * nb, n))   # noqa: E731
    # stored s^2 V: each reduced tile holds numbers of its precision within half an ulp of s^2 V
    # (the device and host exponentials may differ in the last bit of V, so no bitwise comparison)
    S0 = A.block_raw(0, 0, n, n).cpu().numpy()
    for i in range(nt):
        for j in range(i):
            t, p = S0[sl(i), sl(j)], int(pm[i, j])
            ref = s * s * V[sl(i), sl(j)]
            if p == 1:
                assert np.array_equal(t, t.astype(np.float32).astype(np.float64)), (i, j)
                assert np.all(np.abs(t - ref) <= (2.0 ** -24 * 1.0001 + 1e-12) * np.abs(ref)), (i, j)
            elif p == 2:
                assert np.array_equal(t, t.astype(np.float16).astype(np.float64)), (i, j)
                assert np.all(np.abs(t - ref) <= (2.0 ** -11 * 1.0001 + 1e-12) * np.abs(ref) + 2.0 ** -25), (i, j)
    assert g.potrf_mp(ctx, A) == 0 and A.potrf_status == g.OK
    Lg = A.block_raw(0, 0, n, n).cpu().numpy()             # L_s as stored
    L16 = A.block_raw(0, 0, n, n, fp16_copy=True).cpu().numpy()
    Le, ie = oracle.potrf_mp_emul(s * s * V, nb, r.pmap)
    assert ie == 0
    worst = {0: 0.0, 1: 0.0, 2: 0.0}
    for i in range(nt):
        for j in range(i + 1):
            p = 0 if i == j else int(pm[i, j])
            t = Lg[sl(i), sl(j)]
            if p == 1:
                assert np.array_equal(t, t.astype(np.float32).astype(np.float64)), ("not binary32", i, j)
            if p == 2:
                assert np.array_equal(t, t.astype(np.float16).astype(np.float64)), ("not binary16", i, j)
            if i > j:   # the FP16 copy of the off-diagonal factor is binary16 of the stored value
                assert np.array_equal(L16[sl(i), sl(j)], t.astype(np.float16).astype(np.float64)), ("l16", i, j)
            ref = Le[sl(i), sl(j)]
            nr = np.linalg.norm(ref)
            # a tile that underflows to zero in its precision must be zero on both sides
            e = float(np.linalg.norm(t - ref) / nr) if nr > 0 else float(np.linalg.norm(t))
            worst[p] = max(worst[p], e)
            assert e <= TILE_TOL[p], (i, j, p, e)
    print(f"map {A.diag['tiles']} s {s}: worst tile error vs emulation FP64 {worst[0]:.2e} FP32 {worst[1]:.2e} "
          f"FP16 {worst[2]:.2e}")
    # the simulation product against the emulated TRMM of the emulated factor
    nsim = 96
    Z = syn.explicit_normals(n, nsim, seed + 5)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    Me = oracle.trmm_mp_emul(Le, nb, s, Z, fp16_dest=False)
    em = rel(M.cpu().numpy(), Me)
    print(f"  M vs emulated TRMM {em:.2e}")
    assert em <= 1e-4
    A.close()


def test_fp16_destination_emulation(ctx):
    n, nb, nsim = 2000, 256, 128
    x, y = locs(n, 44)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5, "nugget": 1e-4}
    Z = syn.explicit_normals(n, nsim, 45)
    out = {}
    for emu in (False, True):
        A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-8, fp16_dest=emu)
        assert g.potrf_mp(ctx, A) == 0
        out[emu] = (g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))[0].cpu().numpy(), A.info()["s"], A.info()["map"])
        A.close()
    (M0, s, pm), (M1, _, _) = out[False], out[True]
    V = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 1.5, nugget=1e-4)
    Le, _ = oracle.potrf_mp_emul(s * s * V, nb, pm)
    Me0 = oracle.trmm_mp_emul(Le, nb, s, Z, fp16_dest=False)
    Me1 = oracle.trmm_mp_emul(Le, nb, s, Z, fp16_dest=True)
    assert np.array_equal(M1, M1.astype(np.float16).astype(np.float64)), "destination is not binary16"
    effect_o, effect_g = rel(Me1, Me0), rel(M1, M0)
    d1 = rel(M1, Me1)
    print(f"emulated destination: gpu vs oracle {d1:.2e}; effect of the FP16 destination gpu {effect_g:.2e} "
          f"oracle {effect_o:.2e}")
    assert 0.5 <= effect_g / effect_o <= 2.0
    assert d1 <= 0.25 * effect_o
    Lo, _ = oracle.potrf(V)
    assert rel(M1, oracle.trmm(Lo, Z)) <= 1e-2
    # the emulation needs whole 128-blocks per tile
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, 320, amp=1, tol=1e-8, fp16_dest=True)
    assert g.potrf_mp(ctx, A) == 0
    with pytest.raises(g.GpexError) as ei:
        g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    assert ei.value.code == g.ERR_ARG
    A.close()


def test_gaussian_kind_covariance_factor_and_kriging(ctx):
    n, nb, theta = 1100, 160, 0.01
    x, y = locs(n, 61)
    params = {"kind": 1, "sigma2": 1.3, "range": theta, "nu": 0.5, "nugget": 1e-3}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=0)
    V = oracle.cov_matrix(x, y, 1, 1.3, theta, 0.5, nugget=1e-3)
    Vg = A.to_dense().cpu().numpy()
    np.testing.assert_allclose(np.tril(Vg), np.tril(V), rtol=1e-13, atol=1e-300)
    st_g, st_o = A.stats(), oracle.tile_stats(V, nb)
    np.testing.assert_allclose(st_g[:, 0], st_o[:, 0], rtol=1e-12)
    np.testing.assert_allclose(st_g[:, 1:], st_o[:, 1:], rtol=1e-13)
    assert g.potrf_mp(ctx, A) == 0
    Lo, _ = oracle.potrf(V)
    assert rel(A.to_dense().cpu().numpy(), Lo) <= 1e-10
    A.close()
    # kriging with the Gaussian kernel, with and without the trend
    xo, yo = locs(700, 62)
    xp, yp = locs(333, 63)
    y_obs = syn.trend_mean(xo, yo, (0.5, 1.0, -1.0)) + np.random.default_rng(64).standard_normal(700)
    for k in (0, 3):
        W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), 700, dev(np.r_[xp, yp]), 333, dev(y_obs), k, params,
                                   0.01, 128)
        assert info == 0
        ro = oracle.krige(xo, yo, xp, yp, y_obs, k, 1, 1.3, theta, 0.5, 0.01)
        assert rel(W.cpu().numpy(), ro["W"]) <= 1e-9
        assert rel(zhat.cpu().numpy(), ro["zhat"]) <= 1e-9
        assert rel(v.cpu().numpy(), ro["v"]) <= 1e-9


def test_failed_factorization_is_unusable(ctx):
    n, nb = 300, 64
    x, y = syn.uniform_locations(n, 1)
    da = np.full(n, 1e-4)
    da[150] = -1.5
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 0.5, "nugget": 0.0},
                  nb, amp=0, diag_add=dev(da))
    assert g.potrf_mp(ctx, A) == 151
    for call in (lambda: g.potrf_mp(ctx, A), lambda: g.trmm_sim(ctx, A, 8), lambda: A.block(0, 0, 10, 10),
                 lambda: A.to_dense()):
        with pytest.raises(g.GpexError) as ei:
            call()
        assert ei.value.code == g.ERR_STATE
    A.close()


@pytest.mark.parametrize("sigma2", [4.0, 1e6])
def test_large_variance_keeps_fp16_factor_finite(ctx, sigma2):
    # without the bound the FP16 copy of L_s (entries up to s sqrt(sigma2)) would overflow
    n, nb, nsim = 1500, 256, 64
    x, y = locs(n, 71)
    params = {"kind": 0, "sigma2": sigma2, "range": 0.1, "nu": 1.5, "nugget": 1e-4 * sigma2}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-9)
    d = A.diag
    assert d["s"] <= d["u_factor"] and d["u_factor"] == pytest.approx(65504.0 / np.sqrt(sigma2 * 1.0001), rel=1e-12)
    assert g.potrf_mp(ctx, A) == 0 and A.potrf_status == g.OK and not A.diag["fp16_overflow"]
    L16 = A.block_raw(0, 0, n, n, fp16_copy=True).cpu().numpy()
    assert np.all(np.isfinite(L16))
    Z = syn.explicit_normals(n, nsim, 72)
    M, dg, st = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z), status=True)
    assert st == g.OK
    V = oracle.cov_matrix(x, y, 0, sigma2, 0.1, 1.5, nugget=1e-4 * sigma2)
    Lo, _ = oracle.potrf(V)
    assert rel(M.cpu().numpy(), oracle.trmm(Lo, Z)) <= 1e-2
    A.close()


def test_fp16_input_overflow_is_reported(ctx):
    n, nb, nsim = 700, 128, 8
    x, y = locs(n, 81)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5, "nugget": 1e-4}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=1e-8)
    assert g.potrf_mp(ctx, A) == 0
    Z = syn.explicit_normals(n, nsim, 82)
    Z[5, 3] = 1e12              # Z / s far beyond 65504
    M, d, st = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z), status=True)
    assert st == g.WARN_FP16_OVERFLOW and d["fp16_overflow"] == 1
    Z[5, 3] = 0.5               # an ordinary input clears it again
    M, d, st = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z), status=True)
    assert st == g.OK and d["fp16_overflow"] == 0
    A.close()

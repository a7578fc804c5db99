"""GPU parity of GEMM launches that split into a whole-block part and ragged strips.

A launch whose M or N is not a multiple of 128 and that holds at least 512 whole 128 x 128 blocks
runs the whole blocks on the vector path and the leftover strips, bounds-checked, on the context's
side stream.  These cases are sized so that launches split:
  * kriging (Sec. V-A, Eq. 5/6) with n_o = 2048 at tile 256: the first steps of both blocked
    triangular solves hold up to 7 tasks x 2 x 125 whole blocks (N = n_p = 16,033);
  * the conditioning product of Eq. 7 (M = n_p = 16,033, N = nsim = 1207: 125 x 9 whole blocks);
  * the mixed-precision factorization (Sec. IV-B) at n = 12,800, tile 320 (4 whole blocks per tile
    task), whose large trailing-update groups split with typed and run-time-typed strips.
Tolerances as in the other parity tests: FP64 relative Frobenius 1e-10, mixed-precision factor
5e-3 and simulated fields 1e-2.
"""
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
    return torch.tensor(np.ascontiguousarray(np.asarray(a).T), dtype=torch.float64, device="cuda:0").T


def test_split_kriging_solves_and_conditioning_product(ctx):
    n_o, n_p, nb, nsim, u, c = 2048, 16033, 256, 1207, 1.0, 0.9
    xo, yo = syn.uniform_locations(n_o, 31)
    xp, yp = syn.uniform_locations(n_p, 131)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    y_obs = syn.trend_mean(xo, yo, (0.5, 1.0, -1.0)) + np.random.default_rng(31).standard_normal(n_o)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    print(f"\nsplit kriging: n_o {n_o} n_p {n_p} nb {nb} nsim {nsim}", flush=True)
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), 3, params, 0.01,
                               nb)
    assert info == 0
    r = oracle.krige(xo, yo, xp, yp, y_obs, 3, 0, 1.0, 0.1, 1.5, 0.01)
    assert rel(W.cpu().numpy(), r["W"]) <= 1e-10
    assert rel(zhat.cpu().numpy(), r["zhat"]) <= 1e-10
    assert rel(v.cpu().numpy(), r["v"]) <= 1e-10
    # conditioning of an explicit field: S = M_p + W^T (y_o 1^T - M_o)
    M = syn.explicit_normals(n_p + n_o, nsim, 2031)
    out = g.excursion_regions(ctx, dev_cm(M), n_p, n_o, nsim, u, c, W=W, y_o=dev(y_obs), zhat=zhat, v=v,
                              want_S=True)
    assert out["status"] == 0
    So = oracle.condition(M, n_p, r["W"], y_obs)
    assert rel(out["S"].cpu().numpy(), So) <= 1e-10


def test_split_mixed_precision_updates(ctx):
    n, nb, nu, beta, seed, tol = 12800, 320, 1.5, 0.03, 1002, 1e-9
    x, y = syn.uniform_locations(n, seed)
    x, y, _ = syn.ordered_locations(x, y)
    params = {"kind": 0, "sigma2": 1.0, "range": beta, "nu": nu, "nugget": 1e-4}
    A = g.cov_gen(ctx, dev(np.r_[x, y]), n, params, nb, amp=1, tol=tol, nt_rule=False)
    print(f"\nsplit mixed precision: n {n} nb {nb} tiles {A.diag['tiles']}", flush=True)
    assert A.diag["tiles"][1] > 0 and A.diag["tiles"][2] > 0, "case must exercise FP32 and FP16 tiles"
    assert g.potrf_mp(ctx, A) == 0
    L = A.to_dense().cpu().numpy()
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    Lo, _ = oracle.potrf(V)
    del V
    ef = rel(L, Lo)
    del L
    nsim = 64
    Z = syn.explicit_normals(n, nsim, seed + 1)
    M, _ = g.trmm_sim(ctx, A, nsim, Z=dev_cm(Z))
    em = rel(M.cpu().numpy(), oracle.trmm(Lo, Z))
    print(f"factor {ef:.3e} M {em:.3e}", flush=True)
    assert ef <= 5e-3
    assert em <= 1e-2
    A.close()

"""The concurrent schedule gives bitwise the results of the serial one.

The factorization runs a look-ahead of depth one on two streams, and large GEMM launches whose M
or N is ragged run their whole blocks and their edge strips on two streams ("Mixed-Precision GPU
Acceleration for Confidence Regions of Spatial Excursion Sets", Sec. IV-C: task dependencies, not
a global order, protect the data; here events do).  gpex_ctx_set_serial puts every launch on the
context stream in program order.  Each tile then receives the same operations in the same order
from the same kernels, so any difference would come from a missing dependency (a race).

Cases: the mixed-precision factorization at n = 12,800, tile 320 (FP32 and FP16 tiles; every tile
task is ragged, large update launches split into whole blocks and strips), an FP64 factorization
at tile 1024 with a padded last tile, and the kriging solves and conditioning product at
n_o = 2,048, n_p = 16,033 (split launches).  Compared bitwise on the device: the stored factor,
its FP16 copy, the simulations, W, zhat, v, S and the counts.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import gpex_synth as syn

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import gp_conditional_simulation_amd as g  # noqa: E402


def dev(a):
    return torch.tensor(np.ascontiguousarray(a), dtype=torch.float64, device="cuda:0")


def dev_cm(a):
    return torch.tensor(np.ascontiguousarray(np.asarray(a).T), dtype=torch.float64, device="cuda:0").T


def same(a, b):
    return a.shape == b.shape and bool(torch.equal(a, b))


def _factor_and_simulate(ctx, serial, loc, n, nb, params, amp, tol, nt_rule, Z, nsim):
    ctx.set_serial(serial)
    try:
        A = g.cov_gen(ctx, loc, n, params, nb, amp=amp, tol=tol, nt_rule=nt_rule)
        assert g.potrf_mp(ctx, A) == 0
        L = A.block_raw(0, 0, n, n)
        L16 = A.block_raw(0, 0, n, n, fp16_copy=True) if amp else None
        M, _ = g.trmm_sim(ctx, A, nsim, Z=Z)
        tiles = A.diag["tiles"]
        A.close()
    finally:
        ctx.set_serial(False)
    return L, L16, M, tiles


@pytest.mark.parametrize("case", [
    # (n, nb, nu, beta, seed, amp, tol, tile-count-scaled rule)
    (12800, 320, 1.5, 0.03, 1002, 1, 1e-9, False),
    (6000, 1024, 1.5, 0.1, 1005, 0, 0.0, True),
    (6000, 1024, 1.5, 0.03, 1005, 1, 1e-6, True),
], ids=["mixed_n12800_nb320", "fp64_n6000_nb1024", "mixed_n6000_nb1024"])
def test_factor_and_simulation_bitwise_serial(case):
    n, nb, nu, beta, seed, amp, tol, nt_rule = case
    ctx = g.Context(0)
    x, y = syn.uniform_locations(n, seed)
    x, y, _ = syn.ordered_locations(x, y)
    loc = dev(np.r_[x, y])
    params = {"kind": 0, "sigma2": 1.0, "range": beta, "nu": nu, "nugget": 1e-4}
    nsim = 256
    Z = dev_cm(syn.explicit_normals(n, nsim, seed + 9))
    Lc, L16c, Mc, tiles = _factor_and_simulate(ctx, False, loc, n, nb, params, amp, tol, nt_rule, Z, nsim)
    Ls, L16s, Ms, _ = _factor_and_simulate(ctx, True, loc, n, nb, params, amp, tol, nt_rule, Z, nsim)
    print(f"n {n} nb {nb} tiles {tiles}", flush=True)
    if amp and nb == 320:
        assert tiles[1] > 0 and tiles[2] > 0
    assert same(Lc, Ls), "factor differs between the concurrent and the serial schedule"
    if amp:
        assert same(L16c, L16s)
    assert same(Mc, Ms)
    ctx.close()


def test_kriging_and_conditioning_bitwise_serial():
    n_o, n_p, nb, nsim, u, c = 2048, 16033, 256, 1207, 1.0, 0.9
    xo, yo = syn.uniform_locations(n_o, 31)
    xp, yp = syn.uniform_locations(n_p, 131)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    y_obs = dev(syn.trend_mean(xo, yo, (0.5, 1.0, -1.0)) + np.random.default_rng(31).standard_normal(n_o))
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    M = dev_cm(syn.explicit_normals(n_p + n_o, nsim, 2031))
    ctx = g.Context(0)
    res = {}
    for serial in (False, True):
        ctx.set_serial(serial)
        W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, y_obs, 3, params, 0.01, nb)
        assert info == 0
        out = g.excursion_regions(ctx, M, n_p, n_o, nsim, u, c, W=W, y_o=y_obs, zhat=zhat, v=v, want_S=True)
        assert out["status"] == 0
        res[serial] = (W.clone(), zhat.clone(), v.clone(), out["S"].clone(), out["counts"].clone(),
                       out["cin"].clone(), out["cout"].clone())
    ctx.set_serial(False)
    for a, b in zip(res[False], res[True]):
        assert same(a, b)
    ctx.close()

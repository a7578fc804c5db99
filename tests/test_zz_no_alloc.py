"""The allocation-free scan entry point against the allocating one, through the C ABI.

gpex_excursion_regions_noalloc keeps its temporaries in the library's fixed per-GPU scratch array
and evaluates Eq. 7 ("Mixed-Precision GPU Acceleration for Confidence Regions of Spatial
Excursion Sets", Sec. V-B) without the residual matrix.  Two calls in a row on one context, the
second smaller (the array keeps the first call's contents), each compared with
gpex_excursion_regions on the same inputs: S within 1e-10 relative Frobenius, counts, sizes,
psi, phi, regions and quantiles equal (no entry of S lies within 1e-9 of u in these cases, which
is checked).  A request beyond the array's size is rejected.
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


def _inputs(ctx, n_p, n_o, nsim, seed):
    xo, yo = syn.uniform_locations(n_o, seed)
    xp, yp = syn.uniform_locations(n_p, seed + 1)
    xo, yo, _ = syn.ordered_locations(xo, yo)
    xp, yp, _ = syn.ordered_locations(xp, yp)
    y_obs = syn.trend_mean(xo, yo, (0.5, 1.0, -1.0)) + np.random.default_rng(seed).standard_normal(n_o)
    params = {"kind": 0, "sigma2": 1.0, "range": 0.1, "nu": 1.5}
    W, zhat, v, info = g.krige(ctx, dev(np.r_[xo, yo]), n_o, dev(np.r_[xp, yp]), n_p, dev(y_obs), 3, params, 0.01, 256)
    assert info == 0
    M = dev_cm(syn.explicit_normals(n_p + n_o, nsim, seed + 2))
    return M, W, dev(y_obs), zhat, v


def _compare(ctx, n_p, n_o, nsim, seed, regions):
    M, W, y_o, zhat, v = _inputs(ctx, n_p, n_o, nsim, seed) if n_o else (dev_cm(syn.explicit_normals(n_p, nsim, seed)),
                                                                        None, None, None, None)
    kw = dict(W=W, y_o=y_o, zhat=zhat if regions else None, v=v if regions else None, want_S=True)
    ref = g.excursion_regions(ctx, M, n_p, n_o, nsim, 1.0, 0.9, **kw)
    got = g.excursion_regions(ctx, M, n_p, n_o, nsim, 1.0, 0.9, noalloc=True, **kw)
    S_ref, S_got = ref["S"].cpu().numpy(), got["S"].cpu().numpy()
    assert np.linalg.norm(S_got - S_ref) <= 1e-10 * np.linalg.norm(S_ref)
    assert not np.any(np.abs(S_ref - 1.0) < 1e-9), "near-tie: integer outputs may differ legitimately"
    assert got["status"] == ref["status"]
    for k in ("counts", "sizes") + (("cin", "cout") if regions else ()):
        assert torch.equal(got[k], ref[k]), k
    if regions:
        assert np.array_equal(got["psi"], ref["psi"]) and np.array_equal(got["phi"], ref["phi"])
        assert (got["q_in"], got["q_out"], got["n_psi"], got["n_phi"]) == \
               (ref["q_in"], ref["q_out"], ref["n_psi"], ref["n_phi"])


def test_noalloc_matches_allocating_entry_point_twice():
    ctx = g.Context(0)
    _compare(ctx, 6000, 1500, 900, 101, regions=True)     # conditioned, regions
    _compare(ctx, 1200, 300, 130, 202, regions=True)      # second call, smaller
    _compare(ctx, 2000, 0, 64, 303, regions=False)        # unconditional counts only, smaller again
    torch.cuda.synchronize()
    ctx.close()


def test_noalloc_rejects_requests_beyond_the_scratch():
    ctx = g.Context(0)
    n_p, nsim = 5_000_000, 2     # t alone needs 40 MB
    M = torch.zeros((nsim, n_p), dtype=torch.float64, device="cuda:0").T
    with pytest.raises(g.GpexError) as ei:
        g.excursion_regions(ctx, M, n_p, 0, nsim, 1.0, 0.9, noalloc=True)
    assert ei.value.code == g.ERR_ARG
    ctx.close()

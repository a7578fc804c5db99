"""Seeded synthetic inputs shared by the oracle-side tests, the HIP path's tests and the benchmark.

This module holds none of the excursion-set method's arithmetic: it only draws locations,
orders them, builds trend designs and plain random inputs, and records the workload
parameters.  Recipes follow the synthetic-data section (VI-B) of "Mixed-Precision GPU
Acceleration for Confidence Regions of Spatial Excursion Sets": observation locations uniform
on [0,1]^2 from a fixed seed, prediction locations at cell centres of an m x m grid, prediction
rows ordered first, trend design X(s) = (1, x, y).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "grid_centres", "uniform_locations", "morton_order",
    "ordered_locations", "design_matrix", "explicit_normals", "trend_mean",
]

MORTON_BITS = 21


def grid_centres(m: int) -> tuple[np.ndarray, np.ndarray]:
    """Cell centres ((2j+1)h/2, (2i+1)h/2), h = 1/m, i, j = 0..m-1 (section VI-B).

    Returned in row-major order over (i, j): index i*m + j has x from j and y from i."""
    h = 1.0 / m
    c = (2.0 * np.arange(m) + 1.0) * h / 2.0
    yy, xx = np.meshgrid(c, c, indexing="ij")
    return xx.reshape(-1).copy(), yy.reshape(-1).copy()


def uniform_locations(n: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """n locations i.i.d. uniform on [0,1]^2 from numpy's PCG64 stream with the given seed."""
    rng = np.random.default_rng(seed)
    xy = rng.random((n, 2))
    return xy[:, 0].copy(), xy[:, 1].copy()


def _spread_bits(q: np.ndarray) -> np.ndarray:
    out = np.zeros(q.shape, dtype=np.uint64)
    q = q.astype(np.uint64)
    for b in range(MORTON_BITS):
        out |= ((q >> np.uint64(b)) & np.uint64(1)) << np.uint64(2 * b)
    return out


def morton_order(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Stable permutation sorting locations by their Z-order (Morton) code.

    Each coordinate in [0,1] is quantised to 21 bits; x takes the even bit positions and y the
    odd ones.  Ties keep the original index order.  The pages only state the premise that tiles
    near the diagonal hold strongly correlated locations; this ordering realises it."""
    top = (1 << MORTON_BITS) - 1
    qx = np.clip(np.floor(np.asarray(x) * (1 << MORTON_BITS)), 0, top).astype(np.int64)
    qy = np.clip(np.floor(np.asarray(y) * (1 << MORTON_BITS)), 0, top).astype(np.int64)
    code = _spread_bits(qx) | (_spread_bits(qy) << np.uint64(1))
    return np.argsort(code, kind="stable")


def ordered_locations(x: np.ndarray, y: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Apply the Morton permutation; returns (x, y, perm) with x_new = x[perm]."""
    p = morton_order(x, y)
    return x[p].copy(), y[p].copy(), p


def design_matrix(x: np.ndarray, y: np.ndarray, k: int = 3) -> np.ndarray:
    """Trend design with rows X(s) = (1, x, y) (k = 3) or an empty design (k = 0); shape (n, k)."""
    n = len(x)
    if k == 0:
        return np.zeros((n, 0))
    if k != 3:
        raise ValueError("k must be 0 or 3")
    return np.stack([np.ones(n), np.asarray(x, float), np.asarray(y, float)], axis=1)


def trend_mean(x: np.ndarray, y: np.ndarray, beta) -> np.ndarray:
    """Deterministic mean m(s) = X(s)^T b for the (1, x, y) design."""
    return design_matrix(x, y, 3) @ np.asarray(beta, dtype=float)


def explicit_normals(n: int, nsim: int, seed: int) -> np.ndarray:
    """An n x nsim standard-normal matrix (Fortran order) from numpy's generator.

    Used as the explicit random input that both sides receive, so that parity does not depend on
    either side's transcendental functions."""
    rng = np.random.default_rng(seed)
    return np.asfortranarray(rng.standard_normal((n, nsim)))


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.  kind: 0 Matern (half-integer nu), 1 Gaussian."""
    name: str
    n: int
    nb: int
    nu: float
    sigma2: float
    beta: float
    nugget: float
    nsim: int
    seed_sim: int
    u: float
    amp: int
    tol: float
    kind: int = 0
    grid_m: int = 0          # > 0: regular grid of grid_m^2 cell centres
    seed_loc: int = 0
    # universal kriging workload (n_obs > 0): n = n_pred + n_obs, prediction rows first
    n_obs: int = 0
    seed_obs: int = 0
    tau2: float = 0.0
    trend: tuple = ()
    level: float = 0.9

    @property
    def n_pred(self) -> int:
        return self.n - self.n_obs

    def locations(self) -> tuple[np.ndarray, np.ndarray]:
        """Ordered locations; for kriging workloads prediction block first, each block Morton-sorted."""
        if self.n_obs:
            xp, yp = uniform_locations(self.n_pred, self.seed_loc)
            xo, yo = uniform_locations(self.n_obs, self.seed_obs)
            xp, yp, _ = ordered_locations(xp, yp)
            xo, yo, _ = ordered_locations(xo, yo)
            return np.concatenate([xp, xo]), np.concatenate([yp, yo])
        if self.grid_m:
            x, y = grid_centres(self.grid_m)
        else:
            x, y = uniform_locations(self.n, self.seed_loc)
        x, y, _ = ordered_locations(x, y)
        return x, y

    def scaled(self, n: int, nsim: Optional[int] = None, nb: Optional[int] = None) -> "Workload":
        """Same recipe at a smaller size (for parity tests the oracle finishes in seconds)."""
        kw = dataclasses.asdict(self)
        kw.update(name=f"{self.name}@n{n}", n=n, grid_m=0)
        if nsim is not None:
            kw["nsim"] = nsim
        if nb is not None:
            kw["nb"] = nb
        if self.n_obs:
            kw["n_obs"] = n // 2
        return Workload(**kw)


WORKLOADS = {
    # N = 1,600 on a 40 x 40 grid, exponential covariance, all-FP64, 100 columns, u = 0.5
    "grid1600_fp64": Workload("grid1600_fp64", n=1600, nb=160, nu=0.5, sigma2=1.0, beta=0.1, nugget=1e-4,
                              nsim=100, seed_sim=2001, u=0.5, amp=0, tol=0.0, grid_m=40),
    # N = 10,000 uniform, Matern 3/2 at three ranges, tile 320, tolerance 1e-9, 500 columns
    **{f"unif10k_b{b}": Workload(f"unif10k_b{b}", n=10000, nb=320, nu=1.5, sigma2=1.0, beta=b, nugget=1e-4,
                                 nsim=500, seed_sim=2002, u=0.5, amp=1, tol=1e-9, seed_loc=1002)
       for b in (0.03, 0.1, 0.3)},
    # N = 40,000 uniform, Matern 5/2, tile 512, tolerances 1e-8 and 1e-6, 1,000 columns
    "unif40k_tol1e-8": Workload("unif40k_tol1e-8", n=40000, nb=512, nu=2.5, sigma2=1.0, beta=0.1, nugget=1e-4,
                                nsim=1000, seed_sim=2003, u=0.5, amp=1, tol=1e-8, seed_loc=1003),
    "unif40k_tol1e-6": Workload("unif40k_tol1e-6", n=40000, nb=512, nu=2.5, sigma2=1.0, beta=0.1, nugget=1e-4,
                                nsim=1000, seed_sim=2003, u=0.5, amp=1, tol=1e-6, seed_loc=1003),
    # universal kriging: 20,000 prediction + 20,000 observation locations, Matern 3/2, trend (0.5, 1, -1)
    "krige20k": Workload("krige20k", n=40000, nb=512, nu=1.5, sigma2=1.0, beta=0.1, nugget=0.0,
                         nsim=1000, seed_sim=2004, u=1.0, amp=0, tol=1e-8, seed_loc=1104,
                         n_obs=20000, seed_obs=1004, tau2=0.01, trend=(0.5, 1.0, -1.0), level=0.9),
    # N = 100,000 uniform, Matern 3/2, range 0.3, tile 1024, tolerance 1e-8, 2,000 columns
    "unif100k_tol1e-8": Workload("unif100k_tol1e-8", n=100000, nb=1024, nu=1.5, sigma2=1.0, beta=0.3,
                                 nugget=1e-4, nsim=2000, seed_sim=2005, u=0.5, amp=1, tol=1e-8, seed_loc=1005),
    # the same locations and tolerance at medium and weak correlation, where the map holds reduced
    # tiles: range 0.1 gives FP64 and FP32 tiles, range 0.03 FP64, FP32 and FP16 tiles
    **{f"unif100k_b{b}_tol1e-8": Workload(f"unif100k_b{b}_tol1e-8", n=100000, nb=1024, nu=1.5, sigma2=1.0, beta=b,
                                          nugget=1e-4, nsim=2000, seed_sim=2005, u=0.5, amp=1, tol=1e-8,
                                          seed_loc=1005)
       for b in (0.1, 0.03)},
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]

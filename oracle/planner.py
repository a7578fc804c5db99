"""Oracle-side precision plan (TEST INFRASTRUCTURE ONLY).

Follows "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets":
  Sec. IV-B   diagonal tiles stay FP64, off-diagonal tiles may use FP32 or FP16;
  Sec. V-D    the rule compares each tile's Frobenius norm with the global matrix norm, a
              smaller fixedacc keeps more tiles at high precision; Eq. 10 (FP16 representability
              range, strict <) and Eq. 11 (relative magnitude of the FP16 tiles);
  Sec. V-E    Eq. 12 covariance scale s.

Readings where the pages leave a step open:
  * rule: tile (i, j), i > j, with r = ||V_ij||_F / ||V||_F and NT tile rows goes to FP16 when
    FP16 is allowed and r * NT * 2^-10 <= tol, else to FP32 when r * NT * 2^-23 <= tol, else FP64
    (``nt_rule=False`` drops the NT factor);
  * Eq. 11 is read as max(rho1, rho2) < 1e-4 / eps_FP16 with eps_FP16 = 2^-10 (the extraction
    prints the fraction's numerator first, as it does for Eq. 10);
  * Eq. 10 with no FP16 tiles passes vacuously; with a non-positive FP16 minimum it fails;
  * Eq. 12 with no reduced-precision tile present gives u_s = 65504 and s = 65503;
  * the FP16 cast of L_s in Algorithm 1 adds u_L = 65504 / sqrt(max_i V_ii) to the minimum that
    defines u_s (|(L_s)_ij| <= s sqrt(V_ii)); it binds only when max_i V_ii > 1.
||V||_F^2 is summed over tiles in row-packed order t = i(i+1)/2 + j, off-diagonal tiles twice.

Precision codes: 0 = FP64, 1 = FP32, 2 = FP16 (255 above the diagonal).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

FP64, FP32, FP16 = 0, 1, 2
EPS = {FP32: 2.0 ** -23, FP16: 2.0 ** -10}
X_MAX = {FP32: (2.0 - 2.0 ** -23) * 2.0 ** 127, FP16: 65504.0}
X_MIN_NORM = {FP32: 2.0 ** -126, FP16: 2.0 ** -14}
X_MIN_SUB = {FP32: 2.0 ** -149, FP16: 2.0 ** -24}
EQ10_LIMIT = 65504.0 / 2.0 ** -24          # printed as "approximately 1.10 x 10^12"
EQ11_LIMIT = 1e-4 / 2.0 ** -10


AUTO_START = 1e-4        # Sec. V-D: automatic mode starts at fixedacc = 10^-4 ...
AUTO_FACTOR = 0.9        # ... and multiplies it by 0.9 whenever a check fails
AUTO_MAX = 2000          # guard: a tile with zero norm would stay FP16 at every tolerance


@dataclasses.dataclass
class PlanResult:
    pmap: np.ndarray            # uint8 [NT, NT]
    s: float
    frob: float
    l_bound: float
    u_bound: float
    lower_exceeds_upper: bool
    l_bound_sub: float
    r_hp: float
    rho1: float
    rho2: float
    eq10_pass: bool
    eq11_pass: bool
    tiles: tuple                # (n FP64, n FP32, n FP16) over the lower triangle
    tol: float = 0.0            # tolerance of this map (the final one in automatic mode)
    reductions: int = 0         # automatic mode: number of 0.9 reductions
    u_factor: float = float("inf")   # bound on s from the FP16 cast of L_s


def plan_auto(stats: np.ndarray, nt: int, allow_fp16: bool = True, nt_rule: bool = True) -> PlanResult:
    """Automatic fixedacc refinement (Sec. V-D): start at 1e-4, multiply by 0.9 while Eq. 10 or
    Eq. 11 fails, stop when both pass or no FP16 tile remains."""
    tol = AUTO_START
    k = 0
    while True:
        r = plan(stats, nt, tol, amp=1, allow_fp16=allow_fp16, nt_rule=nt_rule)
        if (r.eq10_pass and r.eq11_pass) or r.tiles[2] == 0 or k >= AUTO_MAX:
            r.tol, r.reductions = tol, k
            return r
        tol *= AUTO_FACTOR
        k += 1


def plan(stats: np.ndarray, nt: int, tol: float, amp: int = 1, allow_fp16: bool = True,
         nt_rule: bool = True) -> PlanResult:
    stats = np.asarray(stats, dtype=np.float64).reshape(-1, 3)
    assert stats.shape[0] == nt * (nt + 1) // 2
    pmap = np.full((nt, nt), 255, dtype=np.uint8)
    frob2 = 0.0
    for i in range(nt):
        for j in range(i + 1):
            ss = float(stats[i * (i + 1) // 2 + j, 0])
            frob2 += ss if i == j else 2.0 * ss
    frob = math.sqrt(frob2)
    mult = float(nt) if nt_rule else 1.0
    for i in range(nt):
        for j in range(i + 1):
            p = FP64
            if amp and i != j:
                r = math.sqrt(float(stats[i * (i + 1) // 2 + j, 0])) / frob
                if allow_fp16 and r * mult * EPS[FP16] <= tol:
                    p = FP16
                elif r * mult * EPS[FP32] <= tol:
                    p = FP32
            pmap[i, j] = p
    lower = [(i, j) for i in range(nt) for j in range(i + 1)]
    counts = tuple(sum(1 for (i, j) in lower if pmap[i, j] == p) for p in (FP64, FP32, FP16))
    if not amp:
        return PlanResult(pmap, 1.0, frob, 0.0, 1.0, False, 0.0, float("nan"), 0.0, 0.0, True, True, counts, tol)

    def st(i, j):
        return stats[i * (i + 1) // 2 + j]

    hp = [(i, j) for (i, j) in lower if pmap[i, j] == FP16]
    vmax_all = max(float(st(i, j)[2]) for (i, j) in lower)
    norm_all = max(math.sqrt(float(st(i, j)[0])) for (i, j) in lower)
    if hp:
        vmax_hp = max(float(st(i, j)[2]) for (i, j) in hp)
        vmin_hp = min(float(st(i, j)[1]) for (i, j) in hp)
        if vmin_hp > 0.0:
            r_hp = vmax_hp / vmin_hp
            eq10 = r_hp < EQ10_LIMIT
        else:
            r_hp = float("inf")
            eq10 = False
        rho1 = vmax_hp / vmax_all
        rho2 = max(math.sqrt(float(st(i, j)[0])) for (i, j) in hp) / norm_all
        eq11 = max(rho1, rho2) < EQ11_LIMIT
    else:
        r_hp, rho1, rho2, eq10, eq11 = float("nan"), 0.0, 0.0, True, True
    # Eq. 12 over the reduced formats present
    l_b, l_sub, u_min = 0.0, 0.0, float("inf")
    for f in (FP32, FP16):
        tiles_f = [(i, j) for (i, j) in lower if pmap[i, j] == f]
        if not tiles_f:
            continue
        vmin_f = min(float(st(i, j)[1]) for (i, j) in tiles_f)
        vmax_f = max(float(st(i, j)[2]) for (i, j) in tiles_f)
        lf = math.sqrt(X_MIN_NORM[f] / vmin_f) if vmin_f > 0.0 else float("inf")
        lsf = math.sqrt(X_MIN_SUB[f] / vmin_f) if vmin_f > 0.0 else float("inf")
        uf = math.sqrt(X_MAX[f] / vmax_f) if vmax_f > 0.0 else float("inf")
        l_b = max(l_b, lf)
        l_sub = max(l_sub, lsf)
        u_min = min(u_min, uf)
    # Algorithm 1 casts the scaled factor L_s to FP16 and every entry obeys |(L_s)_ij| <= s sqrt(V_ii)
    # (row i of L_s has squared norm s^2 V_ii), so s <= x_max,FP16 / sqrt(max_i V_ii) keeps it finite.
    vmax_diag = max(float(st(i, i)[2]) for i in range(nt))
    u_factor = X_MAX[FP16] / math.sqrt(vmax_diag) if vmax_diag > 0.0 else float("inf")
    u_s = min(65504.0, u_min, u_factor)
    s_cand = math.floor(u_s) - 1.0
    s = s_cand if s_cand > 1.0 else 1.0
    return PlanResult(pmap, s, frob, l_b, u_s, l_b > u_s, l_sub, r_hp, rho1, rho2, eq10, eq11, counts, tol,
                      u_factor=u_factor)

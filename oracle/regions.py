"""Oracle-side calibration of the inner and outer regions (TEST INFRASTRUCTURE ONLY).

"Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets",
Sec. V-C: the psi and phi samples are sorted separately with empty-set sentinels dropped,
the empirical quantile is Q_p(a) = a_(max{1, min{N, ceil(pN)}}) (Eq. 9), q_out = Q_alpha(psi),
q_in = Q_{1-alpha}(phi), C_out = {t >= q_out} (non-strict), C_in = {t > q_in} (strict), and both
samples must be non-empty.

Reading: p is taken as a decimal with at most six places, P = round(p * 10^6), and
ceil(pN) = ceil(P * N / 10^6) is evaluated in exact integers.
"""
from __future__ import annotations

import numpy as np


class EmptySample(ValueError):
    pass


def quantile_index(p: float, n: int) -> int:
    """1-based order-statistic index of Eq. 9 for a sample of size n >= 1."""
    if n < 1:
        raise EmptySample("empty sample")
    P = int(round(p * 1_000_000))
    k = -((-P * n) // 1_000_000)          # exact integer ceil(P n / 10^6)
    return max(1, min(n, k))


def empirical_quantile(a, p: float) -> float:
    a = np.sort(np.asarray(a, dtype=np.float64))
    return float(a[quantile_index(p, len(a)) - 1])


def calibrate(psi, phi, t, level: float):
    """Returns dict q_out, q_in, n_psi, n_phi, cout (uint8), cin (uint8)."""
    psi = np.asarray(psi, dtype=np.float64)
    phi = np.asarray(phi, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    a_psi = psi[psi != np.inf]
    a_phi = phi[phi != -np.inf]
    if len(a_psi) == 0 or len(a_phi) == 0:
        raise EmptySample("psi or phi sample is empty")
    alpha = round(1.0 - level, 6)
    q_out = empirical_quantile(a_psi, alpha)
    q_in = empirical_quantile(a_phi, round(1.0 - alpha, 6))
    return {
        "q_out": q_out, "q_in": q_in, "n_psi": len(a_psi), "n_phi": len(a_phi),
        "cout": (t >= q_out).astype(np.uint8), "cin": (t > q_in).astype(np.uint8),
    }

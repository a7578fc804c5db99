"""CPU FP64 oracle for the spatial excursion-set hot path (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  It shares no code with the HIP library ``gp_conditional_simulation_amd``
and neither imports the other.

Sources (by page title and section):
  "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets":
  Sec. III (Eq. 1-2), Sec. IV-C (Eq. 3), Sec. V-A..V-E (Eq. 4-12), Algorithm 2.
  "Massively parallel approximate Gaussian process regression": GP predictive equations
  (Eq. 1-2) and the isotropic Gaussian correlation.

The numeric kernels live in ``gpex_oracle.c`` (plain C loops in FP64); the host-side steps
(precision plan, empirical quantiles, regions) are plain Python in ``planner.py`` and
``regions.py``.  Every function is pinned by the CPU tests; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build
from .planner import plan, plan_auto, PlanResult  # noqa: F401
from .regions import empirical_quantile, quantile_index, calibrate  # noqa: F401

_lib = None
_d = np.ctypeslib.ndpointer(dtype=np.float64, flags="F_CONTIGUOUS")
_dv = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64 = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i32 = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_u32 = np.ctypeslib.ndpointer(dtype=np.uint32, flags="C_CONTIGUOUS")
_u8 = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")


def lib():
    """Load (building with gcc when missing) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(_build.LIB)
        I64, D, I = C.c_int64, C.c_double, C.c_int
        L.orc_num_threads.restype = I
        L.orc_cov.restype = D
        L.orc_cov.argtypes = [I, D, D, D, D]
        L.orc_cov_matrix.argtypes = [_dv, _dv, I64, I, D, D, D, D, C.c_void_p, _d, I64]
        L.orc_cov_cross.argtypes = [_dv, _dv, I64, _dv, _dv, I64, I, D, D, D, _d, I64]
        L.orc_tile_stats.argtypes = [_d, I64, I64, I64, _dv]
        L.orc_potrf.restype = I64
        L.orc_potrf.argtypes = [_d, I64, I64]
        L.orc_trmm.argtypes = [_d, I64, I64, _d, I64, I64, _d, I64]
        L.orc_trsm_lower.argtypes = [_d, I64, I64, _d, I64, I64]
        L.orc_trsm_lower_trans.argtypes = [_d, I64, I64, _d, I64, I64]
        L.orc_gemm.argtypes = [I, I, I64, I64, I64, D, _d, I64, _d, I64, D, _d, I64]
        L.orc_krige.restype = I64
        L.orc_krige_mats.restype = I64
        L.orc_krige_mats.argtypes = [_d, _d, _dv, _dv, I64, _dv, _dv, I64, _dv, I, D, _d, _dv, _dv, C.c_void_p]
        L.orc_krige.argtypes = [_dv, _dv, I64, _dv, _dv, I64, _dv, I, I, D, D, D, D, _d, _dv, _dv, C.c_void_p]
        L.orc_condition.argtypes = [_d, I64, I64, I64, I64, _d, _dv, _d, I64]
        L.orc_scan.argtypes = [_d, I64, I64, I64, C.c_void_p, D, _i64, _i32, C.c_void_p, C.c_void_p]
        L.orc_philox4x32_10.argtypes = [_u32, _u32, _u32]
        L.orc_normals.argtypes = [C.c_uint64, C.c_uint32, I64, I64, I64, I64, I64, _d, I64]
        L.orc_round_fp16.restype = D
        L.orc_round_fp16.argtypes = [D]
        L.orc_potrf_mp_emul.restype = I64
        L.orc_potrf_mp_emul.argtypes = [_d, I64, I64, I64, _u8]
        L.orc_trmm_mp_emul.argtypes = [_d, I64, I64, I64, D, _d, I64, I64, I, _d, I64]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _f(a):
    return np.asfortranarray(a, dtype=np.float64)


def _c(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _half_integer(kind, nu) -> bool:
    return kind != 0 or nu in (0.5, 1.5, 2.5)


def matern_correlation(r, nu) -> np.ndarray:
    """Matern correlation of any order nu ("Mixed-Precision GPU Acceleration for Confidence Regions
    of Spatial Excursion Sets", Sec. V-E): 2^(1 - nu) / Gamma(nu) r^nu K_nu(r), 1 at r = 0, with
    scipy's exponentially scaled K_nu (kve) and log-gamma as the library primitives:
    exp((1 - nu) ln 2 - ln Gamma(nu) + nu ln r - r) kve(nu, r)."""
    from scipy.special import gammaln, kve
    r = np.asarray(r, dtype=np.float64)
    out = np.ones_like(r)
    pos = r > 0
    rp = r[pos]
    out[pos] = np.exp((1.0 - nu) * np.log(2.0) - gammaln(nu) + nu * np.log(rp) - rp) * kve(nu, rp)
    return out


def _general(d, sigma2, rng, nu):
    return sigma2 * matern_correlation(np.asarray(d) / rng, nu)


def cov(kind: int, sigma2: float, rng: float, nu: float, d: float) -> float:
    """One covariance value (Matern with kind 0: half-integer nu in closed form in C, any other nu
    by matern_correlation; Gaussian with kind 1)."""
    if not _half_integer(kind, nu):
        return float(_general(d, sigma2, rng, nu))
    return float(lib().orc_cov(kind, sigma2, rng, nu, d))


def cov_matrix(x, y, kind, sigma2, rng, nu, nugget=0.0, diag_add=None) -> np.ndarray:
    x, y = _c(x), _c(y)
    n = len(x)
    if not _half_integer(kind, nu):
        d = np.hypot(x[:, None] - x[None, :], y[:, None] - y[None, :])
        V = np.asfortranarray(_general(d, sigma2, rng, nu))
        V[np.diag_indices(n)] += _c(diag_add) if diag_add is not None else nugget
        return V
    V = np.empty((n, n), order="F")
    da = None
    if diag_add is not None:
        da_arr = _c(diag_add)
        da = da_arr.ctypes.data
    lib().orc_cov_matrix(x, y, n, kind, sigma2, rng, nu, nugget, da, V, n)
    return V


def cov_cross(xa, ya, xb, yb, kind, sigma2, rng, nu) -> np.ndarray:
    xa, ya, xb, yb = _c(xa), _c(ya), _c(xb), _c(yb)
    if not _half_integer(kind, nu):
        d = np.hypot(xa[:, None] - xb[None, :], ya[:, None] - yb[None, :])
        return np.asfortranarray(_general(d, sigma2, rng, nu))
    Cm = np.empty((len(xa), len(xb)), order="F")
    lib().orc_cov_cross(xa, ya, len(xa), xb, yb, len(xb), kind, sigma2, rng, nu, Cm, len(xa))
    return Cm


def tile_stats(V, nb: int) -> np.ndarray:
    """Per lower tile (row-packed t = i(i+1)/2 + j): [sum of squares, min, max]."""
    V = _f(V)
    n = V.shape[0]
    nt = (n + nb - 1) // nb
    st = np.zeros(3 * nt * (nt + 1) // 2)
    lib().orc_tile_stats(V, n, n, nb, st)
    return st.reshape(-1, 3)


def potrf(A) -> tuple[np.ndarray, int]:
    """Cholesky factor (lower, strict upper zeroed) and info (0 or 1-based failing column)."""
    A = np.array(A, dtype=np.float64, order="F", copy=True)
    info = lib().orc_potrf(A, A.shape[0], A.shape[0])
    return A, int(info)


def trmm(L, Z) -> np.ndarray:
    L, Z = _f(L), _f(Z)
    n, nsim = Z.shape
    M = np.empty((n, nsim), order="F")
    lib().orc_trmm(L, L.shape[0], n, Z, n, nsim, M, n)
    return M


def trsm_lower(L, B) -> np.ndarray:
    L = _f(L)
    B = np.array(B, dtype=np.float64, order="F", copy=True)
    if B.ndim == 1:
        B = B.reshape(-1, 1, order="F")
    lib().orc_trsm_lower(L, L.shape[0], L.shape[0], B, B.shape[0], B.shape[1])
    return B


def trsm_lower_trans(L, B) -> np.ndarray:
    L = _f(L)
    B = np.array(B, dtype=np.float64, order="F", copy=True)
    if B.ndim == 1:
        B = B.reshape(-1, 1, order="F")
    lib().orc_trsm_lower_trans(L, L.shape[0], L.shape[0], B, B.shape[0], B.shape[1])
    return B


def gemm(A, B, transa=False, transb=False, alpha=1.0) -> np.ndarray:
    A, B = _f(A), _f(B)
    m = A.shape[1] if transa else A.shape[0]
    k = A.shape[0] if transa else A.shape[1]
    n = B.shape[0] if transb else B.shape[1]
    Cm = np.zeros((m, n), order="F")
    lib().orc_gemm(int(transa), int(transb), m, n, k, alpha, A, A.shape[0], B, B.shape[0], 0.0, Cm, m)
    return Cm


def krige(xo, yo, xp, yp, y_obs, k_trend, kind, sigma2, rng, nu, tau2, want_H=False):
    """Universal kriging (Eq. 5-6).  Returns dict W, zhat, v, info (and H when asked)."""
    xo, yo, xp, yp, y_obs = _c(xo), _c(yo), _c(xp), _c(yp), _c(y_obs)
    n_o, n_p = len(xo), len(xp)
    W = np.zeros((n_o, n_p), order="F")
    zhat = np.zeros(n_p)
    v = np.zeros(n_p)
    H = np.zeros((max(k_trend, 1), n_p), order="F") if want_H else None
    if not _half_integer(kind, nu):
        # covariances of the general Matern order here, the kriging algebra in C as for the others
        Sy = cov_matrix(xo, yo, kind, sigma2, rng, nu, nugget=tau2)
        Vop = cov_cross(xo, yo, xp, yp, kind, sigma2, rng, nu)
        info = lib().orc_krige_mats(Sy, Vop, xo, yo, n_o, xp, yp, n_p, y_obs, k_trend, sigma2, W, zhat, v,
                                    H.ctypes.data if H is not None else None)
    else:
        info = lib().orc_krige(xo, yo, n_o, xp, yp, n_p, y_obs, k_trend, kind, sigma2, rng, nu, tau2,
                               W, zhat, v, H.ctypes.data if H is not None else None)
    out = {"W": W, "zhat": zhat, "v": v, "info": int(info)}
    if want_H:
        out["H"] = H[:k_trend]
    return out


def condition(M, n_p, W, y_obs) -> np.ndarray:
    """Eq. 7: S = M_p + W^T (y_o 1^T - M_o)."""
    M, W = _f(M), _f(W)
    n_o = M.shape[0] - n_p
    nsim = M.shape[1]
    S = np.empty((n_p, nsim), order="F")
    lib().orc_condition(M, M.shape[0], n_p, n_o, nsim, W, _c(y_obs), S, n_p)
    return S


def scan(S, u, t=None):
    """Eq. 8: counts per row, |A+_j|, psi_j, phi_j (sentinels +inf / -inf)."""
    S = _f(S)
    n, nsim = S.shape
    counts = np.zeros(n, dtype=np.int64)
    sizes = np.zeros(nsim, dtype=np.int32)
    psi = np.zeros(nsim)
    phi = np.zeros(nsim)
    tt = _c(t) if t is not None else None
    lib().orc_scan(S, n, n, nsim, tt.ctypes.data if tt is not None else None, u, counts, sizes,
                   psi.ctypes.data if tt is not None else None, phi.ctypes.data if tt is not None else None)
    out = {"counts": counts, "sizes": sizes}
    if t is not None:
        out["psi"], out["phi"] = psi, phi
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(np.asarray(ctr, dtype=np.uint32), np.asarray(key, dtype=np.uint32), out)
    return out


def normals(seed: int, stream: int, n: int, nsim: int, rows=None, cols=None) -> np.ndarray:
    """Seeded N(0,1) block of the logical n x nsim matrix (rows/cols = (start, stop))."""
    i0, i1 = rows if rows else (0, n)
    j0, j1 = cols if cols else (0, nsim)
    out = np.empty((i1 - i0, j1 - j0), order="F")
    lib().orc_normals(seed, stream, n, i0, i1, j0, j1, out, max(i1 - i0, 1))
    return out


def round_fp16(x: float) -> float:
    """Nearest IEEE binary16 value (ties to even) of x, as a float; |x| >= 65520 -> inf."""
    return float(lib().orc_round_fp16(float(x)))


def potrf_mp_emul(A, nb: int, pmap) -> tuple[np.ndarray, int]:
    """Emulated mixed-precision tile Cholesky of the scaled matrix A (Sec. IV-B): every tile
    stored in its precision of pmap (nt x nt), FP32 accumulation in reduced-precision updates.
    Returns (L_s with zeros above the diagonal, info)."""
    A = np.array(A, dtype=np.float64, order="F", copy=True)
    n = A.shape[0]
    nt = (n + nb - 1) // nb
    pm = np.ascontiguousarray(np.asarray(pmap, dtype=np.uint8).reshape(nt, nt))
    info = lib().orc_potrf_mp_emul(A, n, n, nb, pm)
    return A, int(info)


def trmm_mp_emul(Ls, nb: int, s: float, Z, fp16_dest: bool = False, diag16: bool = False) -> np.ndarray:
    """Emulated mixed-precision TRMM of Algorithm 1: M = L_s round16(Z / s) with FP32 diagonal
    products, FP16 off-diagonal products and FP32 sums; fp16_dest keeps the destination in FP16
    between k-tasks as the printed algorithm does; diag16 takes each diagonal tile as two FP16
    parts (hi, lo) inside one FP32 sum with the row's off-diagonal products."""
    if fp16_dest and diag16:
        raise ValueError("fp16_dest and diag16 are separate modes")
    Ls, Z = _f(Ls), _f(Z)
    n, nsim = Z.shape
    M = np.empty((n, nsim), order="F")
    mode = 2 if diag16 else int(bool(fp16_dest))
    lib().orc_trmm_mp_emul(Ls, Ls.shape[0], n, nb, float(s), Z, n, nsim, mode, M, n)
    return M

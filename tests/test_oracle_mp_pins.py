"""Pins of the oracle's random stream, binary16 rounding, emulated mixed-precision factorization and
TRMM, and the Eq. 12 bound the FP16 factor cast adds (CPU only).

Each pin is something other than the oracle itself: published known-answer vectors, numpy's
binary16 conversion, closed forms, exact integer arithmetic and rounding-error bounds.
"""
import json
import math
import os

import numpy as np
import pytest

import gpex_synth as syn
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EPS = {0: 2.0 ** -53, 1: 2.0 ** -24, 2: 2.0 ** -11}   # unit roundoff per tile precision
ETA = {0: 2.0 ** -1075, 1: 2.0 ** -150, 2: 2.0 ** -25}  # half the smallest subnormal spacing


def test_philox_known_answer_vectors():
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "philox4x32_10_kat.json")))
    for v in gold["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        out = oracle.philox4x32_10(ctr, key)
        assert [int(x) for x in out] == [int(x, 16) for x in v["out"]]


def test_round_fp16_matches_numpy_binary16():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 5, 20000),   # normals, subnormals, overflow
        (1.0 + np.arange(-40, 40) * 2.0 ** -11),                          # ties at 1 (every other one even)
        np.arange(1, 200) * 2.0 ** -25,                                   # ties in the subnormal range
        [65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 0.0, -0.0],
    ])
    got = np.array([oracle.round_fp16(v) for v in x])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)


def _case(n, nb, nu, beta, seed, tol, nt_rule):
    x, y = syn.uniform_locations(n, seed)
    x, y, _ = syn.ordered_locations(x, y)
    V = oracle.cov_matrix(x, y, 0, 1.0, beta, nu, nugget=1e-4)
    r = oracle.plan(oracle.tile_stats(V, nb), (n + nb - 1) // nb, tol, nt_rule=nt_rule)
    return V, r


def test_emulated_factor_all_fp64_map_is_cholesky():
    n, nb = 700, 96
    V, _ = _case(n, nb, 1.5, 0.1, 3, 0.0, True)
    nt = (n + nb - 1) // nb
    L, info = oracle.potrf_mp_emul(V, nb, np.zeros((nt, nt), np.uint8))
    Lo, _ = oracle.potrf(V)
    assert info == 0
    assert np.linalg.norm(L - Lo) / np.linalg.norm(Lo) <= 1e-12
    assert np.array_equal(L, np.tril(L))


@pytest.mark.parametrize("case", [(960, 96, 1.5, 0.03, 1002, 1e-9, False), (1100, 128, 1.5, 0.03, 7, 1e-7, True)])
def test_emulated_factor_storage_and_backward_error(case):
    n, nb, nu, beta, seed, tol, nt_rule = case
    V, r = _case(n, nb, nu, beta, seed, tol, nt_rule)
    nt = (n + nb - 1) // nb
    assert r.tiles[1] > 0 and r.tiles[2] > 0
    A = r.s ** 2 * V
    L, info = oracle.potrf_mp_emul(A, nb, r.pmap)
    assert info == 0
    sl = lambda i: slice(i * nb, min((i + 1) * nb, n))   # noqa: E731
    # every stored value is a value of its tile's precision (binary32 / binary16 by numpy)
    for i in range(nt):
        for j in range(i):
            t = L[sl(i), sl(j)]
            if r.pmap[i, j] == 1:
                assert np.array_equal(t, t.astype(np.float32).astype(np.float64)), (i, j)
            if r.pmap[i, j] == 2:
                assert np.array_equal(t, t.astype(np.float16).astype(np.float64)), (i, j)
    # backward error per tile within the rounding bound of the precisions involved (standard model
    # with gradual underflow, |round_p(x) - x| <= eps_p |x| + eta_p):
    # |(L L^T - A)_ij| <= c (eps_P(ij) |A_ij| + eta_P(ij)
    #                        + sum_k [eps_k (|L_ik| |L_jk|^T) + eta_k (1 + rowsum |L_jk|)]),
    # eps_k, eta_k of the widest rounding among P(ij), P(ik), P(jk)
    c = nb + 8
    for i in range(nt):
        for j in range(i + 1):
            pij = 0 if i == j else int(r.pmap[i, j])
            resid = np.abs(sum(L[sl(i), sl(k)] @ L[sl(j), sl(k)].T for k in range(j + 1)) - A[sl(i), sl(j)])
            bound = EPS[pij] * np.abs(A[sl(i), sl(j)]) + ETA[pij]
            for k in range(j + 1):
                pk = max(pij, 0 if i == k else int(r.pmap[i, k]), 0 if j == k else int(r.pmap[j, k]))
                bound = bound + EPS[pk] * (np.abs(L[sl(i), sl(k)]) @ np.abs(L[sl(j), sl(k)]).T)
                bound = bound + ETA[pk] * (1.0 + np.abs(L[sl(j), sl(k)]).sum(axis=1))[None, :]
            assert np.all(resid <= c * bound + 1e-300), (i, j)


@pytest.mark.parametrize("fp16_dest", [False, True])
def test_emulated_trmm_exact_on_integers(fp16_dest):
    # small integers: every operand, product and partial sum is exact in binary16 and binary32,
    # so both accumulation orders give the exact product L Z / s
    n, nb, nsim, s = 200, 32, 7, 8.0
    rng = np.random.default_rng(2)
    L = np.tril(rng.integers(-3, 4, (n, n)).astype(np.float64))
    B = rng.integers(-4, 5, (n, nsim)).astype(np.float64)
    M = oracle.trmm_mp_emul(L, nb, s, s * B, fp16_dest=fp16_dest)
    assert np.array_equal(M, L @ B)


def test_emulated_trmm_diagonal_parts_exact():
    """Whole-row form: diagonal entries 1 + 2^-12 k (hi = 1 in binary16, lo = 2^-12 k exactly) and
    small integer off-diagonal entries and B: every part, product and partial sum is exact in
    binary32, so the result is exactly L B; dropping lo, or pairing it with another row of B,
    changes it."""
    n, nb, nsim, s = 192, 64, 5, 4.0
    rng = np.random.default_rng(7)
    L = np.tril(rng.integers(-3, 4, (n, n)).astype(np.float64), -1)
    for i in range(0, n, nb):   # diagonal tiles: 1 + 2^-12 k, k in [-3, 3], on and below the diagonal
        blk = np.tril(1.0 + rng.integers(-3, 4, (min(nb, n - i),) * 2) * 2.0 ** -12)
        L[i:i + nb, i:i + nb] = blk
    B = rng.integers(-4, 5, (n, nsim)).astype(np.float64)
    M = oracle.trmm_mp_emul(L, nb, s, s * B, diag16=True)
    assert np.array_equal(M, L @ B)
    # the parts really split: hi alone (lo dropped) misses the 2^-12 terms
    hi_only = np.where(np.arange(n)[:, None] // nb == np.arange(n)[None, :] // nb, np.round(L), L)
    assert not np.array_equal(M, hi_only @ B)
    # the FP32-diagonal form agrees here too (cast32 of 1 + 2^-12 k is exact)
    assert np.array_equal(oracle.trmm_mp_emul(L, nb, s, s * B), M)


def test_emulated_trmm_diagonal_parts_accuracy():
    """On a real factor the whole-row form stays within the FP16 rounding of B of the exact product,
    and within about 2^-22 of the FP32-diagonal form (the parts carry L to about 22 bits)."""
    n, nb, nsim, s = 640, 64, 16, 300.0
    V, _ = _case(n, nb, 1.5, 0.1, 4, 0.0, True)
    L, _ = oracle.potrf(V)
    Ls = s * L
    Z = syn.explicit_normals(n, nsim, 9)
    M0 = oracle.trmm_mp_emul(Ls, nb, s, Z)
    M2 = oracle.trmm_mp_emul(Ls, nb, s, Z, diag16=True)
    scale = np.abs(Ls) @ np.abs(Z / s)
    assert np.all(np.abs(M2 - L @ Z) <= 3 * 2.0 ** -11 * scale + 1e-12)
    assert np.all(np.abs(M2 - M0) <= 2.0 ** -20 * scale + 1e-12)
    with pytest.raises(ValueError):
        oracle.trmm_mp_emul(Ls, nb, s, Z, fp16_dest=True, diag16=True)


def test_emulated_trmm_fp16_destination_rounding():
    n, nb, nsim, s = 640, 64, 16, 300.0
    V, _ = _case(n, nb, 1.5, 0.1, 4, 0.0, True)
    L, _ = oracle.potrf(V)
    Ls = s * L
    Z = syn.explicit_normals(n, nsim, 9)
    M0 = oracle.trmm_mp_emul(Ls, nb, s, Z, fp16_dest=False)
    M1 = oracle.trmm_mp_emul(Ls, nb, s, Z, fp16_dest=True)
    exact = L @ Z
    # FP16 destination values are binary16 numbers; each of the NT roundings adds at most half an
    # ulp (2^-11 relative), the operands' FP16 rounding 2^-11 relative each
    assert np.array_equal(M1, M1.astype(np.float16).astype(np.float64))
    nt = (n + nb - 1) // nb
    scale = np.abs(Ls) @ np.abs(Z / s)
    assert np.all(np.abs(M1 - exact) <= (nt + 1) * 2.0 ** -11 * np.abs(M1) + 3 * 2.0 ** -11 * scale + 1e-12)
    assert np.all(np.abs(M0 - exact) <= 3 * 2.0 ** -11 * scale + 1e-12)
    # the destination rounding is visible: about sqrt(NT) half-ulps of FP16 per entry
    d = np.linalg.norm(M1 - M0) / np.linalg.norm(M0)
    assert 1e-5 < d < 3e-3, d


def test_plan_bounds_scale_by_fp16_factor_cast():
    # sigma^2 = 4: without the bound s = 65503 and s * max|L| = s * 2 overflows binary16
    n, nb = 300, 64
    x, y = syn.uniform_locations(n, 11)
    x, y, _ = syn.ordered_locations(x, y)
    V = oracle.cov_matrix(x, y, 0, 4.0, 0.1, 1.5, nugget=1e-4)
    nt = (n + nb - 1) // nb
    r = oracle.plan(oracle.tile_stats(V, nb), nt, 1e-12, nt_rule=True)
    assert r.tiles[1] == r.tiles[2] == 0                # nothing reduced: Eq. 12 alone gives 65503
    assert r.u_factor == pytest.approx(65504.0 / math.sqrt(4.0001), rel=1e-15)
    assert r.s == math.floor(r.u_factor) - 1.0
    L, _ = oracle.potrf(V)
    assert r.s * np.abs(L).max() <= 65504.0
    assert 65503.0 * np.abs(L).max() > 65520.0          # the unbounded scale would overflow
    # unit variance + nugget: the bound is above 65503 - 1 and changes nothing but the integer part
    V1 = oracle.cov_matrix(x, y, 0, 1.0, 0.1, 1.5, nugget=1e-4)
    r1 = oracle.plan(oracle.tile_stats(V1, nb), nt, 1e-12, nt_rule=True)
    assert r1.s == math.floor(65504.0 / math.sqrt(1.0001)) - 1.0

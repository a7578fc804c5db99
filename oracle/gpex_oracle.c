/*
 * gpex_oracle.c -- plain, slow CPU FP64 oracle for the spatial excursion-set hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load this library.  It shares no code, header, table or helper with the HIP library and
 * must never be linked into it.
 *
 * What it follows (cited by page title, section and equation):
 *   [MPX] "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets"
 *         (Zhang, Abdulah, Cao, French, Alomairy, Genton, Keyes).
 *         Sec. III (excursion sets, Eq. 1), Sec. IV-C (TRMM, Eq. 3), Sec. V (joint covariance
 *         Eq. 4, universal kriging Eq. 5, MSPE Eq. 6, conditioning Eq. 7, extrema Eq. 8).
 *   [LAGP] "Massively parallel approximate Gaussian process regression" (Gramacy, Niemi,
 *         Weiss), isotropic Gaussian correlation exp(-||x-x'||^2 / theta).
 *   [PHILOX] Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11),
 *         Philox4x32 with 10 rounds; Box and Muller (1958) for the normal transform.
 *
 * Every function is exactly the textbook definition, written out with loops; no blocking,
 * fusion or reordering beyond what the definition states.  All arithmetic is IEEE FP64.
 * Matrices are column-major: element (i, j) of a matrix with leading dimension ld sits at
 * [i + j*ld].
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms, LAPACK special
 * cases, invariants, brute force); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX(i, j, ld) ((size_t)(i) + (size_t)(j) * (size_t)(ld))

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* Covariance functions.                                                                       */
/* kind 0: Matern with half-integer smoothness nu in {1/2, 3/2, 5/2}, distance scaled by the   */
/*         range beta (r = d / beta), written in the closed forms of the modified Bessel       */
/*         function K_nu at half-integer order:                                                */
/*            nu = 1/2: sigma2 * exp(-r)                                                       */
/*            nu = 3/2: sigma2 * (1 + r) * exp(-r)                                             */
/*            nu = 5/2: sigma2 * (1 + r + r^2/3) * exp(-r)                                     */
/* kind 1: Gaussian correlation [LAGP] scaled by the marginal variance:                        */
/*            sigma2 * exp(-d^2 / theta),  theta = range.                                      */
/* Returns NaN for an unsupported (kind, nu).                                                  */
/* ------------------------------------------------------------------------------------------ */
double orc_cov(int kind, double sigma2, double range, double nu, double d) {
    if (kind == 1) return sigma2 * exp(-(d * d) / range);
    if (kind != 0) return NAN;
    double r = d / range;
    if (nu == 0.5) return sigma2 * exp(-r);
    if (nu == 1.5) return sigma2 * (1.0 + r) * exp(-r);
    if (nu == 2.5) return sigma2 * (1.0 + r + r * r / 3.0) * exp(-r);
    return NAN;
}

static double dist2d(double xa, double ya, double xb, double yb) {
    double dx = xa - xb, dy = ya - yb;
    return sqrt(dx * dx + dy * dy);
}

/* Dense symmetric covariance over n locations.  The diagonal receives diag_add[i] when
 * diag_add is given, else the constant nugget.  ([MPX] Eq. 4: the measurement-error variance
 * is added only on the observation rows, which callers express through diag_add.) */
void orc_cov_matrix(const double* x, const double* y, int64_t n, int kind, double sigma2,
                    double range, double nu, double nugget, const double* diag_add, double* V,
                    int64_t ldv) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < n; ++i) {
            double v = orc_cov(kind, sigma2, range, nu, dist2d(x[i], y[i], x[j], y[j]));
            if (i == j) v += diag_add ? diag_add[i] : nugget;
            V[IDX(i, j, ldv)] = v;
        }
    }
}

/* Cross covariance C[i, j] = cov(a_i, b_j), na x nb. */
void orc_cov_cross(const double* xa, const double* ya, int64_t na, const double* xb,
                   const double* yb, int64_t nb, int kind, double sigma2, double range, double nu,
                   double* C, int64_t ldc) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nb; ++j)
        for (int64_t i = 0; i < na; ++i)
            C[IDX(i, j, ldc)] = orc_cov(kind, sigma2, range, nu, dist2d(xa[i], ya[i], xb[j], yb[j]));
}

/* Per-tile statistics of the lower tiles (i >= j) of an n x n matrix cut into nb x nb tiles
 * (the last tile row/column may be partial).  Tile (i, j) is stored at t = i*(i+1)/2 + j:
 * stats[3t] = sum of squares, stats[3t+1] = minimum entry, stats[3t+2] = maximum entry, over
 * the entries that exist.  ([MPX] Sec. V-D: tile Frobenius norms and entry extrema.) */
void orc_tile_stats(const double* V, int64_t ldv, int64_t n, int64_t nb, double* stats) {
    int64_t nt = (n + nb - 1) / nb;
#pragma omp parallel for schedule(dynamic)
    for (int64_t ti = 0; ti < nt; ++ti) {
        for (int64_t tj = 0; tj <= ti; ++tj) {
            int64_t t = ti * (ti + 1) / 2 + tj;
            double ss = 0.0, mn = INFINITY, mx = -INFINITY;
            for (int64_t j = tj * nb; j < (tj + 1) * nb && j < n; ++j)
                for (int64_t i = ti * nb; i < (ti + 1) * nb && i < n; ++i) {
                    double v = V[IDX(i, j, ldv)];
                    ss += v * v;
                    if (v < mn) mn = v;
                    if (v > mx) mx = v;
                }
            stats[3 * t] = ss;
            stats[3 * t + 1] = mn;
            stats[3 * t + 2] = mx;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Cholesky factorisation A = L L^T of a symmetric positive definite matrix, in place on the  */
/* lower triangle (the strict upper triangle is set to zero).  Right-looking column algorithm: */
/* for each column k, L_kk = sqrt(A_kk), L_ik = A_ik / L_kk, then A_ij -= L_ik L_jk for the   */
/* trailing lower triangle.  Returns 0, or the 1-based column whose pivot is not positive.    */
/* ------------------------------------------------------------------------------------------ */
int64_t orc_potrf(double* A, int64_t n, int64_t lda) {
    for (int64_t k = 0; k < n; ++k) {
        double akk = A[IDX(k, k, lda)];
        if (!(akk > 0.0)) return k + 1;
        double lkk = sqrt(akk);
        A[IDX(k, k, lda)] = lkk;
        for (int64_t i = k + 1; i < n; ++i) A[IDX(i, k, lda)] /= lkk;
#pragma omp parallel for schedule(static)
        for (int64_t j = k + 1; j < n; ++j) {
            double ljk = A[IDX(j, k, lda)];
            for (int64_t i = j; i < n; ++i) A[IDX(i, j, lda)] -= A[IDX(i, k, lda)] * ljk;
        }
    }
    for (int64_t j = 1; j < n; ++j)
        for (int64_t i = 0; i < j; ++i) A[IDX(i, j, lda)] = 0.0;
    return 0;
}

/* Left, lower, no-transpose triangular product M = L Z ([MPX] Eq. 3 with alpha = 1):
 * M[i, j] = sum_{k <= i} L[i, k] Z[k, j].  L is n x n lower triangular (upper part ignored). */
void orc_trmm(const double* L, int64_t ldl, int64_t n, const double* Z, int64_t ldz,
              int64_t nsim, double* M, int64_t ldm) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nsim; ++j) {
        for (int64_t i = 0; i < n; ++i) M[IDX(i, j, ldm)] = 0.0;
        for (int64_t k = 0; k < n; ++k) {
            double zk = Z[IDX(k, j, ldz)];
            for (int64_t i = k; i < n; ++i) M[IDX(i, j, ldm)] += L[IDX(i, k, ldl)] * zk;
        }
    }
}

/* Solve L X = B (forward substitution) in place, L n x n lower triangular, B n x m. */
void orc_trsm_lower(const double* L, int64_t ldl, int64_t n, double* B, int64_t ldb, int64_t m) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < m; ++j) {
        for (int64_t k = 0; k < n; ++k) {
            double xk = B[IDX(k, j, ldb)] / L[IDX(k, k, ldl)];
            B[IDX(k, j, ldb)] = xk;
            for (int64_t i = k + 1; i < n; ++i) B[IDX(i, j, ldb)] -= L[IDX(i, k, ldl)] * xk;
        }
    }
}

/* Solve L^T X = B (back substitution) in place. */
void orc_trsm_lower_trans(const double* L, int64_t ldl, int64_t n, double* B, int64_t ldb,
                          int64_t m) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < m; ++j) {
        for (int64_t i = n - 1; i >= 0; --i) {
            double s = B[IDX(i, j, ldb)];
            for (int64_t k = i + 1; k < n; ++k) s -= L[IDX(k, i, ldl)] * B[IDX(k, j, ldb)];
            B[IDX(i, j, ldb)] = s / L[IDX(i, i, ldl)];
        }
    }
}

/* C = alpha * op(A) * op(B) + beta * C, op = identity or transpose; C is m x n, inner size k. */
void orc_gemm(int transa, int transb, int64_t m, int64_t n, int64_t k, double alpha,
              const double* A, int64_t lda, const double* B, int64_t ldb, double beta, double* C,
              int64_t ldc) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        for (int64_t i = 0; i < m; ++i) {
            double s = 0.0;
            for (int64_t p = 0; p < k; ++p) {
                double a = transa ? A[IDX(p, i, lda)] : A[IDX(i, p, lda)];
                double b = transb ? B[IDX(j, p, ldb)] : B[IDX(p, j, ldb)];
                s += a * b;
            }
            C[IDX(i, j, ldc)] = (beta == 0.0 ? 0.0 : beta * C[IDX(i, j, ldc)]) + alpha * s;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Universal kriging, evaluated without explicit inverses in the order [MPX] Sec. V-A states:  */
/*   Sigma_y = V_o + tau2 I;  Sigma_y = L_o L_o^T;  Sigma_y F = X_o;  G = X_o^T F;             */
/*   G H = F^T V_op - X_p^T;  L_o Y = V_op - X_o H;  L_o^T W = Y;  zhat = W^T y_o;             */
/*   U = Sigma_y W;  v = theta0 1 + colsum(W .* U) - 2 colsum(V_op .* W)   (Eq. 5, Eq. 6).    */
/* With k_trend = 0 the trend terms vanish (simple kriging).  theta0 = sigma2, the latent     */
/* marginal variance; the error variance is not added to it.                                   */
/* Designs: X_o rows (1, x, y) at observation locations, X_p the same at prediction ones.      */
/* Outputs: W (n_o x n_p, ld n_o), zhat (n_p), v (n_p); H (k x n_p) if H_out is given.        */
/* Returns 0; the 1-based failing column of Sigma_y's factor; or -1 if G is not SPD.          */
/* ------------------------------------------------------------------------------------------ */
/* orc_krige_mats: the same from given Sigma_y (n_o x n_o, ld n_o) and V_op (n_o x n_p, ld n_o),
 * which it does not modify; orc_krige builds them from the locations with orc_cov. */
int64_t orc_krige_mats(const double* Sy, const double* Vop, const double* xo, const double* yo, int64_t n_o,
                       const double* xp, const double* yp, int64_t n_p, const double* y_obs, int k_trend,
                       double sigma2, double* W, double* zhat, double* v, double* H_out) {
    size_t no = (size_t)n_o, np_ = (size_t)n_p;
    double* Lo = (double*)malloc(sizeof(double) * no * no);
    double* U = (double*)malloc(sizeof(double) * no * np_);
    int64_t info = 0;
    memcpy(Lo, Sy, sizeof(double) * no * no);
    info = orc_potrf(Lo, n_o, n_o);
    if (info != 0) goto done;
    /* Right-hand side of the weight solves: V_op - X_o H (or V_op without a trend). */
    memcpy(W, Vop, sizeof(double) * no * np_);
    if (k_trend > 0) {
        int k = k_trend;
        double* Xo = (double*)malloc(sizeof(double) * no * k);
        double* Xp = (double*)malloc(sizeof(double) * np_ * k);
        double* F = (double*)malloc(sizeof(double) * no * k);
        double G[9], *Rhs = (double*)malloc(sizeof(double) * k * np_);
        for (int64_t i = 0; i < n_o; ++i) {
            Xo[IDX(i, 0, n_o)] = 1.0; Xo[IDX(i, 1, n_o)] = xo[i]; Xo[IDX(i, 2, n_o)] = yo[i];
        }
        for (int64_t i = 0; i < n_p; ++i) {
            Xp[IDX(i, 0, n_p)] = 1.0; Xp[IDX(i, 1, n_p)] = xp[i]; Xp[IDX(i, 2, n_p)] = yp[i];
        }
        /* Sigma_y F = X_o through the two triangular solves of the retained factor. */
        memcpy(F, Xo, sizeof(double) * no * k);
        orc_trsm_lower(Lo, n_o, n_o, F, n_o, k);
        orc_trsm_lower_trans(Lo, n_o, n_o, F, n_o, k);
        /* G = X_o^T F (k x k). */
        orc_gemm(1, 0, k, k, n_o, 1.0, Xo, n_o, F, n_o, 0.0, G, k);
        /* Rhs = F^T V_op - X_p^T (k x n_p). */
        orc_gemm(1, 0, k, n_p, n_o, 1.0, F, n_o, Vop, n_o, 0.0, Rhs, k);
        for (int64_t j = 0; j < n_p; ++j)
            for (int a = 0; a < k; ++a) Rhs[IDX(a, j, k)] -= Xp[IDX(j, a, n_p)];
        /* Solve G H = Rhs with a k x k Cholesky (the second POSV). */
        if (orc_potrf(G, k, k) != 0) {
            info = -1;
        } else {
            orc_trsm_lower(G, k, k, Rhs, k, n_p);
            orc_trsm_lower_trans(G, k, k, Rhs, k, n_p);
            if (H_out) memcpy(H_out, Rhs, sizeof(double) * k * np_);
            /* W <- V_op - X_o H */
            orc_gemm(0, 0, n_o, n_p, k, -1.0, Xo, n_o, Rhs, k, 1.0, W, n_o);
        }
        free(Xo); free(Xp); free(F); free(Rhs);
        if (info != 0) goto done;
    }
    /* L_o Y = V_op - X_o H, then L_o^T W = Y (the retained factor reused). */
    orc_trsm_lower(Lo, n_o, n_o, W, n_o, n_p);
    orc_trsm_lower_trans(Lo, n_o, n_o, W, n_o, n_p);
    /* zhat = W^T y_o */
    orc_gemm(1, 0, n_p, 1, n_o, 1.0, W, n_o, y_obs, n_o, 0.0, zhat, n_p);
    /* U = Sigma_y W with the unfactored Sigma_y, then Eq. 6 column by column. */
    orc_gemm(0, 0, n_o, n_p, n_o, 1.0, Sy, n_o, W, n_o, 0.0, U, n_o);
    for (int64_t j = 0; j < n_p; ++j) {
        double wu = 0.0, cw = 0.0;
        for (int64_t r = 0; r < n_o; ++r) {
            wu += W[IDX(r, j, n_o)] * U[IDX(r, j, n_o)];
            cw += Vop[IDX(r, j, n_o)] * W[IDX(r, j, n_o)];
        }
        v[j] = sigma2 + wu - 2.0 * cw;
    }
done:
    free(Lo); free(U);
    return info;
}

int64_t orc_krige(const double* xo, const double* yo, int64_t n_o, const double* xp,
                  const double* yp, int64_t n_p, const double* y_obs, int k_trend, int kind,
                  double sigma2, double range, double nu, double tau2, double* W, double* zhat,
                  double* v, double* H_out) {
    double* Sy = (double*)malloc(sizeof(double) * (size_t)n_o * (size_t)n_o);
    double* Vop = (double*)malloc(sizeof(double) * (size_t)n_o * (size_t)n_p);
    orc_cov_matrix(xo, yo, n_o, kind, sigma2, range, nu, tau2, NULL, Sy, n_o);
    orc_cov_cross(xo, yo, n_o, xp, yp, n_p, kind, sigma2, range, nu, Vop, n_o);
    int64_t info = orc_krige_mats(Sy, Vop, xo, yo, n_o, xp, yp, n_p, y_obs, k_trend, sigma2, W, zhat, v, H_out);
    free(Sy); free(Vop);
    return info;
}

/* Conditioning correction [MPX] Eq. 7: S = M_p + W^T (y_o 1^T - M_o), where M holds the
 * n_p prediction rows first and then the n_o observation rows. */
void orc_condition(const double* M, int64_t ldm, int64_t n_p, int64_t n_o, int64_t nsim,
                   const double* W, const double* y_obs, double* S, int64_t lds) {
    double* R = (double*)malloc(sizeof(double) * (size_t)n_o * (size_t)nsim);
    for (int64_t j = 0; j < nsim; ++j)
        for (int64_t r = 0; r < n_o; ++r) R[IDX(r, j, n_o)] = y_obs[r] - M[IDX(n_p + r, j, ldm)];
    for (int64_t j = 0; j < nsim; ++j)
        for (int64_t i = 0; i < n_p; ++i) S[IDX(i, j, lds)] = M[IDX(i, j, ldm)];
    orc_gemm(1, 0, n_p, nsim, n_o, 1.0, W, n_o, R, n_o, 1.0, S, lds);
    free(R);
}

/* Exceedance counts and per-simulation extrema, [MPX] Eq. 8:
 *   counts[i] = #{j : S_ij >= u},  sizes[j] = |A+_j| = #{i : S_ij >= u},
 *   psi[j] = min over A+_j of t_i (+inf when A+_j is empty),
 *   phi[j] = max over A-_j = {i : S_ij <= u} of t_i (-inf when A-_j is empty).
 * t may be NULL (no extrema: psi/phi untouched). */
void orc_scan(const double* S, int64_t lds, int64_t n_p, int64_t nsim, const double* t, double u,
              int64_t* counts, int32_t* sizes, double* psi, double* phi) {
    for (int64_t i = 0; i < n_p; ++i) counts[i] = 0;
    for (int64_t j = 0; j < nsim; ++j) {
        int32_t sz = 0;
        double mn = INFINITY, mx = -INFINITY;
        for (int64_t i = 0; i < n_p; ++i) {
            double s = S[IDX(i, j, lds)];
            if (s >= u) {
                counts[i] += 1;
                sz += 1;
                if (t && t[i] < mn) mn = t[i];
            }
            if (s <= u) {
                if (t && t[i] > mx) mx = t[i];
            }
        }
        sizes[j] = sz;
        if (t) {
            psi[j] = mn;
            phi[j] = mx;
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Philox4x32-10 [PHILOX] and Box-Muller normals.                                             */
/* One round: (hi0, lo0) = mulhilo(0xD2511F53, x0), (hi1, lo1) = mulhilo(0xCD9E8D57, x2),    */
/* x <- (hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0); the key is bumped by the Weyl constants     */
/* (0x9E3779B9, 0xBB67AE85) between rounds.                                                   */
/* ------------------------------------------------------------------------------------------ */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)x0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ x1 ^ k0, n1 = lo1, n2 = hi0 ^ x3 ^ k1, n3 = lo0;
        x0 = n0; x1 = n1; x2 = n2; x3 = n3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* 53-bit uniform in (0, 1) from two 32-bit words: ((w >> 11) + 1/2) * 2^-53, w = hi:lo. */
static double u01_from_words(uint32_t lo, uint32_t hi) {
    uint64_t w = ((uint64_t)hi << 32) | (uint64_t)lo;
    return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

/* Standard normals Z (rows i0..i1-1, columns j0..j1-1 of a logical n_rows x ncols matrix),
 * written to out (ld = ldo, out[(i-i0) + (j-j0)*ldo]).  Element (i, j) has linear index
 * l = j*n_rows + i and belongs to pair p = l / 2.  Pair p uses counter (p mod 2^32, p / 2^32,
 * stream, 0) and key (seed mod 2^32, seed / 2^32); u1 from words 0-1, u2 from words 2-3;
 * Z_{2p} = sqrt(-2 ln u1) cos(2 pi u2), Z_{2p+1} = sqrt(-2 ln u1) sin(2 pi u2). */
void orc_normals(uint64_t seed, uint32_t stream, int64_t n_rows, int64_t i0, int64_t i1,
                 int64_t j0, int64_t j1, double* out, int64_t ldo) {
    const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
    for (int64_t j = j0; j < j1; ++j) {
        for (int64_t i = i0; i < i1; ++i) {
            uint64_t l = (uint64_t)j * (uint64_t)n_rows + (uint64_t)i;
            uint64_t p = l >> 1;
            uint32_t ctr[4] = {(uint32_t)p, (uint32_t)(p >> 32), stream, 0u};
            uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
            uint32_t w[4];
            orc_philox4x32_10(ctr, key, w);
            double u1 = u01_from_words(w[0], w[1]);
            double u2 = u01_from_words(w[2], w[3]);
            double rad = sqrt(-2.0 * log(u1));
            out[IDX(i - i0, j - j0, ldo)] = (l & 1) ? rad * sin(two_pi * u2) : rad * cos(two_pi * u2);
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Emulated adaptive mixed precision ([MPX] Sec. IV-B, Algorithm 1, Sec. V-F).                 */
/* IEEE 754 binary16 and binary32 rounding (round to nearest, ties to even) applied at every   */
/* storage point of the tile algorithms, FP32 accumulation inside each reduced-precision task. */
/* ------------------------------------------------------------------------------------------ */

/* Nearest binary16 value of x (ties to even), as a double; |x| >= 65520 gives +-inf.  Binary16
 * has 11 significant bits, exponents -14..15 for normal numbers and the spacing 2^-24 below
 * 2^-14 (subnormals): x is scaled by the spacing of its binade (a power of two, exact), rounded
 * to an integer by nearbyint (ties to even in the default rounding mode) and scaled back. */
double orc_round_fp16(double x) {
    if (x != x || isinf(x) || x == 0.0) return x;
    double a = fabs(x);
    if (a >= 65520.0) return copysign(INFINITY, x);
    int e;
    frexp(a, &e);            /* a = f 2^e with f in [0.5, 1): the leading bit is 2^(e-1) */
    int lead = e - 1;
    if (lead < -14) lead = -14;
    double q = ldexp(1.0, lead - 10);
    return copysign(nearbyint(a / q) * q, x);
}

/* Nearest binary32 value of x (the C conversion rounds to nearest even). */
static double round_fp32(double x) { return (double)(float)x; }

/* Value of x stored in tile precision p (0 FP64, 1 FP32, 2 FP16). */
static double store_p(double x, int p) {
    if (p == 1) return round_fp32(x);
    if (p == 2) return orc_round_fp16(x);
    return x;
}

/* Emulated mixed-precision tile Cholesky of the n x n matrix A (lower triangle used; in: s^2 V,
 * out: L_s with zeros above the diagonal), tiles of nb with the last one partial, precision map
 * pmap (nt x nt row-major, codes 0 FP64 / 1 FP32 / 2 FP16; diagonal tiles FP64).  The steps are
 * the right-looking tile algorithm with the precision reading of each task:
 *   storage: every lower tile rounded to its precision;
 *   step k: POTRF of tile (k, k) in FP64 (orc_potrf on the tile);
 *           panel tile (i, k): L_ik = A_ik L_kk^-T by FP64 substitution, rounded once to P(i, k);
 *           tile (j, j), j > k: A_jj -= L_jk L_jk^T in FP64;
 *           tile (i, j), i > j > k, in P(i, j): operands rounded to P(i, j), products summed over the
 *           tile column index in that precision's accumulator (FP64; FP32 for FP32 and FP16 tiles,
 *           where FP16 products are exact in FP32), then A_ij = round_P(A_ij - sum).
 * Returns 0 or the 1-based failing column. */
int64_t orc_potrf_mp_emul(double* A, int64_t n, int64_t lda, int64_t nb, const uint8_t* pmap) {
    int64_t nt = (n + nb - 1) / nb;
#define P_(i, j) ((int)pmap[(size_t)(i) * (size_t)nt + (size_t)(j)])
#define R0(i) ((i) * nb)
#define RN(i) (((i) + 1) * nb < n ? nb : n - (i) * nb)
    for (int64_t i = 0; i < nt; ++i)
        for (int64_t j = 0; j < i; ++j)
            for (int64_t c = 0; c < RN(j); ++c)
                for (int64_t r = 0; r < RN(i); ++r) {
                    double* a = &A[IDX(R0(i) + r, R0(j) + c, lda)];
                    *a = store_p(*a, P_(i, j));
                }
    for (int64_t k = 0; k < nt; ++k) {
        int64_t rk = RN(k);
        double* Akk = &A[IDX(R0(k), R0(k), lda)];
        int64_t info = orc_potrf(Akk, rk, lda);
        if (info != 0) return R0(k) + info;
#pragma omp parallel for schedule(dynamic)
        for (int64_t i = k + 1; i < nt; ++i) {
            int64_t ri = RN(i);
            int p = P_(i, k);
            for (int64_t r = 0; r < ri; ++r) {
                /* row r of L_ik: x L_kk^T = a, forward substitution over the columns */
                double x[4096];
                for (int64_t c = 0; c < rk; ++c) {
                    double sacc = A[IDX(R0(i) + r, R0(k) + c, lda)];
                    for (int64_t m = 0; m < c; ++m) sacc -= x[m] * Akk[IDX(c, m, lda)];
                    x[c] = sacc / Akk[IDX(c, c, lda)];
                }
                for (int64_t c = 0; c < rk; ++c) A[IDX(R0(i) + r, R0(k) + c, lda)] = store_p(x[c], p);
            }
        }
        int64_t m_tiles = nt - k - 1;
#pragma omp parallel for schedule(dynamic)
        for (int64_t q = 0; q < m_tiles * m_tiles; ++q) {
            int64_t j = k + 1 + q / m_tiles, i = k + 1 + q % m_tiles;
            if (i < j) continue;
            int64_t ri = RN(i), rj = RN(j);
            int p = (i == j) ? 0 : P_(i, j);
            for (int64_t c = 0; c < rj; ++c)
                for (int64_t r = (i == j ? c : 0); r < ri; ++r) {
                    double* a = &A[IDX(R0(i) + r, R0(j) + c, lda)];
                    if (p == 0) {
                        double sacc = 0.0;
                        for (int64_t m = 0; m < rk; ++m)
                            sacc += A[IDX(R0(i) + r, R0(k) + m, lda)] * A[IDX(R0(j) + c, R0(k) + m, lda)];
                        *a = *a - sacc;
                    } else {
                        float facc = 0.0f;
                        for (int64_t m = 0; m < rk; ++m) {
                            float x = (float)store_p(A[IDX(R0(i) + r, R0(k) + m, lda)], p);
                            float y = (float)store_p(A[IDX(R0(j) + c, R0(k) + m, lda)], p);
                            facc += x * y;
                        }
                        *a = store_p((double)((float)*a - facc), p);
                    }
                }
        }
    }
    for (int64_t j = 1; j < n; ++j)
        for (int64_t i = 0; i < j; ++i) A[IDX(i, j, lda)] = 0.0;
    return 0;
#undef P_
#undef R0
#undef RN
}

/* Emulated mixed-precision TRMM M = L_s B, B = round16(Z / s) ([MPX] Algorithm 1 with AMP = 1):
 * Ls holds the stored factor values (n x n lower), tiles of nb, map pmap as above.  Row tile i of
 * column j:
 *   diagonal: FP32 product of cast32(L_ii) and cast32(B_i) (FP32 products and sums);
 *   off-diagonal tile k < i: FP16 operands cast16(L_ik) and B_k, products exact in FP32, summed in
 *   FP32 over the tile's columns.
 * fp16_dest = 1 (Algorithm 1 as printed, FP16 destination storage): the diagonal product is
 * rounded to FP16, then for k = 0 .. i-1 the running value enters an FP32 sum with tile k's
 * products and the result is rounded to FP16.  fp16_dest = 0: one FP32 sum of all off-diagonal
 * products of the row, added in FP64 to the FP32 diagonal product.  fp16_dest = 2 (the whole-row
 * form, a reading of ours: the pages fix no format for the diagonal product): the diagonal tile
 * enters as two FP16 parts, hi = cast16(L) and lo = cast16(L - hi), both multiplied with B_i, and
 * the row's off-diagonal and diagonal products form one FP32 sum (off-diagonal columns first, then
 * hi and lo of each diagonal column in turn).  M is FP64. */
void orc_trmm_mp_emul(const double* Ls, int64_t ldl, int64_t n, int64_t nb, double s, const double* Z,
                      int64_t ldz, int64_t nsim, int fp16_dest, double* M, int64_t ldm) {
    int64_t nt = (n + nb - 1) / nb;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nsim; ++j) {
        double* b = (double*)malloc(sizeof(double) * (size_t)n);
        for (int64_t i = 0; i < n; ++i) b[i] = orc_round_fp16(Z[IDX(i, j, ldz)] / s);
        for (int64_t ti = 0; ti < nt; ++ti) {
            int64_t r0 = ti * nb, r1 = (ti + 1) * nb < n ? (ti + 1) * nb : n;
            for (int64_t r = r0; r < r1; ++r) {
                if (fp16_dest == 2) {
                    float acc = 0.0f;
                    for (int64_t m = 0; m < r0; ++m) acc += (float)orc_round_fp16(Ls[IDX(r, m, ldl)]) * (float)b[m];
                    for (int64_t m = r0; m <= r; ++m) {
                        const double hi = orc_round_fp16(Ls[IDX(r, m, ldl)]);
                        const double lo = orc_round_fp16(Ls[IDX(r, m, ldl)] - hi);
                        acc += (float)hi * (float)b[m];
                        acc += (float)lo * (float)b[m];
                    }
                    M[IDX(r, j, ldm)] = (double)acc;
                    continue;
                }
                float d = 0.0f;
                for (int64_t m = r0; m <= r; ++m) d += (float)Ls[IDX(r, m, ldl)] * (float)b[m];
                if (fp16_dest) {
                    float dest = (float)orc_round_fp16((double)d);
                    for (int64_t tk = 0; tk < ti; ++tk) {
                        float acc = dest;
                        for (int64_t m = tk * nb; m < (tk + 1) * nb; ++m)
                            acc += (float)orc_round_fp16(Ls[IDX(r, m, ldl)]) * (float)b[m];
                        dest = (float)orc_round_fp16((double)acc);
                    }
                    M[IDX(r, j, ldm)] = (double)dest;
                } else {
                    float acc = 0.0f;
                    for (int64_t m = 0; m < r0; ++m) acc += (float)orc_round_fp16(Ls[IDX(r, m, ldl)]) * (float)b[m];
                    M[IDX(r, j, ldm)] = (double)d + (double)acc;
                }
            }
        }
        free(b);
    }
}

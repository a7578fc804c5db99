// Matern correlation for a general smoothness nu ("Mixed-Precision GPU Acceleration for Confidence
// Regions of Spatial Excursion Sets", Sec. V-E and VI: the Matern kernel with parameters sigma^2,
// range and nu): 2^(1 - nu) / Gamma(nu) r^nu K_nu(r) with r = d / range (the half-integer orders
// 1/2, 3/2, 5/2 have closed forms and do not come here).
//
// K_nu by the trapezoidal rule on the integral K_nu(r) = int_0^inf exp(-r cosh t) cosh(nu t) dt
// (DLMF 10.32.9).  The integrand is analytic in a strip around the real axis, so the rule
// converges exponentially in 1 / h ("The exponentially convergent trapezoidal rule", Trefethen and
// Weideman, SIAM Review 2014).  With e^-r factored out,
//   e^r K_nu(r) = h [1/2 + sum_{k >= 1} exp(-2 r sinh^2(k h / 2)) cosh(nu k h)],
// (cosh t - 1 written as 2 sinh^2(t / 2), without cancellation), with the step narrowed where the
// integrand is narrow (large r: width about 1 / sqrt(r)) or grows fast (large nu):
// h = h0 / sqrt(max(1, r)), h0 = 0.25 / sqrt(max(1, nu / 2)).  cosh(nu k h) is half the sum of
// e^(+-nu k h), each a running product (the three-term recurrence of cosh loses accuracy when nu h
// is small).  The terms are summed until one falls below 1e-17 of the sum.  Against a 30-digit
// reference, for nu in [0.05, 8]: relative error below 6e-15 for r in [1, 60] and 2.5e-14 for r in
// [1e-7, 1]; beyond r = 60 the error is that of exp(-r) for a rounded r, about r ulps (as for the
// closed forms).  About 36 terms for r >= 1 and nu <= 2, more for small r or large nu.  r is
// evaluated no smaller than 1e-30 (for nu below 1/2 this changes entries of points closer than
// 1e-30 range).
#pragma once

namespace gpex {

constexpr double MATERN_NU_MIN = 0.05, MATERN_NU_MAX = 8.0;   // the orders the quadrature was checked for
constexpr double MATERN_R_MIN = 1e-30;
constexpr int MATERN_MAX_TERMS = 4096;

// h0 for the given nu (host and device).
__host__ __device__ inline double matern_h0(double nu) { return 0.25 / sqrt(nu > 2.0 ? 0.5 * nu : 1.0); }

// The correlation (1 at r = 0).  lcoef = log(2^(1 - nu) / Gamma(nu)).
__device__ inline double matern_general(double r, double nu, double h0, double lcoef) {
    if (!(r > 0.0)) return 1.0;
    r = fmax(r, MATERN_R_MIN);
    const double h = r > 1.0 ? h0 / sqrt(r) : h0;
    const double ep = exp(nu * h), em = 1.0 / ep;
    double s = 0.5, e_k = ep, ei_k = em;   // e^(nu k h), e^(-nu k h)
    for (int k = 1; k <= MATERN_MAX_TERMS; ++k) {
        const double sh = sinh(0.5 * h * k);
        const double term = exp(-2.0 * r * sh * sh) * (0.5 * (e_k + ei_k));
        s += term;
        if (term < 1e-17 * s) break;
        e_k *= ep;
        ei_k *= em;
    }
    return exp(lcoef + nu * log(r) - r) * (h * s);
}

}  // namespace gpex

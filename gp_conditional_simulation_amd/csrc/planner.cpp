// Host precision planner: tile map, Eq. 10 / Eq. 11 checks and the Eq. 12 scale.
//
// "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets":
//   Sec. IV-B  diagonal tiles FP64; off-diagonal tiles FP32 or FP16 by numerical significance;
//   Sec. V-D   the rule compares a tile's Frobenius norm with the global norm (smaller fixedacc
//              keeps more tiles in high precision); Eq. 10 representability range (strict <),
//              Eq. 11 relative magnitude of the FP16 tiles;
//   Sec. V-E   Eq. 12: l_f = sqrt(x_min,norm / v_min), u_f = sqrt(x_max / v_max) over present
//              reduced formats, u_s = min(65504, min_f u_f), s = floor(u_s) - 1 when that exceeds 1.
//   Algorithm 1 casts the scaled factor to FP16; |(L_s)_ij| <= s sqrt(V_ii) adds the bound
//              u_L = 65504 / sqrt(max_i V_ii) to u_s (it binds only when max_i V_ii > 1).
// Readings where the page is silent or garbled: the tile rule r * NT * eps_p <= tol with
// r = ||V_ij||_F / ||V||_F and NT tile rows (the unscaled r * eps_p <= tol on request);
// Eq. 11 as max(rho1, rho2) < 1e-4/2^-10;
// no FP16 tile -> Eq. 10/11 pass vacuously; no reduced tile -> u_s = 65504.
// ||V||_F^2 is summed in row-packed tile order, off-diagonal tiles twice.
#include <cmath>
#include <limits>

#include "common.h"

namespace gpex {

static void plan_once(const std::vector<double>& st, int64_t nt, const gpex_prec_opts& o,
                      std::vector<uint8_t>& map, gpex_diag& d) {
    const double eps16 = std::ldexp(1.0, -10), eps32 = std::ldexp(1.0, -23);
    const double xmax32 = (2.0 - std::ldexp(1.0, -23)) * std::ldexp(1.0, 127), xmax16 = 65504.0;
    const double xnorm32 = std::ldexp(1.0, -126), xnorm16 = std::ldexp(1.0, -14);
    const double xsub32 = std::ldexp(1.0, -149), xsub16 = std::ldexp(1.0, -24);
    auto T = [&](int64_t i, int64_t j) { return &st[(size_t)(3 * (i * (i + 1) / 2 + j))]; };

    map.assign((size_t)(nt * nt), 255);
    d = gpex_diag{};
    double f2 = 0.0;
    for (int64_t i = 0; i < nt; ++i)
        for (int64_t j = 0; j <= i; ++j) f2 += (i == j) ? T(i, j)[0] : 2.0 * T(i, j)[0];
    d.frob = std::sqrt(f2);
    const double mult = o.unscaled_rule ? 1.0 : (double)nt;
    for (int64_t i = 0; i < nt; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            uint8_t p = DT_F64;
            if (o.amp && i != j) {
                double r = std::sqrt(T(i, j)[0]) / d.frob;
                if (o.allow_fp16 && r * mult * eps16 <= o.tol) p = DT_F16;
                else if (r * mult * eps32 <= o.tol) p = DT_F32;
            }
            map[(size_t)(i * nt + j)] = p;
            d.tiles[p] += 1;
        }
    d.eq10_pass = d.eq11_pass = 1;
    d.r_hp = std::numeric_limits<double>::quiet_NaN();
    if (!o.amp) {
        d.s = 1.0;
        d.u_bound = 1.0;
        return;
    }
    // Eq. 10 and Eq. 11 over the FP16 tiles
    double vmax_all = -INFINITY, norm_all = 0.0, vmax_hp = -INFINITY, vmin_hp = INFINITY, norm_hp = 0.0;
    bool any_hp = false;
    for (int64_t i = 0; i < nt; ++i)
        for (int64_t j = 0; j <= i; ++j) {
            const double* s = T(i, j);
            vmax_all = std::fmax(vmax_all, s[2]);
            norm_all = std::fmax(norm_all, std::sqrt(s[0]));
            if (map[(size_t)(i * nt + j)] == DT_F16) {
                any_hp = true;
                vmax_hp = std::fmax(vmax_hp, s[2]);
                vmin_hp = std::fmin(vmin_hp, s[1]);
                norm_hp = std::fmax(norm_hp, std::sqrt(s[0]));
            }
        }
    if (any_hp) {
        if (vmin_hp > 0.0) {
            d.r_hp = vmax_hp / vmin_hp;
            d.eq10_pass = d.r_hp < 65504.0 / xsub16;
        } else {
            d.r_hp = INFINITY;
            d.eq10_pass = 0;
        }
        d.rho1 = vmax_hp / vmax_all;
        d.rho2 = norm_hp / norm_all;
        d.eq11_pass = std::fmax(d.rho1, d.rho2) < 1e-4 / eps16;
    }
    // Eq. 12 over the present reduced formats
    double l = 0.0, lsub = 0.0, umin = INFINITY;
    for (int f = DT_F32; f <= DT_F16; ++f) {
        double vmin = INFINITY, vmax = -INFINITY;
        bool present = false;
        for (int64_t i = 0; i < nt; ++i)
            for (int64_t j = 0; j <= i; ++j)
                if (map[(size_t)(i * nt + j)] == f) {
                    present = true;
                    vmin = std::fmin(vmin, T(i, j)[1]);
                    vmax = std::fmax(vmax, T(i, j)[2]);
                }
        if (!present) continue;
        const double xn = f == DT_F32 ? xnorm32 : xnorm16;
        const double xs = f == DT_F32 ? xsub32 : xsub16;
        const double xm = f == DT_F32 ? xmax32 : xmax16;
        double lf = vmin > 0.0 ? std::sqrt(xn / vmin) : INFINITY;
        double lsf = vmin > 0.0 ? std::sqrt(xs / vmin) : INFINITY;
        double uf = vmax > 0.0 ? std::sqrt(xm / vmax) : INFINITY;
        l = std::fmax(l, lf);
        lsub = std::fmax(lsub, lsf);
        umin = std::fmin(umin, uf);
    }
    // The simulation product casts L_s to FP16 (Algorithm 1), and |(L_s)_ij| <= s sqrt(V_ii): the
    // factor stays finite in FP16 when s <= x_max,FP16 / sqrt(max_i V_ii).
    double vmax_diag = -INFINITY;
    for (int64_t i = 0; i < nt; ++i) vmax_diag = std::fmax(vmax_diag, T(i, i)[2]);
    d.u_factor = vmax_diag > 0.0 ? xmax16 / std::sqrt(vmax_diag) : INFINITY;
    d.l_bound = l;
    d.l_bound_sub = lsub;
    d.u_bound = std::fmin(std::fmin(65504.0, umin), d.u_factor);
    d.lower_exceeds_upper = l > d.u_bound;
    double sc = std::floor(d.u_bound) - 1.0;
    d.s = sc > 1.0 ? sc : 1.0;
}

// Sec. V-D automatic mode: fixedacc starts at 1e-4 and is reduced by a factor of 0.9 whenever
// either check fails; iteration stops when both pass or no FP16 tile remains.  A tile whose norm
// is exactly zero would stay FP16 at any tolerance, so the loop is capped at 2000 reductions.
void plan_precision(const std::vector<double>& st, int64_t nt, const gpex_prec_opts& o,
                    std::vector<uint8_t>& map, gpex_diag& d) {
    gpex_prec_opts q = o;
    int64_t red = 0;
    if (o.amp && o.auto_tol) {
        q.tol = 1e-4;
        for (;;) {
            plan_once(st, nt, q, map, d);
            if ((d.eq10_pass && d.eq11_pass) || d.tiles[DT_F16] == 0 || red >= 2000) break;
            q.tol *= 0.9;
            ++red;
        }
    } else {
        plan_once(st, nt, q, map, d);
    }
    d.tol = q.tol;
    d.tol_reductions = red;
}

}  // namespace gpex

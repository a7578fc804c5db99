// Universal kriging predictor and pointwise MSPE.
//
// "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets", Sec. V-A:
//   W = Sigma_y^-1 [V_op - X_o (X_o^T Sigma_y^-1 X_o)^-1 (X_o^T Sigma_y^-1 V_op - X_p^T)]   (Eq. 5)
//   zhat = W^T y_o,  v_i = (V_p)_ii + w_i^T Sigma_y w_i - 2 w_i^T c_i                      (Eq. 6)
// evaluated without explicit inverses: Sigma_y = L_o L_o^T (FP64 tile Cholesky), Sigma_y F = X_o,
// G = X_o^T F, G H = F^T V_op - X_p^T (3 x 3), L_o Y = V_op - X_o H, L_o^T W = Y (the retained
// factor is reused), zhat = W^T y_o.  The kriging stage is FP64 throughout.
//
// Differences from the page's implementation, same values in exact arithmetic:
//   * the triangular solves are blocked over the tiles of L_o and apply each diagonal block
//     through its explicit inverse T_k (kept by the factorisation), so every step is a
//     matrix-core GEMM over the full n_p-wide panel;
//   * U = Sigma_y W is not formed by a second n_o^2 n_p product: Sigma_y W = V_op - X_o H holds
//     by construction, so v = sigma2 1 - colsum(W .* (V_op + X_o H)).
#include <algorithm>
#include <cmath>

#include <vector>

#include "common.h"
#include "matern.h"

namespace gpex {

struct CovK {
    int kind;
    double sigma2, range, nu;
    double h0, lcoef;   // Matern of another nu (matern.h)
};

__device__ __forceinline__ double covk(const CovK& p, double d) {
    if (p.kind == 1) return p.sigma2 * exp(-(d * d) / p.range);
    double r = d / p.range;
    if (!(p.nu == 0.5 || p.nu == 1.5 || p.nu == 2.5)) return p.sigma2 * matern_general(r, p.nu, p.h0, p.lcoef);
    const double e = exp(-r);
    if (p.nu == 0.5) return p.sigma2 * e;
    if (p.nu == 1.5) return p.sigma2 * (1.0 + r) * e;
    return p.sigma2 * (1.0 + r + r * r / 3.0) * e;
}

// C (na x nb, leading dim na) = cov(a_i, b_j); thread per entry, rows fastest (coalesced).
__global__ void k_cov_cross(const double* la, int64_t na, const double* lb, int64_t nbv, CovK p, double* C) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= na * nbv) return;
    int64_t i = idx % na, j = idx / na;
    double dx = la[i] - lb[j], dy = la[na + i] - lb[nbv + j];
    C[idx] = covk(p, sqrt(dx * dx + dy * dy));
}

// X (n x 3, leading dim ldx) = rows (1, x, y), zero rows beyond n up to rows_pad.
__global__ void k_design(const double* loc, int64_t n, int64_t rows_pad, double* X, int64_t ldx) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows_pad) return;
    bool ok = i < n;
    X[i] = ok ? 1.0 : 0.0;
    X[i + ldx] = ok ? loc[i] : 0.0;
    X[i + 2 * ldx] = ok ? loc[n + i] : 0.0;
}

// Rhs (3 x np) -= X_p^T, then H = Ginv * Rhs (Ginv given as 9 row-major values).
__global__ void k_trend_h(double* Rhs, const double* locp, int64_t np, double g0, double g1, double g2,
                          double g3, double g4, double g5, double g6, double g7, double g8) {
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= np) return;
    double r0 = Rhs[3 * j] - 1.0, r1 = Rhs[3 * j + 1] - locp[j], r2 = Rhs[3 * j + 2] - locp[np + j];
    Rhs[3 * j] = g0 * r0 + g1 * r1 + g2 * r2;
    Rhs[3 * j + 1] = g3 * r0 + g4 * r1 + g5 * r2;
    Rhs[3 * j + 2] = g6 * r0 + g7 * r1 + g8 * r2;
}

// v_j = sigma2 - sum_r W_rj (V_op_rj + (X_o H)_rj), one workgroup per column, fixed-order sum.
__global__ __launch_bounds__(256) void k_mspe(const double* W, const double* Vop, const double* Xo,
                                              int64_t ldx, const double* H, int ktr, int64_t no,
                                              int64_t np, double sigma2, double* v) {
    int64_t j = blockIdx.x;
    if (j >= np) return;
    double h0 = 0, h1 = 0, h2 = 0;
    if (ktr) { h0 = H[3 * j]; h1 = H[3 * j + 1]; h2 = H[3 * j + 2]; }
    double acc = 0.0;
    for (int64_t r = threadIdx.x; r < no; r += 256) {
        double xh = ktr ? Xo[r] * h0 + Xo[r + ldx] * h1 + Xo[r + 2 * ldx] * h2 : 0.0;
        acc += W[r + j * no] * (Vop[r + j * no] + xh);
    }
    __shared__ double red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) v[j] = sigma2 - red[0];
}

// W (no x np) -= X_o H
__global__ void k_sub_xh(double* W, const double* Xo, int64_t ldx, const double* H, int64_t no, int64_t np) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= no * np) return;
    int64_t r = idx % no, j = idx / no;
    W[idx] -= Xo[r] * H[3 * j] + Xo[r + ldx] * H[3 * j + 1] + Xo[r + 2 * ldx] * H[3 * j + 2];
}

static unsigned nblk(int64_t n) { return (unsigned)((n + 255) / 256); }

// In place B (n x m, leading dim ldb, n = L->n) <- L^-1 B (trans = 0) or L^-T B (trans = 1), using
// the tiles of the FP64 factor and the inverse diagonal tiles.  tmp: nb x m FP64 scratch.
// Step k applies T_k (or T_k^T) to block row k, then subtracts its contribution from every block
// row still to be solved in one batched launch (the full-height rows; a ragged last row of tiles
// gets a launch of its own).
static int tile_trsm(gpex_ctx_t ctx, gpex_tiled_t L, double* B, int64_t ldb, int64_t m, int trans, double* tmp,
                     GemmTask* d_tasks) {
    const int64_t nt = L->nt, nb = L->nb, n = L->n;
    hipStream_t s = ctx->stream;
    auto rows = [&](int64_t k) { return std::min<int64_t>(nb, n - k * nb); };
    struct Step { int64_t k, b0, b1; bool ragged; };
    std::vector<GemmTask> tasks;
    std::vector<Step> steps;
    auto task = [&](int64_t i, int64_t k) {
        GemmTask g{};
        g.A = trans ? L->tile(k, i) : L->tile(i, k); g.ta = DT_F64; g.lda = nb; g.transA = (int8_t)trans;
        g.B = B + k * nb; g.tb = DT_F64; g.ldb = ldb; g.transB = 0;
        g.C = B + i * nb; g.tc = DT_F64; g.ldc = ldb;
        g.M = (int)rows(i); g.N = (int)m; g.K = (int)rows(k);
        g.alpha = -1.0; g.beta = 1.0;
        return g;
    };
    for (int64_t step = 0; step < nt; ++step) {
        const int64_t k = trans ? nt - 1 - step : step;
        Step st{k, (int64_t)tasks.size(), 0, false};
        if (!trans) {   // B_i -= L_ik B_k, i > k
            for (int64_t i = k + 1; i < nt; ++i)
                if (rows(i) == nb) tasks.push_back(task(i, k));
            st.ragged = k + 1 < nt && rows(nt - 1) < nb;
        } else {        // B_i -= L_ki^T B_k, i < k (all full height)
            for (int64_t i = 0; i < k; ++i) tasks.push_back(task(i, k));
        }
        st.b1 = (int64_t)tasks.size();
        steps.push_back(st);
    }
    // d_tasks holds nt (nt - 1) / 2 tasks; the upload is ordered after the previous solve's launches
    if (!tasks.empty())
        GPEX_HIP(ctx, hipMemcpyAsync(d_tasks, tasks.data(), sizeof(GemmTask) * tasks.size(), hipMemcpyHostToDevice, s));
    int r = GPEX_OK;
    for (const Step& st : steps) {
        const int64_t k = st.k, rk = rows(k);
        double* Bk = B + k * nb;
        // Bk <- T_k Bk  (or T_k^T Bk); T_k is lower triangular
        GemmTask d{};
        d.A = L->tinv_tile(k); d.ta = DT_F64; d.lda = nb; d.transA = (int8_t)trans;
        d.B = Bk; d.tb = DT_F64; d.ldb = ldb; d.transB = 0;
        d.C = tmp; d.tc = DT_F64; d.ldc = nb;
        d.M = (int)rk; d.N = (int)m; d.K = (int)rk; d.alpha = 1.0; d.beta = 0.0;
        d.tri = trans ? 0 : TRI_A_LOWER;
        r = gemm_launch(ctx, s, DT_F64, nullptr, 1, d);
        if (r >= 0) r = copy2d(ctx, s, tmp, DT_F64, nb, Bk, DT_F64, ldb, rk, m, 1.0);
        if (r >= 0 && st.b1 > st.b0)
            r = gemm_launch(ctx, s, DT_F64, d_tasks + st.b0, (int)(st.b1 - st.b0), tasks[(size_t)st.b0]);
        if (r >= 0 && st.ragged) {
            GemmTask g = task(nt - 1, k);
            r = gemm_launch(ctx, s, DT_F64, nullptr, 1, g);
        }
        if (r < 0) break;
    }
    // the host task list must outlive its upload
    if (hipStreamSynchronize(s) != hipSuccess && r >= 0) r = set_err(ctx, GPEX_ERR_HIP, "solve sync");
    return r;
}

}  // namespace gpex

using namespace gpex;

extern "C" int gpex_krige(gpex_ctx_t ctx, const double* d_loc_o, int64_t n_o, const double* d_loc_p,
                          int64_t n_p, const double* d_y_o, int k_trend, const gpex_cov_params* params,
                          double tau2, int nb, double* d_W, double* d_zhat, double* d_v, int64_t* info) {
    if (!ctx) return GPEX_ERR_ARG;
    if (!d_loc_o || !d_loc_p || !d_y_o || !params || !d_W || !d_zhat || !d_v || !info || n_o < 1 || n_p < 1)
        return set_err(ctx, GPEX_ERR_ARG, "gpex_krige: null pointer or empty size");
    if (k_trend != 0 && k_trend != 3) return set_err(ctx, GPEX_ERR_ARG, "gpex_krige: k_trend must be 0 or 3");
    if (k_trend == 3 && n_o < 3) return set_err(ctx, GPEX_ERR_ARG, "gpex_krige: the trend needs n_o >= 3");
    if (!(tau2 >= 0.0)) return set_err(ctx, GPEX_ERR_ARG, "gpex_krige: tau2 must be >= 0");
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    hipStream_t s = ctx->stream;
    *info = 0;
    gpex_cov_params cp = *params;
    cp.nugget = tau2;
    gpex_prec_opts po{0, 0.0, 0, 0, 0, 0};
    gpex_tiled_t Sy = nullptr;
    int r = gpex_cov_gen(ctx, d_loc_o, n_o, nullptr, &cp, nb, &po, &Sy, nullptr);
    if (r < 0) return r;
    r = gpex_potrf_mp(ctx, Sy, info);
    if (r != GPEX_OK) {
        gpex_tiled_destroy(Sy);
        return r;
    }
    const int64_t ntile = Sy->nt;
    const int64_t rows_pad = ntile * nb;
    auto cleanup = [&]() { gpex_tiled_destroy(Sy); };
    const int64_t mtmp = std::max<int64_t>(n_p, 3);
    // workspace: V_op, the solve scratch, X_o, F, G, H and the solve task list
    Carve cv;
    const size_t p_vop = cv.add(sizeof(double) * n_o * n_p), p_tmp = cv.add(sizeof(double) * nb * mtmp),
                 p_xo = cv.add(sizeof(double) * rows_pad * 3), p_f = cv.add(sizeof(double) * n_o * 3),
                 p_g = cv.add(sizeof(double) * 9), p_h = cv.add(sizeof(double) * 3 * n_p),
                 p_tk = cv.add(sizeof(GemmTask) * (size_t)(ntile * (ntile - 1) / 2));
    void* wsb = nullptr;
    r = ws_get(ctx, WS_KRIGE, cv.total, &wsb, "kriging workspace");
    if (r < 0) { cleanup(); return r; }
    double* Vop = cv.get<double>(wsb, p_vop);
    double* tmp = cv.get<double>(wsb, p_tmp);
    double* Xo = cv.get<double>(wsb, p_xo);
    double* F = cv.get<double>(wsb, p_f);
    double* G = cv.get<double>(wsb, p_g);
    double* H = cv.get<double>(wsb, p_h);
    GemmTask* d_tk = cv.get<GemmTask>(wsb, p_tk);
    CovK ck{params->kind, params->sigma2, params->range, params->nu, matern_h0(params->nu),
            (1.0 - params->nu) * std::log(2.0) - std::lgamma(params->nu)};
    hipLaunchKernelGGL(k_cov_cross, dim3(nblk(n_o * n_p)), dim3(256), 0, s, d_loc_o, n_o, d_loc_p, n_p, ck, Vop);
    hipLaunchKernelGGL(k_design, dim3(nblk(rows_pad)), dim3(256), 0, s, d_loc_o, n_o, rows_pad, Xo, rows_pad);
    if (hipGetLastError() != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "krige setup launch"); }
    r = copy2d(ctx, s, Vop, DT_F64, n_o, d_W, DT_F64, n_o, n_o, n_p, 1.0);
    if (r < 0) { cleanup(); return r; }
    if (k_trend == 3) {
        // F = Sigma_y^-1 X_o
        r = copy2d(ctx, s, Xo, DT_F64, rows_pad, F, DT_F64, n_o, n_o, 3, 1.0);
        if (r >= 0) r = tile_trsm(ctx, Sy, F, n_o, 3, 0, tmp, d_tk);
        if (r >= 0) r = tile_trsm(ctx, Sy, F, n_o, 3, 1, tmp, d_tk);
        // G = X_o^T F (3 x 3);  Rhs = F^T V_op (3 x n_p) into H
        if (r >= 0) r = gemm1(ctx, DT_F64, Xo, DT_F64, 1, rows_pad, F, DT_F64, 0, n_o, G, DT_F64, 3, 3, 3, (int)n_o, 1.0, 0.0);
        if (r >= 0) r = gemm1(ctx, DT_F64, F, DT_F64, 1, n_o, Vop, DT_F64, 0, n_o, H, DT_F64, 3, 3, (int)n_p, (int)n_o, 1.0, 0.0);
        if (r < 0) { cleanup(); return r; }
        double g[9];
        hipError_t e = hipMemcpyAsync(g, G, sizeof(g), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "G copy"); }
        // 3 x 3 SPD inverse by Cholesky on the host (the small second POSV of the page)
        double a = g[0], b = g[3], c = g[6], d = g[4], e2 = g[7], f = g[8];
        double l11 = a > 0 ? std::sqrt(a) : NAN;
        double l21 = b / l11, l31 = c / l11;
        double t22 = d - l21 * l21;
        double l22 = t22 > 0 ? std::sqrt(t22) : NAN;
        double l32 = (e2 - l31 * l21) / l22;
        double t33 = f - l31 * l31 - l32 * l32;
        double l33 = t33 > 0 ? std::sqrt(t33) : NAN;
        if (!(l11 > 0 && l22 > 0 && l33 > 0)) {
            *info = -1;
            cleanup();
            return set_err(ctx, GPEX_ERR_NOT_SPD, "gpex_krige: trend system G is not positive definite");
        }
        // Linv (lower) then Ginv = Linv^T Linv
        double i11 = 1 / l11, i22 = 1 / l22, i33 = 1 / l33;
        double i21 = -l21 * i11 * i22, i32 = -l32 * i22 * i33;
        double i31 = -(l31 * i11 + l32 * i21) * i33;
        double Li[3][3] = {{i11, 0, 0}, {i21, i22, 0}, {i31, i32, i33}};
        double Gi[9];
        for (int p = 0; p < 3; ++p)
            for (int q = 0; q < 3; ++q) {
                double acc = 0;
                for (int k = 0; k < 3; ++k) acc += Li[k][p] * Li[k][q];
                Gi[3 * p + q] = acc;
            }
        hipLaunchKernelGGL(k_trend_h, dim3(nblk(n_p)), dim3(256), 0, s, H, d_loc_p, n_p, Gi[0], Gi[1], Gi[2], Gi[3],
                           Gi[4], Gi[5], Gi[6], Gi[7], Gi[8]);
        hipLaunchKernelGGL(k_sub_xh, dim3(nblk(n_o * n_p)), dim3(256), 0, s, d_W, Xo, rows_pad, H, n_o, n_p);
        if (hipGetLastError() != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "trend launch"); }
    }
    // L_o Y = V_op - X_o H;  L_o^T W = Y
    r = tile_trsm(ctx, Sy, d_W, n_o, n_p, 0, tmp, d_tk);
    if (r >= 0) r = tile_trsm(ctx, Sy, d_W, n_o, n_p, 1, tmp, d_tk);
    // zhat = W^T y_o
    if (r >= 0) r = gemm1(ctx, DT_F64, d_W, DT_F64, 1, n_o, d_y_o, DT_F64, 0, n_o, d_zhat, DT_F64, n_p, (int)n_p, 1, (int)n_o, 1.0, 0.0);
    if (r < 0) { cleanup(); return r; }
    hipLaunchKernelGGL(k_mspe, dim3((unsigned)n_p), dim3(256), 0, s, d_W, Vop, Xo, rows_pad, H, k_trend == 3 ? 1 : 0,
                       n_o, n_p, params->sigma2, d_v);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    cleanup();
    if (e != hipSuccess) return set_err(ctx, GPEX_ERR_HIP, std::string("krige: ") + hipGetErrorString(e));
    return GPEX_OK;
}

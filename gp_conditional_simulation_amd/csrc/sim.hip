// Conditional simulation: standard normals, compensated FP16 input, mixed-precision TRMM,
// conditioning, the fused exceedance/extrema scan and the calibration of the regions.
//
// "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets":
//   Algorithm 1 and Eq. 3 (Sec. IV-C): M = L_s B with B = Mrand / s; every right-hand-side tile
//     in FP16; off-diagonal factor tiles converted to FP16 for an FP16 product, the diagonal tile
//     applied in FP32; result in FP64.
//   Sec. V-B (Eq. 7): S = M_p + W^T (y_o 1^T - M_o).
//   Sec. V-C (Eq. 8, 9): A+_j = {S_ij >= u}, A-_j = {S_ij <= u}, psi_j = min over A+_j of t,
//     phi_j = max over A-_j of t, both in one pass; samples sorted separately without the
//     empty-set sentinels; q_out = Q_alpha(psi), q_in = Q_{1-alpha}(phi); C_out = {t >= q_out},
//     C_in = {t > q_in}.
// Normals: Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3") and the
// Box-Muller transform, counter = element pair index, so any block can be regenerated alone.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "devutil.h"

namespace gpex {

__device__ __forceinline__ void philox4x32_10(uint32_t x[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint32_t hi0 = __umulhi(0xD2511F53u, x[0]), lo0 = 0xD2511F53u * x[0];
        uint32_t hi1 = __umulhi(0xCD9E8D57u, x[2]), lo1 = 0xCD9E8D57u * x[2];
        uint32_t n0 = hi1 ^ x[1] ^ k0, n2 = hi0 ^ x[3] ^ k1;
        x[0] = n0; x[1] = lo1; x[2] = n2; x[3] = lo0;
    }
}

__device__ __forceinline__ double u01(uint32_t lo, uint32_t hi) {
    uint64_t w = ((uint64_t)hi << 32) | lo;
    return ((double)(w >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

// The N(0,1) pair p: elements 2p (cosine branch) and 2p + 1 (sine branch) of the linear index.
__device__ __forceinline__ void normal_pair(uint64_t seed, uint32_t stream, uint64_t p, double& z0, double& z1) {
    uint32_t x[4] = {(uint32_t)p, (uint32_t)(p >> 32), stream, 0u};
    philox4x32_10(x, (uint32_t)seed, (uint32_t)(seed >> 32));
    const double u1 = u01(x[0], x[1]), u2 = u01(x[2], x[3]);
    const double rad = sqrt(-2.0 * log(u1));
    double sa, ca;
    sincos(6.283185307179586476925286766559 * u2, &sa, &ca);
    z0 = rad * ca;
    z1 = rad * sa;
}

// One thread per pair: both elements from one generator call (linear index l = j n + i).
__global__ void k_normals(uint64_t seed, uint32_t stream, int64_t n, int64_t nsim, double* Z, int64_t ld) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = n * nsim;
    if (2 * p >= total) return;
    double z[2];
    normal_pair(seed, stream, (uint64_t)p, z[0], z[1]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int64_t l = 2 * p + e;
        if (l < total) Z[l % n + (l / n) * ld] = z[e];
    }
}

// B (rows_pad x cols_pad, leading dim rows_pad): B_ij = Z_ij / s for i < n, j < nsim, stored in
// FP16 (RNE) when amp, else FP64; one thread per element pair of the n x nsim block (linear index
// l = j n + i).  Per-block partial sums of (Z/s)^2 go to part.  The padding is k_zero_pad's.
__global__ __launch_bounds__(256) void k_make_B(const double* Zin, int64_t n, int64_t nsim,
                                                uint64_t seed, int64_t rows_pad, double inv_s, int amp,
                                                void* B, double* part) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = n * nsim;
    double sq = 0.0;
    if (2 * p < total) {
        double z[2];
        if (Zin) {
            z[0] = Zin[2 * p];
            z[1] = 2 * p + 1 < total ? Zin[2 * p + 1] : 0.0;
        } else {
            normal_pair(seed, 0u, (uint64_t)p, z[0], z[1]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t l = 2 * p + e;
            if (l >= total) break;
            const double b = amp ? z[e] * inv_s : z[e];
            sq += b * b;
            const int64_t at = l % n + (l / n) * rows_pad;
            if (amp) static_cast<_Float16*>(B)[at] = f64_to_f16(b);
            else static_cast<double*>(B)[at] = b;
        }
    }
    __shared__ double red[256];
    red[threadIdx.x] = sq;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// Zeros of B outside the n x nsim block: rows [n, rows_pad) of every column and every row of
// columns [nsim, cols_pad).  One thread per element of the padding strip it is launched over.
__global__ void k_zero_pad(int64_t n, int64_t nsim, int64_t rows_pad, int64_t cols_pad, int amp, void* B) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tail_rows = rows_pad - n;                 // strip 1: (rows_pad - n) x nsim
    const int64_t n1 = tail_rows * nsim, n2 = rows_pad * (cols_pad - nsim);
    int64_t at;
    if (idx < n1) at = n + idx % tail_rows + (idx / tail_rows) * rows_pad;
    else if (idx < n1 + n2) at = nsim * rows_pad + (idx - n1);   // strip 2: whole padded columns
    else return;
    if (amp) static_cast<_Float16*>(B)[at] = (_Float16)0.0f;
    else static_cast<double*>(B)[at] = 0.0;
}

// ---- scan ------------------------------------------------------------------------------------
constexpr int SR = 128, SC = 64;   // rows x columns per scan workgroup

// Per workgroup: rows [rb*SR, +SR) x columns [cb*SC, +SC) of S.  Phase 1 (thread = row, half of
// the columns): coalesced column reads, exceedance counts per row (one atomic per row and
// workgroup), >=/<= flags to LDS.  Phase 2 (thread = column, quarter of the rows): min of t over
// the >= set, max over the <= set, size of the >= set -> per-(row block, column) partials.
__global__ __launch_bounds__(256) void k_scan(const double* __restrict__ S, int64_t lds, int64_t np,
                                              int64_t nsim, const double* __restrict__ t, double u,
                                              unsigned long long* __restrict__ counts,
                                              double* __restrict__ psi_part, double* __restrict__ phi_part,
                                              int* __restrict__ size_part) {
    __shared__ uint8_t ge[SR][SC + 1], le[SR][SC + 1];
    __shared__ double ts[SR];
    __shared__ int cnt2[SR];
    __shared__ double red_mn[4][SC], red_mx[4][SC];
    __shared__ int red_sz[4][SC];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * SR, c0 = (int64_t)blockIdx.y * SC;
    {
        int r = tid % SR, half = tid / SR;
        int64_t gr = r0 + r;
        int cnt = 0;
        for (int c = half * (SC / 2); c < (half + 1) * (SC / 2); ++c) {
            int64_t gc = c0 + c;
            uint8_t g = 0, e = 0;
            if (gr < np && gc < nsim) {
                double v = S[gr + gc * lds];
                g = v >= u;
                e = v <= u;
            }
            ge[r][c] = g;
            le[r][c] = e;
            cnt += g;
        }
        if (half == 1) cnt2[r] = cnt;
        if (half == 0) ts[r] = (t && gr < np) ? t[gr] : 0.0;
        __syncthreads();
        if (half == 0 && gr < np) {
            int tot = cnt + cnt2[r];
            if (tot) atomicAdd(&counts[gr], (unsigned long long)tot);
        }
    }
    __syncthreads();
    {
        int c = tid % SC, q = tid / SC;
        double mn = INFINITY, mx = -INFINITY;
        int sz = 0;
        for (int r = q * (SR / 4); r < (q + 1) * (SR / 4); ++r) {
            if (ge[r][c]) {
                sz += 1;
                mn = fmin(mn, ts[r]);
            }
            if (le[r][c]) mx = fmax(mx, ts[r]);
        }
        red_mn[q][c] = mn;
        red_mx[q][c] = mx;
        red_sz[q][c] = sz;
        __syncthreads();
        if (q == 0 && c0 + c < nsim) {
            for (int k = 1; k < 4; ++k) {
                mn = fmin(mn, red_mn[k][c]);
                mx = fmax(mx, red_mx[k][c]);
                sz += red_sz[k][c];
            }
            int64_t o = (int64_t)blockIdx.x * nsim + c0 + c;
            psi_part[o] = mn;
            phi_part[o] = mx;
            size_part[o] = sz;
        }
    }
}

__global__ void k_scan_finish(const double* psi_part, const double* phi_part, const int* size_part,
                              int64_t nrb, int64_t nsim, double* psi, double* phi, int* sizes) {
    int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nsim) return;
    double mn = INFINITY, mx = -INFINITY;
    int sz = 0;
    for (int64_t b = 0; b < nrb; ++b) {
        mn = fmin(mn, psi_part[b * nsim + j]);
        mx = fmax(mx, phi_part[b * nsim + j]);
        sz += size_part[b * nsim + j];
    }
    psi[j] = mn;
    phi[j] = mx;
    sizes[j] = sz;
}

// t = (zhat - u) / sqrt(v) (Eq. 1); a non-positive v raises the MSPE flag.
__global__ void k_tstat(const double* zhat, const double* v, double u, int64_t np, double* t,
                        unsigned long long* flags) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= np) return;
    double vi = v[i];
    if (!(vi > 0.0)) {
        atomicOr(&flags[FLAG_MSPE], 1ull);
        t[i] = NAN;
        return;
    }
    t[i] = (zhat[i] - u) / sqrt(vi);
}

// R = y_o 1^T - M_o (n_o x nsim, leading dim n_o).
__global__ void k_residual(const double* M, int64_t ldm, int64_t np, int64_t no, int64_t nsim,
                           const double* yo, double* R) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= no * nsim) return;
    int64_t r = idx % no, j = idx / no;
    R[idx] = yo[r] - M[np + r + j * ldm];
}

__global__ void k_regions(const double* t, int64_t np, double q_in, double q_out, uint8_t* cin,
                          uint8_t* cout) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= np) return;
    double ti = t[i];
    cout[i] = ti >= q_out;
    cin[i] = ti > q_in;
}

__global__ void k_u64_to_i64(const unsigned long long* a, int64_t* b, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) b[i] = (int64_t)a[i];
}

static unsigned blocks(int64_t n, int t = 256) { return (unsigned)((n + t - 1) / t); }

// Eq. 9 index with p read as a six-place decimal, exact integer ceiling.
static int64_t quantile_index(double p, int64_t n) {
    long long P = std::llround(p * 1e6);
    long long num = P * (long long)n;
    long long k = (num + 999999) / 1000000;
    if (k < 1) k = 1;
    if (k > n) k = n;
    return k;
}

}  // namespace gpex

using namespace gpex;

extern "C" int gpex_normals(gpex_ctx_t ctx, uint64_t seed, uint32_t stream, int64_t n, int64_t nsim,
                            double* d_Z, int64_t ld) {
    if (!ctx) return GPEX_ERR_ARG;
    if (!d_Z || n < 0 || nsim < 0 || ld < n) return set_err(ctx, GPEX_ERR_ARG, "gpex_normals: bad argument");
    if (n * nsim == 0) return GPEX_OK;
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    hipLaunchKernelGGL(k_normals, dim3(blocks((n * nsim + 1) / 2)), dim3(256), 0, ctx->stream, seed, stream, n, nsim,
                       d_Z, ld);
    GPEX_HIP(ctx, hipGetLastError());
    return GPEX_OK;
}

extern "C" int gpex_trmm_sim(gpex_ctx_t ctx, gpex_tiled_t L, int64_t nsim, uint64_t seed, const double* d_Z,
                             double* d_M, int64_t ldm, gpex_diag* diag) {
    if (!ctx) return GPEX_ERR_ARG;
    if (!L || !d_M || nsim < 1 || ldm < (L ? L->n : 0))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_trmm_sim: bad argument (handle, d_M, nsim or ldm)");
    if (!L->factored) return set_err(ctx, GPEX_ERR_STATE, "gpex_trmm_sim: matrix is not factored");
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    hipStream_t s = ctx->stream;
    const int64_t nt = L->nt, nb = L->nb, n = L->n;
    const int64_t rows = nt * nb;
    const int64_t cols = ((nsim + 127) / 128) * 128;
    const int amp = L->opts.amp ? 1 : 0;
    void* B = nullptr;
    double* Mp = nullptr;
    double* part = nullptr;
    GemmTask* d_tasks = nullptr;
    auto cleanup = [&]() { dev_free(d_tasks); };
    const int64_t nblkB = (n * nsim / 2 + 1 + 255) / 256;   // k_make_B: one thread per element pair
    const int64_t npad = (rows - n) * nsim + rows * (cols - nsim);
    auto al256 = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t bB = al256((size_t)rows * cols * (amp ? 2 : 8)), bM = al256(sizeof(double) * rows * cols),
                 bP = al256(sizeof(double) * nblkB);
    int r = GPEX_OK;
    if (ctx->sim_ws_bytes < bB + bM + bP) {   // the previous call has completed: it synchronised
        dev_free(ctx->sim_ws);
        ctx->sim_ws = nullptr;
        ctx->sim_ws_bytes = 0;
        r = dev_alloc(ctx, &ctx->sim_ws, bB + bM + bP, "simulation workspace");
        if (r >= 0) ctx->sim_ws_bytes = bB + bM + bP;
    }
    if (r >= 0) {
        B = ctx->sim_ws;
        Mp = reinterpret_cast<double*>(static_cast<uint8_t*>(ctx->sim_ws) + bB);
        part = reinterpret_cast<double*>(static_cast<uint8_t*>(ctx->sim_ws) + bB + bM);
    }
    // An all-FP64 factor whose tiles of each row are stored back to back (column-major nb x nb
    // tiles with no alignment gap): the off-diagonal tiles of row i then form one column-major
    // nb x (i nb) matrix with leading dimension nb, so the row's whole contribution is one product.
    bool rowpanel64 = !amp && nt > 1;
    for (int64_t i = 1; rowpanel64 && i < nt; ++i)
        for (int64_t j = 0; rowpanel64 && j < i; ++j)
            rowpanel64 = L->prec(i, j) == DT_F64 &&
                         (j == 0 || static_cast<uint8_t*>(L->tile(i, j)) ==
                                        static_cast<uint8_t*>(L->tile(i, j - 1)) + (size_t)nb * nb * 8);
    const bool fused = (amp && L->l16) || rowpanel64;
    // otherwise: off-diagonal tasks for every step, built once and grouped by the factor tile's
    // storage type (one typed kernel per launch)
    struct Group { int64_t b0, b1; };
    std::vector<GemmTask> tasks;
    std::vector<Group> groups;
    std::vector<int64_t> gbeg((size_t)nt + 1, 0);
    for (int64_t k = 0; k < nt && !fused; ++k) {
        gbeg[(size_t)k] = (int64_t)groups.size();
        for (int ta = DT_F64; ta <= DT_F16; ++ta) {
            int64_t b0 = (int64_t)tasks.size();
            for (int64_t i = k + 1; i < nt; ++i) {
                if (L->prec(i, k) != ta) continue;
                GemmTask g{};
                g.A = L->tile(i, k); g.ta = (int8_t)ta; g.lda = nb; g.transA = 0;
                g.B = static_cast<uint8_t*>(B) + (size_t)k * nb * (amp ? 2 : 8); g.tb = amp ? DT_F16 : DT_F64;
                g.ldb = rows; g.transB = 0;
                g.C = Mp + i * nb; g.tc = DT_F64; g.ldc = rows;
                g.M = (int)nb; g.N = (int)cols; g.K = (int)nb;
                g.alpha = 1.0; g.beta = k == 0 ? 0.0 : 1.0;
                tasks.push_back(g);
            }
            if ((int64_t)tasks.size() > b0) groups.push_back(Group{b0, (int64_t)tasks.size()});
        }
    }
    gbeg[(size_t)nt] = (int64_t)groups.size();
    if (r >= 0 && !tasks.empty()) {
        r = dev_alloc(ctx, (void**)&d_tasks, sizeof(GemmTask) * tasks.size(), "trmm tasks");
        if (r >= 0 && hipMemcpy(d_tasks, tasks.data(), sizeof(GemmTask) * tasks.size(), hipMemcpyHostToDevice) != hipSuccess)
            r = set_err(ctx, GPEX_ERR_HIP, "trmm task upload");
    }
    if (r >= 0 && hipMemsetAsync(ctx->d_flags + FLAG_BADTASK, 0, sizeof(long long), s) != hipSuccess)
        r = set_err(ctx, GPEX_ERR_HIP, "trmm flag reset");
    if (r < 0) { cleanup(); return r; }
    hipEvent_t ev[4] = {};
    std::vector<hipEvent_t> kev;
    if (ctx->timing) {
        for (auto& e : ev) (void)hipEventCreate(&e);
        (void)hipEventRecord(ev[0], s);
    }
    hipLaunchKernelGGL(k_make_B, dim3((unsigned)nblkB), dim3(256), 0, s, d_Z, n, nsim, seed, rows,
                       1.0 / L->s, amp, B, part);
    if (npad > 0)
        hipLaunchKernelGGL(k_zero_pad, dim3((unsigned)((npad + 255) / 256)), dim3(256), 0, s, n, nsim, rows, cols, amp, B);
    if (hipGetLastError() != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "make_B launch"); }
    if (ctx->timing) (void)hipEventRecord(ev[1], s);
    if (fused) {
        // diagonal tiles, one launch: FP32 products of cast32(L_kk) and cast32(B_k) (mixed
        // precision) or FP64 products
        std::vector<GemmTask> dg;
        for (int64_t k = 0; k < nt; ++k) {
            GemmTask g{};
            g.A = L->tile(k, k); g.ta = DT_F64; g.lda = nb; g.transA = 0;
            g.B = static_cast<uint8_t*>(B) + (size_t)k * nb * (amp ? 2 : 8); g.tb = amp ? DT_F16 : DT_F64;
            g.ldb = rows; g.transB = 0;
            g.C = Mp + k * nb; g.tc = DT_F64; g.ldc = rows;
            g.M = (int)nb; g.N = (int)cols; g.K = (int)nb;
            g.alpha = 1.0; g.beta = 0.0;
            g.tri = TRI_A_LOWER;   // L_kk is lower triangular
            dg.push_back(g);
        }
        // off-diagonal part of tile row i: one product of the row panel (nb x i nb) with
        // B[0 : i nb], longest rows first: FP16 (the row-major cast16 panels) or FP64 (the tiles)
        std::vector<GemmTask> od;
        for (int64_t i = nt - 1; i >= 1; --i) {
            GemmTask g{};
            if (amp) {
                g.A = L->l16_panel(i); g.ta = DT_F16; g.lda = i * nb; g.transA = 1;
            } else {
                g.A = L->tile(i, 0); g.ta = DT_F64; g.lda = nb; g.transA = 0;
            }
            g.B = B; g.tb = amp ? DT_F16 : DT_F64; g.ldb = rows; g.transB = 0;
            g.C = Mp + i * nb; g.tc = DT_F64; g.ldc = rows;
            g.M = (int)nb; g.N = (int)cols; g.K = (int)(i * nb);
            g.alpha = 1.0; g.beta = 1.0;
            od.push_back(g);
        }
        // Task t of a batched launch runs on XCD t mod 8.  Reversing every second group of eight
        // (a snake order) gives each XCD a near-equal share of the K = i nb work; in plain order
        // XCD 0 gets the longest row of every group (15% above the mean at 98 tile rows).
        for (size_t g0 = 8; g0 < od.size(); g0 += 16)
            std::reverse(od.begin() + (std::ptrdiff_t)g0, od.begin() + (std::ptrdiff_t)std::min(g0 + 8, od.size()));
        GemmTask* d2 = nullptr;
        r = dev_alloc(ctx, (void**)&d2, sizeof(GemmTask) * (dg.size() + od.size()), "trmm panel tasks");
        if (r >= 0 && hipMemcpy(d2, dg.data(), sizeof(GemmTask) * dg.size(), hipMemcpyHostToDevice) != hipSuccess)
            r = set_err(ctx, GPEX_ERR_HIP, "trmm task upload");
        if (r >= 0 && !od.empty() &&
            hipMemcpy(d2 + dg.size(), od.data(), sizeof(GemmTask) * od.size(), hipMemcpyHostToDevice) != hipSuccess)
            r = set_err(ctx, GPEX_ERR_HIP, "trmm task upload");
        if (r >= 0) r = gemm_launch(ctx, s, amp ? DT_F32 : DT_F64, d2, (int)dg.size(), dg[0], GEMM_TRMM);
        if (r >= 0 && !od.empty())
            r = gemm_launch(ctx, s, amp ? DT_F16 : DT_F64, d2 + dg.size(), (int)od.size(), od[0], GEMM_TRMM);
        // d2 is released after the stream synchronisation below
        dev_free(d_tasks);
        d_tasks = d2;
        if (r < 0) { cleanup(); return r; }
    } else {
        for (int64_t k = 0; k < nt; ++k) {
            GemmTask g{};
            g.A = L->tile(k, k); g.ta = DT_F64; g.lda = nb; g.transA = 0;
            g.B = static_cast<uint8_t*>(B) + (size_t)k * nb * (amp ? 2 : 8); g.tb = amp ? DT_F16 : DT_F64;
            g.ldb = rows; g.transB = 0;
            g.C = Mp + k * nb; g.tc = DT_F64; g.ldc = rows;
            g.M = (int)nb; g.N = (int)cols; g.K = (int)nb;
            g.alpha = 1.0; g.beta = k == 0 ? 0.0 : 1.0;
            g.tri = TRI_A_LOWER;   // L_kk is lower triangular
            r = gemm_launch(ctx, s, amp ? DT_F32 : DT_F64, nullptr, 1, g, GEMM_TRMM);
            for (int64_t gi = gbeg[(size_t)k]; r >= 0 && gi < gbeg[(size_t)k + 1]; ++gi) {
                const Group& G = groups[(size_t)gi];
                r = gemm_launch(ctx, s, amp ? DT_F16 : DT_F64, d_tasks + G.b0, (int)(G.b1 - G.b0), tasks[(size_t)G.b0],
                                GEMM_TRMM);
            }
            if (r < 0) { cleanup(); return r; }
        }
    }
    if (ctx->timing) (void)hipEventRecord(ev[2], s);
    r = copy2d(ctx, s, Mp, DT_F64, rows, d_M, DT_F64, ldm, n, nsim, 1.0);
    if (ctx->timing) (void)hipEventRecord(ev[3], s);
    if (r < 0) { cleanup(); return r; }
    long long bad = 0;
    if (diag || ctx->timing) {
        std::vector<double> h((size_t)nblkB);
        hipError_t e = hipMemcpyAsync(h.data(), part, sizeof(double) * nblkB, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipMemcpyAsync(&bad, ctx->d_flags + FLAG_BADTASK, sizeof(long long), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "trmm sync"); }
        double ss = 0.0;
        for (double v : h) ss += v;
        if (diag) {
            *diag = L->diag;
            diag->norm_B = std::sqrt(ss);
        }
        if (ctx->timing) {
            float a = 0, b = 0;
            (void)hipEventElapsedTime(&a, ev[0], ev[3]);
            (void)hipEventElapsedTime(&b, ev[1], ev[2]);
            ctx->timings[10] = a;
            ctx->timings[11] = b;
            for (auto& e2 : ev) (void)hipEventDestroy(e2);
        }
    } else {
        // buffers are freed below; make sure the queued work no longer needs them
        hipError_t e = hipMemcpyAsync(&bad, ctx->d_flags + FLAG_BADTASK, sizeof(long long), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "trmm sync"); }
    }
    cleanup();
    if (bad) return set_err(ctx, GPEX_ERR_STATE, "gpex_trmm_sim: internal task-type mismatch");
    return GPEX_OK;
}

extern "C" int gpex_excursion_regions(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                                      int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                                      const double* d_zhat, const double* d_v, double u, double level_c,
                                      int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                                      uint8_t* d_cin, uint8_t* d_cout, double* d_S, gpex_region_stats* st) {
    if (!ctx) return GPEX_ERR_ARG;
    if (!d_M || n_p < 1 || n_o < 0 || nsim < 1 || ldm < n_p + n_o || !d_counts || !d_sizes)
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: bad sizes or null M/counts/sizes");
    if (n_o > 0 && (!d_W || !d_y_o))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: W and y_o are needed when n_o > 0");
    const bool regions = d_zhat != nullptr;
    if (regions && (!d_v || !h_psi || !h_phi || !d_cin || !d_cout))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: v, psi, phi, cin, cout are needed with zhat");
    if (regions && !(level_c > 0.0 && level_c < 1.0))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: level must lie in (0, 1)");
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    hipStream_t s = ctx->stream;
    auto* fl = reinterpret_cast<unsigned long long*>(ctx->d_flags);
    double *Sbuf = nullptr, *R = nullptr, *t = nullptr, *pp = nullptr, *pq = nullptr, *psi = nullptr, *phi = nullptr;
    int* sp = nullptr;
    unsigned long long* cnt = nullptr;
    auto cleanup = [&]() {
        if (!d_S) dev_free(Sbuf);
        dev_free(R); dev_free(t); dev_free(pp); dev_free(pq); dev_free(psi); dev_free(phi);
        dev_free(sp); dev_free(cnt);
    };
    int r = GPEX_OK;
    const double* S = d_M;
    int64_t lds = ldm;
    if (n_o > 0) {
        if (d_S) Sbuf = d_S;
        else r = dev_alloc(ctx, (void**)&Sbuf, sizeof(double) * n_p * nsim, "S");
        if (r >= 0) r = dev_alloc(ctx, (void**)&R, sizeof(double) * n_o * nsim, "residual");
        if (r >= 0) r = copy2d(ctx, s, d_M, DT_F64, ldm, Sbuf, DT_F64, n_p, n_p, nsim, 1.0);
        if (r >= 0) {
            hipLaunchKernelGGL(k_residual, dim3(blocks(n_o * nsim)), dim3(256), 0, s, d_M, ldm, n_p, n_o, nsim, d_y_o, R);
            if (hipGetLastError() != hipSuccess) r = set_err(ctx, GPEX_ERR_HIP, "residual launch");
        }
        if (r >= 0)
            r = gemm1(ctx, DT_F64, d_W, DT_F64, 1, n_o, R, DT_F64, 0, n_o, Sbuf, DT_F64, n_p,
                      (int)n_p, (int)nsim, (int)n_o, 1.0, 1.0);
        S = Sbuf;
        lds = n_p;
    } else if (d_S) {
        r = copy2d(ctx, s, d_M, DT_F64, ldm, d_S, DT_F64, n_p, n_p, nsim, 1.0);
    }
    const int64_t nrb = (n_p + SR - 1) / SR, ncb = (nsim + SC - 1) / SC;
    if (r >= 0) r = dev_alloc(ctx, (void**)&t, sizeof(double) * n_p, "t");
    if (r >= 0) r = dev_alloc(ctx, (void**)&pp, sizeof(double) * nrb * nsim, "psi partials");
    if (r >= 0) r = dev_alloc(ctx, (void**)&pq, sizeof(double) * nrb * nsim, "phi partials");
    if (r >= 0) r = dev_alloc(ctx, (void**)&sp, sizeof(int) * nrb * nsim, "size partials");
    if (r >= 0) r = dev_alloc(ctx, (void**)&psi, sizeof(double) * nsim, "psi");
    if (r >= 0) r = dev_alloc(ctx, (void**)&phi, sizeof(double) * nsim, "phi");
    if (r >= 0) r = dev_alloc(ctx, (void**)&cnt, sizeof(unsigned long long) * n_p, "counts");
    if (r < 0) { cleanup(); return r; }
    hipError_t e = hipMemsetAsync(cnt, 0, sizeof(unsigned long long) * n_p, s);
    if (e == hipSuccess) e = hipMemsetAsync(ctx->d_flags + FLAG_MSPE, 0, sizeof(long long), s);
    if (e != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "scan setup"); }
    if (regions) hipLaunchKernelGGL(k_tstat, dim3(blocks(n_p)), dim3(256), 0, s, d_zhat, d_v, u, n_p, t, fl);
    hipLaunchKernelGGL(k_scan, dim3((unsigned)nrb, (unsigned)ncb), dim3(256), 0, s, S, lds, n_p, nsim,
                       regions ? t : nullptr, u, cnt, pp, pq, sp);
    hipLaunchKernelGGL(k_scan_finish, dim3(blocks(nsim)), dim3(256), 0, s, pp, pq, sp, nrb, nsim, psi, phi, d_sizes);
    hipLaunchKernelGGL(k_u64_to_i64, dim3(blocks(n_p)), dim3(256), 0, s, cnt, d_counts, n_p);
    if (hipGetLastError() != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "scan launch"); }
    if (!regions) {
        // the temporaries are released below; wait for the queued kernels that read them
        if (hipStreamSynchronize(s) != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "scan sync"); }
        cleanup();
        return GPEX_OK;
    }
    long long mflag = 0;
    e = hipMemcpyAsync(h_psi, psi, sizeof(double) * nsim, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h_phi, phi, sizeof(double) * nsim, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&mflag, ctx->d_flags + FLAG_MSPE, sizeof(long long), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) { cleanup(); return set_err(ctx, GPEX_ERR_HIP, "psi/phi copy"); }
    // host: gather, sort each sample without its sentinel, Eq. 9
    std::vector<double> a, b;
    for (int64_t j = 0; j < nsim; ++j) {
        if (h_psi[j] != INFINITY) a.push_back(h_psi[j]);
        if (h_phi[j] != -INFINITY) b.push_back(h_phi[j]);
    }
    std::sort(a.begin(), a.end());
    std::sort(b.begin(), b.end());
    gpex_region_stats rs{};
    rs.n_psi = (int64_t)a.size();
    rs.n_phi = (int64_t)b.size();
    rs.q_out = rs.q_in = NAN;
    if (mflag) {
        if (st) *st = rs;
        cleanup();
        return set_err(ctx, GPEX_ERR_MSPE_NONPOS, "gpex_excursion_regions: some MSPE v_i <= 0");
    }
    if (a.empty() || b.empty()) {
        if (st) *st = rs;
        cleanup();
        return set_err(ctx, GPEX_ERR_EMPTY_SAMPLE, "gpex_excursion_regions: psi or phi sample is empty");
    }
    double alpha = std::round((1.0 - level_c) * 1e6) / 1e6;
    rs.q_out = a[(size_t)(quantile_index(alpha, rs.n_psi) - 1)];
    rs.q_in = b[(size_t)(quantile_index(1.0 - alpha, rs.n_phi) - 1)];
    hipLaunchKernelGGL(k_regions, dim3(blocks(n_p)), dim3(256), 0, s, t, n_p, rs.q_in, rs.q_out, d_cin, d_cout);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    cleanup();
    if (e != hipSuccess) return set_err(ctx, GPEX_ERR_HIP, "regions");
    if (st) *st = rs;
    return GPEX_OK;
}

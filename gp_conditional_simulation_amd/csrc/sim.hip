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

#include <cstring>
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
        // each 32 x 32 -> 64-bit product in one multiply-add (both halves at once)
        const uint64_t p0 = (uint64_t)0xD2511F53u * x[0], p1 = (uint64_t)0xCD9E8D57u * x[2];
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
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
// FP16 (RNE) when amp, else FP64; element pairs p of the n x nsim block (linear index l = j n + i)
// in a grid-stride loop (at most MAKEB_BLOCKS workgroups, so the per-block partial sums of (Z/s)^2
// in part stay few and k_fold_sum adds them quickly).  The padding is k_zero_pad's.
constexpr int MAKEB_BLOCKS = 8192;
__global__ __launch_bounds__(256) void k_make_B(const double* Zin, int64_t n, int64_t nsim,
                                                uint64_t seed, int64_t rows_pad, double inv_s, int amp,
                                                void* B, double* part, unsigned long long* flags) {
    const int64_t total = n * nsim;
    const bool small = total <= (int64_t)0xffffffff;
    double sq = 0.0;
    bool ovf = false;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 2 * p < total;
         p += (int64_t)gridDim.x * blockDim.x) {
        double z[2];
        if (Zin) {
            z[0] = Zin[2 * p];
            z[1] = 2 * p + 1 < total ? Zin[2 * p + 1] : 0.0;
        } else {
            normal_pair(seed, 0u, (uint64_t)p, z[0], z[1]);
        }
        // row and column of element 2p by one division (32-bit when the block allows), then of 2p + 1
        int64_t col, row;
        if (small) {
            const uint32_t u = (uint32_t)(2 * p), q = u / (uint32_t)n;
            col = q;
            row = (int64_t)(u - q * (uint32_t)n);
        } else {
            col = (2 * p) / n;
            row = 2 * p - col * n;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t l = 2 * p + e;
            if (l >= total) break;
            const double b = amp ? z[e] * inv_s : z[e];
            sq += b * b;
            const int64_t at = row + col * rows_pad;
            if (++row == n) {
                row = 0;
                ++col;
            }
            if (amp) {
                const _Float16 h = f64_to_f16(b);
                ovf |= __builtin_isinf((float)h) && !__builtin_isinf(b);
                static_cast<_Float16*>(B)[at] = h;
            } else {
                static_cast<double*>(B)[at] = b;
            }
        }
    }
    if (ovf) atomicOr(&flags[FLAG_FP16_OVF], 1ull);
    __shared__ double red[256];
    red[threadIdx.x] = sq;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

// Sum of the nblk block partials in a fixed order (one workgroup: thread t adds partials t,
// t + 1024, ... in turn, then a tree), so the result is reproducible; out[0] = the sum.
constexpr int FOLD_THR = 1024;
__global__ __launch_bounds__(FOLD_THR) void k_fold_sum(const double* __restrict__ part, int64_t nblk,
                                                       double* __restrict__ out) {
    __shared__ double red[FOLD_THR];
    double s = 0.0;
    for (int64_t b = threadIdx.x; b < nblk; b += FOLD_THR) s += part[b];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int h = FOLD_THR / 2; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
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
constexpr int SROWS = 256, SCOLS = 64;   // rows of a scan tile (one per thread), columns of a block
constexpr int SCAN_MAX_GROUPS = 256;     // row groups: per-(group, column) partials
constexpr int SBATCH = 16;               // loads in flight per thread

// Workgroup (g, cb) scans the row tiles g, g + G, g + 2G, ... of column block cb (SCOLS columns).
// Phase 1, thread = row: reads the row's SCOLS values of S (each column read by 256 consecutive
// rows: whole cache lines), adds its exceedance count to counts[row] (one atomic per row and
// block) and leaves the >= / <= flags of the row as two 64-bit masks in LDS.  Phase 2, thread =
// (column, quarter of the rows): min of t over the >= rows, max over the <= rows, size of the >=
// set, kept in registers across the group's tiles.  The quarters are folded in order at the end
// and written as the group's partials of each column; k_scan_finish folds the groups.  Rows beyond
// np and columns beyond nsim carry no flags.  sgn = -1 scans -S against -u (the lower excursion
// set by sign reversal; sgn = 1 leaves every value as it is).
__global__ __launch_bounds__(256) void k_scan(const double* __restrict__ S, int64_t lds, int64_t np,
                                              int64_t nsim, const double* __restrict__ t, double sgn, double u, int G,
                                              unsigned long long* __restrict__ counts,
                                              double* __restrict__ psi_part, double* __restrict__ phi_part,
                                              int* __restrict__ size_part) {
    __shared__ uint64_t ge[SROWS], le[SROWS];
    __shared__ double ts[SROWS];
    __shared__ double red_mn[4][SCOLS], red_mx[4][SCOLS];
    __shared__ int red_sz[4][SCOLS];
    const int tid = threadIdx.x;
    const int g = blockIdx.x;
    const int64_t c0 = (int64_t)blockIdx.y * SCOLS;
    const int ncol = (int)(nsim - c0 < SCOLS ? nsim - c0 : SCOLS);
    const int64_t nrt = (np + SROWS - 1) / SROWS;
    const int c = tid % SCOLS, q = tid / SCOLS;
    double mn = INFINITY, mx = -INFINITY;
    int sz = 0;
    for (int64_t rt = g; rt < nrt; rt += G) {
        const int64_t gr = rt * SROWS + tid;
        uint64_t fg = 0, fe = 0;
        if (gr < np) {
            const double* col = S + gr + c0 * lds;
            int cnt = 0;
            // batches of SBATCH loads issued together; a ragged block re-reads its last column
            // (an in-bounds address) instead of branching, and masks those flags off
            for (int cb = 0; cb < SCOLS; cb += SBATCH) {
                double v[SBATCH];
#pragma unroll
                for (int k = 0; k < SBATCH; ++k) v[k] = col[(int64_t)min(cb + k, ncol - 1) * lds];
                const double su = sgn * u;
#pragma unroll
                for (int k = 0; k < SBATCH; ++k) {
                    const bool ok = cb + k < ncol;
                    const double w = sgn * v[k];
                    const bool a = ok && w >= su, b = ok && w <= su;
                    fg |= (uint64_t)a << (cb + k);
                    fe |= (uint64_t)b << (cb + k);
                    cnt += a;
                }
            }
            if (cnt) atomicAdd(&counts[gr], (unsigned long long)cnt);
            ts[tid] = t ? t[gr] : 0.0;
        }
        ge[tid] = fg;
        le[tid] = fe;
        __syncthreads();
#pragma unroll 8
        for (int r = q * (SROWS / 4); r < (q + 1) * (SROWS / 4); ++r) {
            const uint64_t a = ge[r], b = le[r];
            const double tr = ts[r];
            if ((a >> c) & 1u) {
                sz += 1;
                mn = fmin(mn, tr);
            }
            if ((b >> c) & 1u) mx = fmax(mx, tr);
        }
        __syncthreads();
    }
    red_mn[q][c] = mn;
    red_mx[q][c] = mx;
    red_sz[q][c] = sz;
    __syncthreads();
    if (q == 0 && c < ncol) {
        for (int k = 1; k < 4; ++k) {
            mn = fmin(mn, red_mn[k][c]);
            mx = fmax(mx, red_mx[k][c]);
            sz += red_sz[k][c];
        }
        const int64_t o = (int64_t)g * nsim + c0 + c;
        psi_part[o] = mn;
        phi_part[o] = mx;
        size_part[o] = sz;
    }
}

// Column j: fold the G group partials (min, max and integer sums: exact in any order).
__global__ void k_scan_finish(const double* __restrict__ psi_part, const double* __restrict__ phi_part,
                              const int* __restrict__ size_part, int G, int64_t nsim, double* __restrict__ psi,
                              double* __restrict__ phi, int* __restrict__ sizes) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= nsim) return;
    double mn = INFINITY, mx = -INFINITY;
    int sz = 0;
#pragma unroll 8
    for (int b = 0; b < G; ++b) {
        mn = fmin(mn, psi_part[(int64_t)b * nsim + j]);
        mx = fmax(mx, phi_part[(int64_t)b * nsim + j]);
        sz += size_part[(int64_t)b * nsim + j];
    }
    psi[j] = mn;
    phi[j] = mx;
    sizes[j] = sz;
}

// Zero the per-row counts and the MSPE flag.
__global__ void k_scan_init(int64_t* __restrict__ counts, int64_t np, long long* __restrict__ mspe_flag) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < np) counts[i] = 0;
    if (i == 0) *mspe_flag = 0;
}

// Row groups of a scan: enough workgroups to fill the GPU (2048), at most one per row tile and
// at most SCAN_MAX_GROUPS.
static int scan_groups(int64_t np, int64_t nsim) {
    const int64_t nrt = (np + SROWS - 1) / SROWS, ncb = (nsim + SCOLS - 1) / SCOLS;
    int64_t G = (2048 + ncb - 1) / ncb;
    if (G > nrt) G = nrt;
    if (G > SCAN_MAX_GROUPS) G = SCAN_MAX_GROUPS;
    return (int)(G < 1 ? 1 : G);
}

// S (n x m, leading dim n) += g 1^T
__global__ void k_add_rows(double* S, int64_t n, int64_t m, const double* g) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < n * m) S[idx] += g[idx % n];
}


// t = (zhat - u) / sqrt(v) (Eq. 1) of the field times sgn (sgn = -1: -zhat against -u); a
// non-positive v raises the MSPE flag.
__global__ void k_tstat(const double* zhat, const double* v, double sgn, double u, int64_t np, double* t,
                        unsigned long long* flags) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= np) return;
    double vi = v[i];
    if (!(vi > 0.0)) {
        atomicOr(&flags[FLAG_MSPE], 1ull);
        t[i] = NAN;
        return;
    }
    t[i] = (sgn * zhat[i] - sgn * u) / sqrt(vi);
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
    if (L->failed) return set_err(ctx, GPEX_ERR_STATE, "gpex_trmm_sim: the factorization of this matrix failed");
    if (!L->factored) return set_err(ctx, GPEX_ERR_STATE, "gpex_trmm_sim: matrix is not factored");
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    hipStream_t s = ctx->stream;
    const int64_t nt = L->nt, nb = L->nb, n = L->n;
    const int64_t rows = nt * nb;
    const int64_t cols = ((nsim + 127) / 128) * 128;
    const int amp = L->opts.amp ? 1 : 0;
    // FP16 destination storage between the k-tasks of Algorithm 1 (the pages' default path)
    const int emu = amp && L->opts.fp16_dest_emulation ? 1 : 0;
    if (emu && nb % 128 != 0)
        return set_err(ctx, GPEX_ERR_ARG, "gpex_trmm_sim: FP16 destination emulation needs a tile size that is a multiple of 128");
    const int64_t nblkB = std::min<int64_t>((n * nsim / 2 + 1 + 255) / 256, MAKEB_BLOCKS);   // k_make_B workgroups
    const int64_t npad = (rows - n) * nsim + rows * (cols - nsim);
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
    // workspace: the input B (padded to whole tiles and 128-column blocks), the norm partials and
    // the task list; the products write the caller's M directly (rows and columns beyond n and nsim
    // are computed in the padding but not stored)
    const size_t ntask = fused ? (size_t)(2 * nt) : (size_t)(nt * (nt + 1) / 2);
    Carve cv;
    const size_t p_B = cv.add((size_t)rows * cols * (amp ? 2 : 8)), p_part = cv.add(sizeof(double) * (nblkB + 1)),
                 p_tasks = cv.add(sizeof(GemmTask) * ntask);
    void* wsb = nullptr;
    GPEX_TRY(ws_get(ctx, WS_SIM, cv.total, &wsb, "simulation workspace"));
    void* B = cv.get<void>(wsb, p_B);
    double* part = cv.get<double>(wsb, p_part);
    GemmTask* d_tasks = cv.get<GemmTask>(wsb, p_tasks);
    auto* fl = reinterpret_cast<unsigned long long*>(ctx->d_flags);
    const int32_t kround = emu ? (int32_t)nb : 0;

    // B first: the normals run on the device while the host builds and uploads the task list
    GPEX_HIP(ctx, hipMemsetAsync(ctx->d_flags + FLAG_FP16_OVF, 0, sizeof(long long) * (FLAG_BADTASK - FLAG_FP16_OVF + 1), s));
    hipEvent_t ev[6] = {};
    if (ctx->timing) {
        for (size_t q = 0; q < 6; ++q) GPEX_TRY(ctx_timing_event(ctx, q, &ev[q]));
        (void)hipEventRecord(ev[0], s);
    }
    hipLaunchKernelGGL(k_make_B, dim3((unsigned)nblkB), dim3(256), 0, s, d_Z, n, nsim, seed, rows,
                       1.0 / L->s, amp, B, part, fl);
    if (npad > 0)
        hipLaunchKernelGGL(k_zero_pad, dim3((unsigned)((npad + 255) / 256)), dim3(256), 0, s, n, nsim, rows, cols, amp, B);
    GPEX_HIP(ctx, hipGetLastError());

    std::vector<GemmTask> tasks;   // uploaded once; alive until the final synchronisation
    // diagonal tiles: FP32 products of cast32(L_kk) and cast32(B_k) (mixed precision) or FP64
    auto diag_task = [&](int64_t k, double beta) {
        GemmTask g{};
        g.A = L->tile(k, k); g.ta = DT_F64; g.lda = nb; g.transA = 0;
        g.B = static_cast<uint8_t*>(B) + (size_t)k * nb * (amp ? 2 : 8); g.tb = amp ? DT_F16 : DT_F64;
        g.ldb = rows; g.transB = 0;
        g.C = d_M + k * nb; g.tc = DT_F64; g.ldc = ldm;
        g.M = (int)nb; g.N = (int)cols; g.K = (int)nb;
        g.m_store = (int32_t)std::min<int64_t>(nb, n - k * nb); g.n_store = (int32_t)nsim;
        g.alpha = 1.0; g.beta = beta;
        g.tri = TRI_A_LOWER;   // L_kk is lower triangular
        g.kround = kround;     // cast16 of the diagonal product (Algorithm 1)
        return g;
    };
    // p16: a launch of the 256 x 256 row-panel kernel (panel16_launch)
    struct Launch { int64_t b0, b1; int compute; bool p16; };
    std::vector<Launch> launches;
    // Tile row i of the product as one task: the row panel times B[0 : i nb] (off-diagonal tiles):
    // FP16 (the row-major FP16 panels) or FP64 (the tiles).  With `whole`, the FP16 panel's two
    // parts of the diagonal tile join it (K = (i + 2) nb: the last 2 nb values of k are the tile's
    // (hi, lo) slab pairs, both meeting B's rows of tile i), so one launch on the 256 x 256 kernel
    // forms the whole row and stores it once (beta = 0).
    auto row_task = [&](int64_t i, bool whole) {
        GemmTask g{};
        if (amp) {
            g.A = L->l16_panel(i); g.ta = DT_F16; g.lda = L->l16_ld(i); g.transA = 1;
        } else {
            g.A = L->tile(i, 0); g.ta = DT_F64; g.lda = nb; g.transA = 0;
        }
        g.B = B; g.tb = amp ? DT_F16 : DT_F64; g.ldb = rows; g.transB = 0;
        g.C = d_M + i * nb; g.tc = DT_F64; g.ldc = ldm;
        g.M = (int)nb; g.N = (int)cols; g.K = (int)((whole ? i + 2 : i) * nb);
        g.kdup = whole ? (int32_t)nb : 0;
        g.m_store = (int32_t)std::min<int64_t>(nb, n - i * nb); g.n_store = (int32_t)nsim;
        g.alpha = 1.0; g.beta = whole ? 0.0 : 1.0;
        g.kround = kround;   // GEMM16 stores its destination in FP16 after each k-task
        return g;
    };
    const bool whole_rows = fused && amp && !emu && panel16_takes(row_task(nt - 1, true), (int)nt);
    if (fused) {
        if (!whole_rows) {
            for (int64_t k = 0; k < nt; ++k) tasks.push_back(diag_task(k, 0.0));
            launches.push_back(Launch{0, nt, amp ? DT_F32 : DT_F64, false});
        }
        std::vector<GemmTask> od;   // longest rows first
        for (int64_t i = nt - 1; i >= (whole_rows ? 0 : 1); --i) od.push_back(row_task(i, whole_rows));
        // Task t of a batched launch runs on XCD t mod 8.  Reversing every second group of eight
        // (a snake order) gives each XCD a near-equal share of the K = i nb work; in plain order
        // XCD 0 gets the longest row of every group (15% above the mean at 98 tile rows).
        for (size_t g0 = 8; g0 < od.size(); g0 += 16)
            std::reverse(od.begin() + (std::ptrdiff_t)g0, od.begin() + (std::ptrdiff_t)std::min(g0 + 8, od.size()));
        if (!od.empty()) {
            launches.push_back(Launch{(int64_t)tasks.size(), (int64_t)(tasks.size() + od.size()), amp ? DT_F16 : DT_F64,
                                      whole_rows});
            tasks.insert(tasks.end(), od.begin(), od.end());
        }
    } else {
        // per step k: the diagonal tile, then the tiles below it, grouped by the factor tile's
        // storage type (one typed kernel per launch)
        for (int64_t k = 0; k < nt; ++k) {
            tasks.push_back(diag_task(k, k == 0 ? 0.0 : 1.0));
            launches.push_back(Launch{(int64_t)tasks.size() - 1, (int64_t)tasks.size(), amp ? DT_F32 : DT_F64, false});
            for (int ta = DT_F64; ta <= DT_F16; ++ta) {
                const int64_t b0 = (int64_t)tasks.size();
                for (int64_t i = k + 1; i < nt; ++i) {
                    if (L->prec(i, k) != ta) continue;
                    GemmTask g{};
                    g.A = L->tile(i, k); g.ta = (int8_t)ta; g.lda = nb; g.transA = 0;
                    g.B = static_cast<uint8_t*>(B) + (size_t)k * nb * (amp ? 2 : 8); g.tb = amp ? DT_F16 : DT_F64;
                    g.ldb = rows; g.transB = 0;
                    g.C = d_M + i * nb; g.tc = DT_F64; g.ldc = ldm;
                    g.M = (int)nb; g.N = (int)cols; g.K = (int)nb;
                    g.m_store = (int32_t)std::min<int64_t>(nb, n - i * nb); g.n_store = (int32_t)nsim;
                    g.alpha = 1.0; g.beta = k == 0 ? 0.0 : 1.0;
                    tasks.push_back(g);
                }
                if ((int64_t)tasks.size() > b0) launches.push_back(Launch{b0, (int64_t)tasks.size(), amp ? DT_F16 : DT_F64, false});
            }
        }
    }
    if (tasks.size() > ntask) return set_err(ctx, GPEX_ERR_STATE, "gpex_trmm_sim: task count exceeds its workspace");
    GPEX_HIP(ctx, hipMemcpyAsync(d_tasks, tasks.data(), sizeof(GemmTask) * tasks.size(), hipMemcpyHostToDevice, s));
    if (ctx->timing) (void)hipEventRecord(ev[1], s);
    int r = GPEX_OK;
    // the row panels' launch (timed on its own): the last one of the fused product
    const size_t q_rows = fused && launches.size() > (whole_rows ? 0u : 1u) ? launches.size() - 1 : launches.size();
    for (size_t q = 0; q < launches.size() && r >= 0; ++q) {
        const Launch& Lq = launches[q];
        if (ctx->timing && q == q_rows) (void)hipEventRecord(ev[4], s);
        if (Lq.p16)
            r = panel16_launch(ctx, s, d_tasks + Lq.b0, (int)(Lq.b1 - Lq.b0), tasks[(size_t)Lq.b0]);
        else
            r = gemm_launch(ctx, s, Lq.compute, d_tasks + Lq.b0, (int)(Lq.b1 - Lq.b0), tasks[(size_t)Lq.b0], GEMM_TRMM);
        if (ctx->timing && q == q_rows) (void)hipEventRecord(ev[5], s);
    }
    if (ctx->timing) {
        (void)hipEventRecord(ev[2], s);
        (void)hipEventRecord(ev[3], s);
    }
    // ||Z / s||_F^2: the block partials folded on the device in a fixed order, one value back;
    // both readbacks land in the context's pinned words
    double ss = 0.0;
    long long flags[FLAG_COUNT] = {};
    if (diag) hipLaunchKernelGGL(k_fold_sum, dim3(1), dim3(FOLD_THR), 0, s, part, nblkB, part + nblkB);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && diag)
        e = hipMemcpyAsync(ctx->h_ret + FLAG_COUNT, part + nblkB, sizeof(double), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(ctx->h_ret, ctx->d_flags, sizeof(flags), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);   // also keeps `tasks` alive for its upload
    if (e == hipSuccess) {
        std::memcpy(flags, ctx->h_ret, sizeof(flags));
        if (diag) std::memcpy(&ss, ctx->h_ret + FLAG_COUNT, sizeof(double));
    }
    if (r < 0) return r;
    if (e != hipSuccess) return set_err(ctx, GPEX_ERR_HIP, std::string("trmm sync: ") + hipGetErrorString(e));
    if (ctx->timing) {
        float a = 0, b = 0, c = 0;
        (void)hipEventElapsedTime(&a, ev[0], ev[3]);
        (void)hipEventElapsedTime(&b, ev[1], ev[2]);
        if (q_rows < launches.size()) (void)hipEventElapsedTime(&c, ev[4], ev[5]);
        ctx->timings[10] = a;
        ctx->timings[11] = b;
        ctx->timings[18] = c;
        ctx->timings[19] = whole_rows ? 1.0 : 0.0;
    }
    if (diag) {
        *diag = L->diag;
        diag->norm_B = std::sqrt(ss);
        diag->fp16_overflow = flags[FLAG_FP16_OVF] ? 1 : 0;
    }
    if (flags[FLAG_BADTASK]) return set_err(ctx, GPEX_ERR_STATE, "gpex_trmm_sim: internal task-type mismatch");
    if (flags[FLAG_FP16_OVF])
        return set_err(ctx, GPEX_WARN_FP16_OVERFLOW, "gpex_trmm_sim: an entry of Z / s overflowed in FP16");
    return GPEX_OK;
}

// Device temporaries of one gpex_excursion_regions call (S and the residual only when n_o > 0;
// gvec instead of the residual in the residual-free conditioning of the allocation-free variant).
struct ScanMem {
    double *S, *R, *t, *pp, *pq, *psi, *phi;
    int* sp;
    double* gvec;
};

constexpr int SCAN_PIECES = 8;

static void scan_carve(Carve& cv, int64_t n_p, int64_t n_o, int64_t nsim, bool need_S, size_t piece[SCAN_PIECES]) {
    const int G = scan_groups(n_p, nsim);
    piece[0] = cv.add(need_S ? sizeof(double) * n_p * nsim : 0);
    piece[1] = cv.add(n_o > 0 ? sizeof(double) * n_o * nsim : 0);
    piece[2] = cv.add(sizeof(double) * n_p);
    piece[3] = cv.add(sizeof(double) * G * nsim);
    piece[4] = cv.add(sizeof(double) * G * nsim);
    piece[5] = cv.add(sizeof(int) * G * nsim);
    piece[6] = cv.add(sizeof(double) * nsim);
    piece[7] = cv.add(sizeof(double) * nsim);
}

static ScanMem scan_mem(const Carve& cv, void* base, const size_t piece[SCAN_PIECES]) {
    ScanMem m{};
    m.S = cv.get<double>(base, piece[0]);
    m.R = cv.get<double>(base, piece[1]);
    m.t = cv.get<double>(base, piece[2]);
    m.pp = cv.get<double>(base, piece[3]);
    m.pq = cv.get<double>(base, piece[4]);
    m.sp = cv.get<int>(base, piece[5]);
    m.psi = cv.get<double>(base, piece[6]);
    m.phi = cv.get<double>(base, piece[7]);
    return m;
}

static int excursion_check(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p, int64_t n_o, int64_t nsim,
                           const double* d_W, const double* d_y_o, const double* d_zhat, const double* d_v,
                           double level_c, int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                           uint8_t* d_cin, uint8_t* d_cout) {
    if (!d_M || n_p < 1 || n_o < 0 || nsim < 1 || ldm < n_p + n_o || !d_counts || !d_sizes)
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: bad sizes or null M/counts/sizes");
    if (n_o > 0 && (!d_W || !d_y_o))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: W and y_o are needed when n_o > 0");
    if (d_zhat && (!d_v || !h_psi || !h_phi || !d_cin || !d_cout))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: v, psi, phi, cin, cout are needed with zhat");
    if (d_zhat && !(level_c > 0.0 && level_c < 1.0))
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions: level must lie in (0, 1)");
    return GPEX_OK;
}

// Conditioning, scan and calibration on the temporaries m (S and R used only when n_o > 0 and,
// for S, d_S is NULL).
static int excursion_run(gpex_ctx_t ctx, const ScanMem& m, const double* d_M, int64_t ldm, int64_t n_p, int64_t n_o,
                         int64_t nsim, const double* d_W, const double* d_y_o, const double* d_zhat,
                         const double* d_v, double u, double level_c, int64_t* d_counts, int32_t* d_sizes,
                         double* h_psi, double* h_phi, uint8_t* d_cin, uint8_t* d_cout, double* d_S,
                         gpex_region_stats* st, double sgn) {
    hipStream_t s = ctx->stream;
    auto* fl = reinterpret_cast<unsigned long long*>(ctx->d_flags);
    const bool regions = d_zhat != nullptr;
    const double* S = d_M;
    int64_t lds = ldm;
    if (n_o > 0 && m.gvec) {
        // residual-free Eq. 7 (no n_o x nsim temporary): S = M_p - W^T M_o, then S += (W^T y_o) 1^T
        GPEX_TRY(copy2d(ctx, s, d_M, DT_F64, ldm, d_S, DT_F64, n_p, n_p, nsim, 1.0));
        GPEX_TRY(gemm1(ctx, DT_F64, d_W, DT_F64, 1, n_o, d_M + n_p, DT_F64, 0, ldm, d_S, DT_F64, n_p, (int)n_p,
                       (int)nsim, (int)n_o, -1.0, 1.0));
        GPEX_TRY(gemm1(ctx, DT_F64, d_W, DT_F64, 1, n_o, d_y_o, DT_F64, 0, n_o, m.gvec, DT_F64, n_p, (int)n_p, 1,
                       (int)n_o, 1.0, 0.0));
        hipLaunchKernelGGL(k_add_rows, dim3(blocks(n_p * nsim)), dim3(256), 0, s, d_S, n_p, nsim, m.gvec);
        GPEX_HIP(ctx, hipGetLastError());
        S = d_S;
        lds = n_p;
    } else if (n_o > 0) {
        double* Sbuf = d_S ? d_S : m.S;
        GPEX_TRY(copy2d(ctx, s, d_M, DT_F64, ldm, Sbuf, DT_F64, n_p, n_p, nsim, 1.0));
        hipLaunchKernelGGL(k_residual, dim3(blocks(n_o * nsim)), dim3(256), 0, s, d_M, ldm, n_p, n_o, nsim, d_y_o, m.R);
        GPEX_HIP(ctx, hipGetLastError());
        GPEX_TRY(gemm1(ctx, DT_F64, d_W, DT_F64, 1, n_o, m.R, DT_F64, 0, n_o, Sbuf, DT_F64, n_p, (int)n_p, (int)nsim,
                       (int)n_o, 1.0, 1.0));
        S = Sbuf;
        lds = n_p;
    } else if (d_S) {
        GPEX_TRY(copy2d(ctx, s, d_M, DT_F64, ldm, d_S, DT_F64, n_p, n_p, nsim, 1.0));
    }
    const int G = scan_groups(n_p, nsim);
    const int64_t ncb = (nsim + SCOLS - 1) / SCOLS;
    hipLaunchKernelGGL(k_scan_init, dim3(blocks(n_p)), dim3(256), 0, s, d_counts, n_p, ctx->d_flags + FLAG_MSPE);
    if (regions) hipLaunchKernelGGL(k_tstat, dim3(blocks(n_p)), dim3(256), 0, s, d_zhat, d_v, sgn, u, n_p, m.t, fl);
    hipLaunchKernelGGL(k_scan, dim3((unsigned)G, (unsigned)ncb), dim3(256), 0, s, S, lds, n_p, nsim,
                       regions ? m.t : nullptr, sgn, u, G, reinterpret_cast<unsigned long long*>(d_counts), m.pp, m.pq,
                       m.sp);
    hipLaunchKernelGGL(k_scan_finish, dim3(blocks(nsim)), dim3(256), 0, s, m.pp, m.pq, m.sp, G, nsim, m.psi, m.phi,
                       d_sizes);
    GPEX_HIP(ctx, hipGetLastError());
    if (!regions) return GPEX_OK;   // counts and sizes are queued on the context stream
    long long mflag = 0;
    hipError_t e = hipMemcpyAsync(h_psi, m.psi, sizeof(double) * nsim, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h_phi, m.phi, sizeof(double) * nsim, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipMemcpyAsync(&mflag, ctx->d_flags + FLAG_MSPE, sizeof(long long), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return set_err(ctx, GPEX_ERR_HIP, "psi/phi copy");
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
        return set_err(ctx, GPEX_ERR_MSPE_NONPOS, "gpex_excursion_regions: some MSPE v_i <= 0");
    }
    if (a.empty() || b.empty()) {
        if (st) *st = rs;
        return set_err(ctx, GPEX_ERR_EMPTY_SAMPLE, "gpex_excursion_regions: psi or phi sample is empty");
    }
    double alpha = std::round((1.0 - level_c) * 1e6) / 1e6;
    rs.q_out = a[(size_t)(quantile_index(alpha, rs.n_psi) - 1)];
    rs.q_in = b[(size_t)(quantile_index(1.0 - alpha, rs.n_phi) - 1)];
    hipLaunchKernelGGL(k_regions, dim3(blocks(n_p)), dim3(256), 0, s, m.t, n_p, rs.q_in, rs.q_out, d_cin, d_cout);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return set_err(ctx, GPEX_ERR_HIP, "regions");
    if (st) *st = rs;
    return GPEX_OK;
}

static int excursion_regions(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p, int64_t n_o,
                             int64_t nsim, const double* d_W, const double* d_y_o, const double* d_zhat,
                             const double* d_v, double u, double level_c, int64_t* d_counts, int32_t* d_sizes,
                             double* h_psi, double* h_phi, uint8_t* d_cin, uint8_t* d_cout, double* d_S,
                             gpex_region_stats* st, double sgn) {
    if (!ctx) return GPEX_ERR_ARG;
    GPEX_TRY(excursion_check(ctx, d_M, ldm, n_p, n_o, nsim, d_W, d_y_o, d_zhat, d_v, level_c, d_counts, d_sizes,
                             h_psi, h_phi, d_cin, d_cout));
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    Carve cv;
    size_t piece[SCAN_PIECES];
    scan_carve(cv, n_p, n_o, nsim, n_o > 0 && !d_S, piece);
    void* wsb = nullptr;
    GPEX_TRY(ws_get(ctx, WS_SCAN, cv.total, &wsb, "scan workspace"));
    return excursion_run(ctx, scan_mem(cv, wsb, piece), d_M, ldm, n_p, n_o, nsim, d_W, d_y_o, d_zhat, d_v, u, level_c,
                         d_counts, d_sizes, h_psi, h_phi, d_cin, d_cout, d_S, st, sgn);
}

extern "C" int gpex_excursion_regions(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                                      int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                                      const double* d_zhat, const double* d_v, double u, double level_c,
                                      int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                                      uint8_t* d_cin, uint8_t* d_cout, double* d_S, gpex_region_stats* st) {
    return excursion_regions(ctx, d_M, ldm, n_p, n_o, nsim, d_W, d_y_o, d_zhat, d_v, u, level_c, d_counts, d_sizes,
                             h_psi, h_phi, d_cin, d_cout, d_S, st, 1.0);
}

// The lower excursion set {y <= u} by sign reversal: the same computation on -S, -u and -zhat.
extern "C" int gpex_excursion_regions_below(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                                            int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                                            const double* d_zhat, const double* d_v, double u, double level_c,
                                            int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                                            uint8_t* d_cin, uint8_t* d_cout, double* d_S, gpex_region_stats* st) {
    return excursion_regions(ctx, d_M, ldm, n_p, n_o, nsim, d_W, d_y_o, d_zhat, d_v, u, level_c, d_counts, d_sizes,
                             h_psi, h_phi, d_cin, d_cout, d_S, st, -1.0);
}

// Allocation-free variant: the temporaries live in the library's fixed per-GPU scratch array and
// the conditioning runs without the n_o x nsim residual.
extern "C" int gpex_excursion_regions_noalloc(gpex_ctx_t ctx, const double* d_M, int64_t ldm, int64_t n_p,
                                              int64_t n_o, int64_t nsim, const double* d_W, const double* d_y_o,
                                              const double* d_zhat, const double* d_v, double u, double level_c,
                                              int64_t* d_counts, int32_t* d_sizes, double* h_psi, double* h_phi,
                                              uint8_t* d_cin, uint8_t* d_cout, double* d_S,
                                              gpex_region_stats* st) {
    if (!ctx) return GPEX_ERR_ARG;
    GPEX_TRY(excursion_check(ctx, d_M, ldm, n_p, n_o, nsim, d_W, d_y_o, d_zhat, d_v, level_c, d_counts, d_sizes,
                             h_psi, h_phi, d_cin, d_cout));
    if (n_o > 0 && !d_S)
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions_noalloc: d_S is needed when n_o > 0");
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    void* base = scratch_ptr(ctx->device);
    if (!base) return set_err(ctx, GPEX_ERR_STATE, "gpex_excursion_regions_noalloc: no scratch on this device");
    Carve cv;
    size_t piece[SCAN_PIECES];
    scan_carve(cv, n_p, 0, nsim, false, piece);   // t, partials, psi, phi
    const size_t p_g = cv.add(n_o > 0 ? sizeof(double) * n_p : 0);
    if (cv.total > SCRATCH_BYTES)
        return set_err(ctx, GPEX_ERR_ARG, "gpex_excursion_regions_noalloc: needs " + std::to_string(cv.total) +
                                              " bytes of scratch, the maximum is " + std::to_string(SCRATCH_BYTES));
    ScanMem m = scan_mem(cv, base, piece);
    m.S = nullptr;
    m.R = nullptr;
    m.gvec = n_o > 0 ? cv.get<double>(base, p_g) : nullptr;
    // the conditioning product stays on the context stream (no side stream to create)
    const bool serial = ctx->serial;
    ctx->serial = true;
    const int r = excursion_run(ctx, m, d_M, ldm, n_p, n_o, nsim, d_W, d_y_o, d_zhat, d_v, u, level_c, d_counts,
                                d_sizes, h_psi, h_phi, d_cin, d_cout, d_S, st, 1.0);
    ctx->serial = serial;
    return r;
}

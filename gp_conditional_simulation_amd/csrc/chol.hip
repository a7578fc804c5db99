// Adaptive mixed-precision tile Cholesky on one MI355X.
//
// "Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets",
// Sec. IV-B and Algorithm 2 (step 12): the scaled covariance s^2 V, cut into nb x nb tiles with a
// per-tile precision map, is factored right-looking.  Step k:
//   * diagonal tile (k, k): FP64 POTRF.  Here it is factored together with its explicit inverse
//     T_k = L_kk^-1 by recursive halving down to leaves of order <= 128 (factor and inverse in one
//     pass of one workgroup); the halves are joined with FP64 matrix-core GEMMs.
//   * panel tiles (i, k), i > k: L_ik = A_ik L_kk^-T evaluated as the product A_ik T_k^T on FP64
//     matrix cores for every tile and rounded once to the tile's storage precision (one batched
//     launch).  An FP32 product through the explicit inverse carries an error of about
//     kappa(L_kk) u_32 and, on strongly correlated covariances, costs positive definiteness.
//   * trailing tiles (i, j), k < j <= i: A_ij -= L_ik L_jk^T in the precision of A_ij with the
//     operands converted to it (FP16 on FP16 matrix cores with FP32 accumulation), one batched
//     launch per compute precision; diagonal tiles (the SYRK tasks) are FP64.  The conversions
//     are done once: the panel solve writes an FP32 / FP64 copy of each panel tile that feeds
//     FP32 / FP64 outputs of another precision, and FP16 outputs read the row-major FP16 copy
//     of the factor (k contiguous), so every update reads operands of its own type.
// The T_k are kept in the handle: kriging reuses them for its blocked triangular solves.
#include <algorithm>
#include <cmath>
#include <map>

#include "common.h"
#include "devutil.h"

namespace gpex {

// ---------------------------------------------------------------------------------------------
__global__ void k_copy2d(const void* src, int tsrc, int64_t lds, void* dst, int tdst, int64_t ldd,
                         int64_t rows, int64_t cols, double scale, unsigned long long* flags) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t c = blockIdx.y;
    bool ovf = false;
    for (; c < cols; c += gridDim.y) {
        if (r < rows) {
            double v = load_as_double(src, tsrc, r + c * lds);
            if (scale != 1.0) v *= scale;
            ovf |= store_from_double(dst, tdst, r + c * ldd, v);
        }
    }
    if (ovf && flags) atomicOr(&flags[FLAG_FP16_OVF], 1ull);
}

int copy2d(gpex_ctx_t ctx, hipStream_t s, const void* src, int tsrc, int64_t lds, void* dst,
           int tdst, int64_t ldd, int64_t rows, int64_t cols, double scale) {
    if (rows <= 0 || cols <= 0) return GPEX_OK;
    dim3 grid((unsigned)((rows + 255) / 256), (unsigned)std::min<int64_t>(cols, 65535));
    hipLaunchKernelGGL(k_copy2d, grid, dim3(256), 0, s, src, tsrc, lds, dst, tdst, ldd, rows, cols,
                       scale, reinterpret_cast<unsigned long long*>(ctx->d_flags));
    GPEX_HIP(ctx, hipGetLastError());
    return GPEX_OK;
}

__global__ void k_zero2d(double* dst, int64_t ldd, int64_t rows, int64_t cols) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t c = blockIdx.y; c < cols; c += gridDim.y)
        if (r < rows) dst[r + c * ldd] = 0.0;
}

int zero2d(gpex_ctx_t ctx, hipStream_t s, double* dst, int64_t ldd, int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return GPEX_OK;
    dim3 grid((unsigned)((rows + 255) / 256), (unsigned)std::min<int64_t>(cols, 65535));
    hipLaunchKernelGGL(k_zero2d, grid, dim3(256), 0, s, dst, ldd, rows, cols);
    GPEX_HIP(ctx, hipGetLastError());
    return GPEX_OK;
}

// Batched raw byte copy: task q copies bytes[q] bytes (a multiple of 16) from src[q] to dst[q].
struct CopyTask {
    const void* src;
    void* dst;
    int64_t bytes;
};

__global__ void k_copy_tasks(const CopyTask* tasks, int64_t chunk) {
    const CopyTask& T = tasks[blockIdx.y];
    int64_t beg = (int64_t)blockIdx.x * chunk;
    int64_t end = beg + chunk < T.bytes ? beg + chunk : T.bytes;
    const uint4* s = static_cast<const uint4*>(T.src);
    uint4* d = static_cast<uint4*>(T.dst);
    for (int64_t i = beg / 16 + threadIdx.x; i < end / 16; i += blockDim.x) d[i] = s[i];
}

// ---------------------------------------------------------------------------------------------
// Leaf: factor an n x n (n <= 128) FP64 block and invert its factor in one pass of one
// workgroup of 512 threads (two waves per SIMD, so that one wave's LDS and pivot latencies hide
// behind the other's arithmetic).  The block is a 16 x 32 grid of 8 x 4 sub-blocks, thread
// (bi, bj) = (t / 32, t % 32) holding sub-block (bi, bj) in registers; rows and columns n..127
// are identity padding.  Column k of the register block is the Schur complement of A while k is
// ahead of the current step and becomes column k of X = L^-1 once step k has passed, so the
// factor and its inverse share one set of registers.
// Column k of the Schur complement is published before step k with its pivot a_kk in a slot of
// its own and zeros on and above the diagonal, so that no update needs a mask.  Step k (one
// barrier, which orders LDS only):
//   * X update of column k - 1 (right-looking on L X = I): X_ij -= l_i,k-1 X_k-1,j, i > k - 1.
//   * Pivot: 1 / l_kk from the hardware reciprocal square root and two Newton steps.
//   * Schur update a_ij -= (a_ik / a_kk) a_jk for i, j > k; column k + 1 is updated first and
//     published by its owners.
//   * Owners of column k reset it to e_k (its X part); owners of row k scale X_k,j (j <= k) by
//     1 / l_kk and publish the row; threads 0..127 store column k of L = a_ik / l_kk to A.
// LDS holds only the published columns (three in flight) and rows (two), and the registers are
// capped at 128 per thread, so the kernel fits in the registers and LDS one trailing-update
// workgroup frees and can run beside the update kernel on the look-ahead stream.  Writes L
// (upper part zeroed) to A and L^-1 (upper part zeroed) to T.  A non-positive pivot at local
// column k records col0 + k + 1 in flags[FLAG_INFO] unless an earlier failure is recorded.
constexpr int LEAF = 128;
constexpr int LEAF_BR = 8, LEAF_BC = 4;                          // sub-block rows x columns
constexpr int LEAF_GC = LEAF / LEAF_BC;                          // sub-block columns
constexpr int LEAF_THREADS = (LEAF / LEAF_BR) * LEAF_GC;         // 512

// Workgroup barrier that orders LDS accesses only.  The leaf's global stores of L need no
// ordering against the other threads, and a full barrier would wait for them at every column.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ __launch_bounds__(LEAF_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4)))
void k_potrf_leaf(double* A, int64_t lda, double* T, int64_t ldt, int n, int64_t col0, unsigned long long* flags) {
    __shared__ __attribute__((aligned(16))) double Lc[3][LEAF];   // a_ik below the diagonal, column k in slot k % 3
    __shared__ double Pv[3];                                      // a_kk in slot k % 3
    __shared__ __attribute__((aligned(16))) double Xr[2][LEAF];   // row k of X (zero beyond k) in slot k % 2
    const int t = threadIdx.x, bi = t / LEAF_GC, bj = t % LEAF_GC;
    const int r0 = bi * LEAF_BR, c0 = bj * LEAF_BC;
    double y[LEAF_BR][LEAF_BC];
#pragma unroll
    for (int a = 0; a < LEAF_BR; ++a)
#pragma unroll
        for (int b = 0; b < LEAF_BC; ++b) {
            const int i = r0 + a, j = c0 + b;
            y[a][b] = (j <= i && i < n) ? A[i + (int64_t)j * lda] : (i == j ? 1.0 : 0.0);
        }
    if (bj == 0) {
#pragma unroll
        for (int a = 0; a < LEAF_BR; ++a) Lc[0][r0 + a] = r0 + a > 0 ? y[a][0] : 0.0;
        if (bi == 0) Pv[0] = y[0][0];
    }
    __syncthreads();
    const int nkg = (n + 7) / 8;   // groups of 8 columns: one sub-block row, two sub-block columns
    double rlp = 0.0;              // 1 / l_k-1,k-1
    int bad = 0;
    for (int kg = 0; kg < nkg && !bad; ++kg) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int k = kg * 8 + kk;
            const int cb = kg * 2 + kk / LEAF_BC, cc = kk % LEAF_BC;   // sub-block column of k, local column
            const double* lc = Lc[k % 3];
            if (k > 0) {   // X update of column k - 1: independent of this step's pivot
                const double* lp = Lc[(k + 2) % 3];
                const double* xp = Xr[(k + 1) & 1];
                double u[LEAF_BR], v[LEAF_BC];
#pragma unroll
                for (int a = 0; a < LEAF_BR; ++a) u[a] = lp[r0 + a] * rlp;
#pragma unroll
                for (int b = 0; b < LEAF_BC; ++b) v[b] = xp[c0 + b];
#pragma unroll
                for (int a = 0; a < LEAF_BR; ++a)
#pragma unroll
                    for (int b = 0; b < LEAF_BC; ++b) y[a][b] = fma(-u[a], v[b], y[a][b]);
            }
            const double akk = Pv[k % 3];   // the same value in every thread: a uniform decision
            if (!(akk > 0.0)) {
                bad = k + 1;
                break;
            }
            double rl = __builtin_amdgcn_rsq(akk);   // refined to 1 / sqrt(a_kk) by two Newton steps
            rl = fma(0.5 * rl, fma(-akk * rl, rl, 1.0), rl);
            rl = fma(0.5 * rl, fma(-akk * rl, rl, 1.0), rl);
            const double lkk = akk * rl, rk = rl * rl;
            // Schur update with column k; column k + 1 first, then published
            double u[LEAF_BR], v[LEAF_BC];
#pragma unroll
            for (int a = 0; a < LEAF_BR; ++a) u[a] = lc[r0 + a] * rk;
#pragma unroll
            for (int b = 0; b < LEAF_BC; ++b) v[b] = lc[c0 + b];
            const int cbn = kg * 2 + (kk + 1) / LEAF_BC, ccn = (kk + 1) % LEAF_BC;   // column k + 1
            const int rbn = kg + (kk == 7 ? 1 : 0), ran = (kk + 1) % 8;              // row k + 1
#pragma unroll
            for (int a = 0; a < LEAF_BR; ++a) y[a][ccn] = fma(-u[a], v[ccn], y[a][ccn]);
            if (bj == cbn) {
#pragma unroll
                for (int a = 0; a < LEAF_BR; ++a) Lc[(k + 1) % 3][r0 + a] = r0 + a > k + 1 ? y[a][ccn] : 0.0;
                if (bi == rbn) Pv[(k + 1) % 3] = y[ran][ccn];
            }
#pragma unroll
            for (int a = 0; a < LEAF_BR; ++a)
#pragma unroll
                for (int b = 0; b < LEAF_BC; ++b)
                    if (b != ccn) y[a][b] = fma(-u[a], v[b], y[a][b]);
            if (bj == cb) {   // column k of X starts as e_k
#pragma unroll
                for (int a = 0; a < LEAF_BR; ++a) y[a][cc] = r0 + a == k ? 1.0 : 0.0;
            }
            if (bi == kg) {   // row k of X is final up to the division by l_kk
#pragma unroll
                for (int b = 0; b < LEAF_BC; ++b) {
                    y[kk][b] *= rl;
                    Xr[k & 1][c0 + b] = c0 + b <= k ? y[kk][b] : 0.0;
                }
            }
            if (t < n && k < n) A[t + (int64_t)k * lda] = t == k ? lkk : lc[t] * rl;   // column k of L
            rlp = rl;
            lds_barrier();
        }
    }
    if (bad) {
        if (t == 0 && flags) atomicCAS(&flags[FLAG_INFO], 0ull, (unsigned long long)(col0 + bad));
        return;
    }
#pragma unroll
    for (int a = 0; a < LEAF_BR; ++a)
#pragma unroll
        for (int b = 0; b < LEAF_BC; ++b) {
            const int i = r0 + a, j = c0 + b;
            if (i < n && j < n) T[i + (int64_t)j * ldt] = j <= i ? y[a][b] : 0.0;
        }
}

// End of a halving step: L21 (n2 x n1 in ws, leading dimension n2) into A21, and zeros in the
// upper-right n1 x n2 blocks of the factor and of its inverse.  blockIdx.y picks the region.
__global__ void k_join(const double* ws, double* A, int64_t lda, double* T, int64_t ldt, int n1, int n2) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n1 * n2) return;
    if (blockIdx.y == 0) {
        const int64_t r = idx % n2, c = idx / n2;                    // L21(r, c)
        A[n1 + r + c * lda] = ws[idx];
    } else {
        const int64_t r = idx % n1, c = n1 + idx / n1;               // upper-right (r, c)
        if (blockIdx.y == 1) A[r + c * lda] = 0.0;
        else T[r + c * ldt] = 0.0;
    }
}

// The diagonal tiles of the factor as two FP16 parts each, for the simulation product: row r of
// tile k goes to row r of FP16 row panel k (leading dimension (k + 2) nb), hi = cast16(L) and
// lo = cast16(L - hi), zeros above the diagonal, in pairs of w-wide slabs from column k nb
// (w = l16_pair_w(nb): column c's hi at k nb + 2 w (c / w) + c % w, its lo w further).  hi + lo
// carries L to about 22 bits (an FP32 copy: 24), and the simulation product takes both on its
// FP16 matrix cores against the same rows of Z / s.  One workgroup per 64 x 64 part of a tile
// (blockIdx.z = k), through LDS: column-major reads, row-major writes.
constexpr int D16_T = 64;
__global__ __launch_bounds__(256) void k_diag16(const uint8_t* const* tiles, int nb, _Float16* l16,
                                                unsigned long long* flags) {
    __shared__ double t[D16_T][D16_T + 1];
    const int k = blockIdx.z, r0 = blockIdx.y * D16_T, c0 = blockIdx.x * D16_T;
    const double* L = reinterpret_cast<const double*>(tiles[k]);
    const int tx = threadIdx.x % D16_T, ty = threadIdx.x / D16_T;
    for (int c = ty; c < D16_T; c += 4) {   // t[row][col], column-major reads
        const int gr = r0 + tx, gc = c0 + c;
        t[tx][c] = (gr < nb && gc < nb && gc <= gr) ? L[gr + (int64_t)gc * nb] : 0.0;
    }
    __syncthreads();
    const int64_t ld = (int64_t)(k + 2) * nb;
    _Float16* panel = l16 + (size_t)nb * nb * (size_t)((int64_t)k * (k - 1) / 2 + 2 * (int64_t)k);
    const int w = l16_pair_w(nb);
    bool ovf = false;
    for (int r = ty; r < D16_T; r += 4) {   // row-major writes
        const int gr = r0 + r, gc = c0 + tx;
        if (gr >= nb || gc >= nb) continue;
        const double v = t[r][tx];
        const _Float16 hi = f64_to_f16(v);
        const _Float16 lo = f64_to_f16(v - (double)hi);
        if (__builtin_isinf((float)hi) && !__builtin_isinf(v)) ovf = true;
        _Float16* at = panel + gr * ld + (int64_t)k * nb + 2 * w * (gc / w) + gc % w;
        at[0] = hi;
        at[w] = lo;
    }
    if (ovf && flags) atomicOr(&flags[FLAG_FP16_OVF], 1ull);
}

// Size of the first half when a diagonal block of order n > LEAF is split: whole leaves first
// (a multiple of LEAF, half of ceil(n / LEAF) leaves), so the recursion ends in the fewest leaves
// ceil(n / LEAF) and the fewest halving steps; orders that are multiples of 2 LEAF halve exactly.
static int split_first(int n) { return LEAF * (((n + LEAF - 1) / LEAF) / 2); }

// Footprint in doubles of the workspace potrf_inv uses for order n: n^2 / 2 (rounded up).
static int64_t potrf_ws_need(int n) {
    if (n <= LEAF) return 0;
    const int n1 = split_first(n), n2 = n - n1;
    const int64_t blk = (int64_t)n2 * n1;
    return std::max(blk, potrf_ws_need(n2)) + blk;
}

// Factor of the n x n diagonal block A and its inverse T by recursive halving.  Each step:
//   ws   = A21 T11^T           (L21)
//   A22 -= ws ws^T
//   wsb  = ws T11              (kept past the second half: placed beyond its footprint)
//   join: A21 = ws, upper-right blocks of A and T zeroed
//   second half on A22
//   T21  = -T22 wsb
// ws holds potrf_ws_need(n) doubles (n^2 / 2 suffice).
int potrf_inv(gpex_ctx_t ctx, hipStream_t s, double* A, int64_t lda, double* T, int64_t ldt, int n,
              double* ws, int64_t col0) {
    auto* fl = reinterpret_cast<unsigned long long*>(ctx->d_flags);
    if (n <= LEAF) {
        hipLaunchKernelGGL(k_potrf_leaf, dim3(1), dim3(LEAF_THREADS), 0, s, A, lda, T, ldt, n, col0, fl);
        GPEX_HIP(ctx, hipGetLastError());
        return GPEX_OK;
    }
    const int n1 = split_first(n), n2 = n - n1;
    double* A21 = A + n1;
    double* A22 = A + n1 + (int64_t)n1 * lda;
    double* T21 = T + n1;
    double* T22 = T + n1 + (int64_t)n1 * ldt;
    const int64_t blk = (int64_t)n2 * n1;
    double* wsb = ws + std::max(blk, potrf_ws_need(n2));
    auto g = [&](const void* a, int tA, int64_t la, const void* b, int tB, int64_t lb, void* c,
                 int64_t lc, int M, int N, int K, double al, double be, int tri) {
        GemmTask t{};
        t.A = a; t.B = b; t.C = c; t.lda = la; t.ldb = lb; t.ldc = lc;
        t.M = M; t.N = N; t.K = K; t.ta = DT_F64; t.tb = DT_F64; t.tc = DT_F64;
        t.transA = (int8_t)tA; t.transB = (int8_t)tB; t.alpha = al; t.beta = be; t.tri = (int8_t)tri;
        return gemm_launch(ctx, s, DT_F64, nullptr, 1, t);
    };
    GPEX_TRY(potrf_inv(ctx, s, A, lda, T, ldt, n1, ws, col0));
    // L21 = A21 T11^T into ws (T11^T is upper triangular)
    GPEX_TRY(g(A21, 0, lda, T, 1, ldt, ws, n2, n2, n1, n1, 1.0, 0.0, TRI_B_UPPER));
    // A22 -= L21 L21^T (only its lower triangle is used)
    GPEX_TRY(g(ws, 0, n2, ws, 1, n2, A22, lda, n2, n2, n1, -1.0, 1.0, TRI_C_LOWER));
    // wsb = L21 T11
    GPEX_TRY(g(ws, 0, n2, T, 0, ldt, wsb, n2, n2, n1, n1, 1.0, 0.0, 0));
    hipLaunchKernelGGL(k_join, dim3((unsigned)((blk + 255) / 256), 3), dim3(256), 0, s, ws, A, lda, T, ldt, n1, n2);
    GPEX_HIP(ctx, hipGetLastError());
    GPEX_TRY(potrf_inv(ctx, s, A22, lda, T22, ldt, n2, ws, col0 + n1));
    // T21 = -T22 wsb (T22 is lower triangular)
    GPEX_TRY(g(T22, 0, ldt, wsb, 0, n2, T21, ldt, n2, n1, n2, -1.0, 0.0, TRI_A_LOWER));
    return GPEX_OK;
}

// ---------------------------------------------------------------------------------------------
namespace {
struct Timer {
    gpex_ctx_t ctx;
    std::vector<hipEvent_t> ev;
    size_t used = 0;
    hipEvent_t next() {
        if (used == ev.size()) {
            hipEvent_t e;
            if (hipEventCreate(&e) != hipSuccess) return nullptr;
            ev.push_back(e);
        }
        return ev[used++];
    }
    ~Timer() {
        for (auto e : ev) (void)hipEventDestroy(e);
    }
};
}  // namespace

}  // namespace gpex

using namespace gpex;

extern "C" int gpex_potrf_mp(gpex_ctx_t ctx, gpex_tiled_t a, int64_t* info) {
    if (!ctx) return GPEX_ERR_ARG;
    if (!a || !info) return set_err(ctx, GPEX_ERR_ARG, "gpex_potrf_mp: null handle or info");
    if (a->failed) return set_err(ctx, GPEX_ERR_STATE, "gpex_potrf_mp: an earlier factorization of this matrix failed");
    if (a->factored) return set_err(ctx, GPEX_ERR_STATE, "gpex_potrf_mp: matrix already factored");
    GPEX_HIP(ctx, hipSetDevice(ctx->device));
    const int64_t nt = a->nt;
    const int nb = a->nb;
    const size_t tile_el = (size_t)nb * nb;
    hipStream_t s = ctx->stream;
    if (!a->tinv)
        GPEX_TRY(tiled_alloc(ctx, a, (void**)&a->tinv, sizeof(double) * tile_el * nt, "inverse diagonal tiles"));
    // FP16 copy of the factor for the simulation product: off-diagonal tiles written by the panel
    // solves, the two FP16 parts of the diagonal tiles once the factorization is done
    if (a->opts.amp && nt > 1 && !a->l16)
        GPEX_TRY(tiled_alloc(ctx, a, (void**)&a->l16, sizeof(_Float16) * a->l16_elems(), "FP16 factor panels"));
    // rows of tile row i that exist (the last one may be padding beyond n)
    auto rows = [&](int64_t i) { return (double)std::min<int64_t>(nb, a->n - i * nb); };
    // FP64 tiles still hold V (the generator scaled only the reduced-precision tiles): step 0 applies
    // s^2 to them, as alpha of their panel solves and beta of their updates; tile (0, 0) is scaled
    // before its factorization
    const double s2_first = a->unscaled64 ? a->s * a->s : 1.0;

    // Per-step task groups, built once on the host and uploaded in one copy.  A group holds the
    // tasks of one step with one compute precision and one operand-type signature (a launch runs
    // one typed kernel).  Panel solves: FP64 compute for every tile; updates: the output tile's
    // precision.
    struct Group { int64_t b0, b1; int compute, role, k, next; };
    std::vector<GemmTask> tasks;
    std::vector<CopyTask> copies;
    std::vector<Group> groups;
    std::vector<int64_t> group_beg((size_t)nt + 1, 0);
    std::vector<int64_t> copy_beg((size_t)nt + 1, 0);
    std::vector<double> upd_flops(3, 0.0), upd_flops_exact(3, 0.0);
    auto sig = [](int compute, const GemmTask& g) {
        return compute * 1000 + g.ta * 100 + g.tb * 10 + g.tc;
    };
    // Operand copies of the panel tiles for the updates.  A trailing update computes in its output
    // tile's precision with the operands converted to it; a panel tile of another precision that
    // feeds FP32 or FP64 outputs gets its FP32 / FP64 version written once by the panel solve, and
    // those updates read the copy (the same values the kernels would convert on every load; the
    // updates of one step and precision then run one kernel signature, in one launch, instead of
    // one launch per operand-type pair).  Two buffers, by step parity: step k's updates
    // (look-ahead stream) still read step k's copies while step k + 1's panel solves write theirs.
    // FP16 updates read their operands from the row-major FP16 factor panels instead (the same
    // values, with k contiguous: both operands then move in 16-byte vectors with no transposition);
    // those panels are written by the same panel solves and never reused, so they need no copy.
    const bool l16_ops = a->l16 != nullptr;
    auto feeds = [&](int64_t i, int64_t k, int want) {   // does tile (i, k) feed an update computing in `want`?
        for (int64_t j = k + 1; j < i; ++j)
            if (a->prec(i, j) == want) return true;
        for (int64_t j = i + 1; j < nt; ++j)
            if (a->prec(j, i) == want) return true;
        return false;
    };
    std::vector<uint8_t> need32((size_t)(nt * nt), 0), need64((size_t)(nt * nt), 0);
    bool any32 = false, any64 = false;
    for (int64_t k = 0; k + 1 < nt && a->opts.amp; ++k)
        for (int64_t i = k + 1; i < nt; ++i) {
            const int p = a->prec(i, k);
            if (p != DT_F32 && feeds(i, k, DT_F32)) any32 = need32[(size_t)(i * nt + k)] = 1;
            if (p != DT_F64 && feeds(i, k, DT_F64)) any64 = need64[(size_t)(i * nt + k)] = 1;
        }
    // workspace: panel copies (FP64-sized slots), diagonal scratch, operand copies, task and copy lists
    Carve cv;
    const size_t p_pws = cv.add(nt > 1 ? 8 * tile_el * (size_t)(nt - 1) : 0), p_ws = cv.add(sizeof(double) * tile_el);
    const size_t p_c32 = cv.add(any32 ? 2 * 4 * tile_el * (size_t)(nt - 1) : 0),
                 p_c64 = cv.add(any64 ? 2 * 8 * tile_el * (size_t)(nt - 1) : 0);
    size_t ntask = 0;
    for (int64_t k = 0; k < nt; ++k) ntask += (size_t)(nt - k - 1) + (size_t)(nt - k - 1) * (nt - k) / 2;
    const size_t p_tasks = cv.add(sizeof(GemmTask) * ntask), p_copies = cv.add(sizeof(CopyTask) * (size_t)(nt * (nt - 1) / 2));
    const size_t p_dtiles = cv.add(a->l16 ? sizeof(void*) * (size_t)nt : 0);
    void* wsb = nullptr;
    GPEX_TRY(ws_get(ctx, WS_POTRF, cv.total, &wsb, "factorization workspace"));
    uint8_t* pws = cv.get<uint8_t>(wsb, p_pws);
    double* ws = cv.get<double>(wsb, p_ws);
    float* c32 = cv.get<float>(wsb, p_c32);
    double* c64 = cv.get<double>(wsb, p_c64);
    auto copy32 = [&](int64_t i, int64_t k) { return c32 + ((size_t)(k % 2) * (nt - 1) + (size_t)(i - k - 1)) * tile_el; };
    auto copy64 = [&](int64_t i, int64_t k) { return c64 + ((size_t)(k % 2) * (nt - 1) + (size_t)(i - k - 1)) * tile_el; };
    // operand (i, k) of an update computing in `want`: the copy when there is one, else the tile
    auto operand = [&](int64_t i, int64_t k, int want, const void*& ptr, int8_t& type) {
        const int p = a->prec(i, k);
        if (want == DT_F32 && need32[(size_t)(i * nt + k)]) { ptr = copy32(i, k); type = DT_F32; return; }
        if (want == DT_F64 && need64[(size_t)(i * nt + k)]) { ptr = copy64(i, k); type = DT_F64; return; }
        ptr = a->tile(i, k);
        type = (int8_t)p;
    };
    GemmTask* d_tasks = cv.get<GemmTask>(wsb, p_tasks);
    CopyTask* d_copies = cv.get<CopyTask>(wsb, p_copies);
    const uint8_t** d_diag_tiles = cv.get<const uint8_t*>(wsb, p_dtiles);
    std::vector<const uint8_t*> diag_tiles;
    if (a->l16)
        for (int64_t k = 0; k < nt; ++k) diag_tiles.push_back(static_cast<const uint8_t*>(a->tile(k, k)));
    tasks.reserve(ntask);
    copies.reserve((size_t)(nt * (nt - 1) / 2));
    for (int64_t k = 0; k < nt; ++k) {
        for (int64_t i = k + 1; i < nt; ++i) {
            CopyTask c{a->tile(i, k), pws + 8 * tile_el * (i - k - 1), (int64_t)(dt_size(a->prec(i, k)) * tile_el)};
            copies.push_back(c);
        }
        copy_beg[(size_t)k + 1] = (int64_t)copies.size();
        group_beg[(size_t)k] = (int64_t)groups.size();
        std::map<int, std::vector<GemmTask>> panel, update, update_next;
        for (int64_t i = k + 1; i < nt; ++i) {
            int p = a->prec(i, k);
            GemmTask g{};
            g.A = pws + 8 * tile_el * (i - k - 1);
            g.B = a->tinv_tile(k);
            g.C = a->tile(i, k);
            g.lda = g.ldb = g.ldc = nb;
            g.M = g.N = g.K = nb;
            g.ta = (int8_t)p; g.tb = DT_F64; g.tc = (int8_t)p;
            g.transA = 0; g.transB = 1;
            g.alpha = (k == 0 && p == DT_F64) ? s2_first : 1.0;   // an FP64 tile still holds V
            g.beta = 0.0;
            g.tri = TRI_B_UPPER;   // T_kk^T is upper triangular
            if (a->l16) {   // tile (i, k) lands at columns [k nb, (k+1) nb) of row panel i
                g.C2 = a->l16_panel(i) + (size_t)k * nb;
                g.ldc2 = a->l16_ld(i);
            }
            if (need32[(size_t)(i * nt + k)]) g.C3 = copy32(i, k);
            if (need64[(size_t)(i * nt + k)]) g.C4 = copy64(i, k);
            panel[sig(DT_F64, g)].push_back(g);
        }
        for (int64_t j = k + 1; j < nt; ++j)
            for (int64_t i = j; i < nt; ++i) {
                int p = (i == j) ? DT_F64 : a->prec(i, j);
                GemmTask g{};
                if (p == DT_F16 && l16_ops) {
                    // op(A)[r, c] = L_ik[r, c] and op(B)[c, r'] = L_jk[r', c], both k-contiguous
                    g.A = a->l16_panel(i) + (size_t)k * nb; g.lda = a->l16_ld(i); g.ta = DT_F16; g.transA = 1;
                    g.B = a->l16_panel(j) + (size_t)k * nb; g.ldb = a->l16_ld(j); g.tb = DT_F16; g.transB = 0;
                } else {
                    operand(i, k, p, g.A, g.ta);
                    operand(j, k, p, g.B, g.tb);
                    g.lda = g.ldb = nb;
                    g.transA = 0; g.transB = 1;
                }
                g.C = a->tile(i, j);
                g.ldc = nb;
                g.M = g.N = g.K = nb;
                g.tc = (int8_t)p;
                g.alpha = -1.0;
                g.beta = (k == 0 && p == DT_F64) ? s2_first : 1.0;   // s^2 V - L_i0 L_j0^T for FP64 tiles
                g.tri = (i == j) ? TRI_C_LOWER : 0;   // diagonal tiles: only the lower triangle is used
                (j == k + 1 ? update_next : update)[sig(p, g)].push_back(g);
                upd_flops[(size_t)p] += (i == j ? 1.0 : 2.0) * nb * (double)nb * nb;
                upd_flops_exact[(size_t)p] += (i == j ? 1.0 : 2.0) * rows(i) * rows(j) * rows(k);
            }
        for (auto& kv : panel) {
            groups.push_back(Group{(int64_t)tasks.size(), 0, DT_F64, GEMM_GENERIC, (int)k, 0});
            tasks.insert(tasks.end(), kv.second.begin(), kv.second.end());
            groups.back().b1 = (int64_t)tasks.size();
        }
        for (int nx = 1; nx >= 0; --nx)
            for (auto& kv : (nx ? update_next : update)) {
                groups.push_back(Group{(int64_t)tasks.size(), 0, kv.first / 1000, GEMM_UPDATE, (int)k, nx});
                tasks.insert(tasks.end(), kv.second.begin(), kv.second.end());
                groups.back().b1 = (int64_t)tasks.size();
            }
    }
    group_beg[(size_t)nt] = (int64_t)groups.size();
    if (tasks.size() > ntask || copies.size() > (size_t)(nt * (nt - 1) / 2))
        return set_err(ctx, GPEX_ERR_STATE, "gpex_potrf_mp: task count exceeds its workspace");
    // uploads are ordered after earlier users of the workspace on the context stream; the host
    // vectors stay alive until the final synchronisation
    if (!tasks.empty()) GPEX_HIP(ctx, hipMemcpyAsync(d_tasks, tasks.data(), sizeof(GemmTask) * tasks.size(), hipMemcpyHostToDevice, s));
    if (!copies.empty()) GPEX_HIP(ctx, hipMemcpyAsync(d_copies, copies.data(), sizeof(CopyTask) * copies.size(), hipMemcpyHostToDevice, s));
    if (!diag_tiles.empty())
        GPEX_HIP(ctx, hipMemcpyAsync(d_diag_tiles, diag_tiles.data(), sizeof(void*) * diag_tiles.size(), hipMemcpyHostToDevice, s));
    GPEX_HIP(ctx, hipMemsetAsync(ctx->d_flags + FLAG_INFO, 0, sizeof(long long) * (FLAG_BADTASK + 1), s));

    Timer tm{ctx, {}, 0};
    struct Rec { hipEvent_t b, e; int prec; };
    std::vector<Rec> recs;
    hipEvent_t e_all0 = nullptr, e_all1 = nullptr;
    if (ctx->timing) {
        e_all0 = tm.next();
        (void)hipEventRecord(e_all0, s);
    }
    // Look-ahead of depth one on two streams (both at the default priority):
    //   stream A (the context stream): [wait rest(k-1)] next-column update of step k, then the panel
    //            work of step k+1 (diagonal factor + inverse, panel copy, panel solves);
    //   stream B (the context's look-ahead stream): [wait panel(k)] the rest of step k's update.
    // The panel work of step k+1 thus overlaps the bulk update of step k.  Tiles touched
    // concurrently are disjoint: rest(k) writes columns >= k+2, the panel of k+1 column k+1.
    // In serial mode stream B is the context stream: the same launches in the same order per tile.
    const bool two = !ctx->serial && nt > 1;
    if (two && !ctx->ahead) GPEX_HIP(ctx, hipStreamCreateWithFlags(&ctx->ahead, hipStreamNonBlocking));
    hipStream_t sb = two ? ctx->ahead : s;
    // events: fork, then panel(k) and rest(k) per step
    hipEvent_t evfork = nullptr;
    std::vector<hipEvent_t> evp((size_t)nt, nullptr), evr((size_t)nt, nullptr);
    if (two) {
        GPEX_TRY(ctx_event(ctx, 0, &evfork));
        for (int64_t k = 0; k < nt; ++k) {
            GPEX_TRY(ctx_event(ctx, 1 + 2 * (size_t)k, &evp[(size_t)k]));
            GPEX_TRY(ctx_event(ctx, 2 + 2 * (size_t)k, &evr[(size_t)k]));
        }
    }
    auto record = [&](hipEvent_t e, hipStream_t st) -> int {
        if (two) GPEX_HIP(ctx, hipEventRecord(e, st));
        return GPEX_OK;
    };
    auto wait = [&](hipStream_t st, hipEvent_t e) -> int {
        if (two) GPEX_HIP(ctx, hipStreamWaitEvent(st, e, 0));
        return GPEX_OK;
    };
    auto launch_groups = [&](int64_t k, int want_role, int want_next, hipStream_t st) -> int {
        for (int64_t gi = group_beg[(size_t)k]; gi < group_beg[(size_t)k + 1]; ++gi) {
            const Group& G = groups[(size_t)gi];
            if (G.role != want_role || (want_role == GEMM_UPDATE && G.next != want_next)) continue;
            const bool upd = G.role == GEMM_UPDATE;
            Rec rc{nullptr, nullptr, G.compute};
            if (ctx->timing && upd) {
                rc.b = tm.next();
                (void)hipEventRecord(rc.b, st);
            }
            GPEX_TRY(gemm_launch(ctx, st, G.compute, d_tasks + G.b0, (int)(G.b1 - G.b0), tasks[(size_t)G.b0], G.role));
            if (ctx->timing && upd) {
                rc.e = tm.next();
                (void)hipEventRecord(rc.e, st);
                recs.push_back(rc);
            }
        }
        return GPEX_OK;
    };
    auto panel_work = [&](int64_t k) -> int {
        GPEX_TRY(potrf_inv(ctx, s, static_cast<double*>(a->tile(k, k)), nb, a->tinv_tile(k), nb, nb, ws, k * nb));
        int64_t nc = copy_beg[(size_t)k + 1] - copy_beg[(size_t)k];
        if (nc > 0) {
            const int64_t chunk = 1 << 16;
            int64_t mx = (int64_t)(8 * tile_el);
            dim3 grid((unsigned)((mx + chunk - 1) / chunk), (unsigned)nc);
            hipLaunchKernelGGL(k_copy_tasks, grid, dim3(256), 0, s, d_copies + copy_beg[(size_t)k], chunk);
            GPEX_HIP(ctx, hipGetLastError());
        }
        return launch_groups(k, GEMM_GENERIC, 0, s);
    };
    auto schedule = [&]() -> int {
        if (s2_first != 1.0)
            GPEX_TRY(copy2d(ctx, s, a->tile(0, 0), DT_F64, nb, a->tile(0, 0), DT_F64, nb, nb, nb, s2_first));
        // fork: stream B starts after everything queued so far on the context stream
        GPEX_TRY(record(evfork, s));
        GPEX_TRY(wait(sb, evfork));
        GPEX_TRY(panel_work(0));
        GPEX_TRY(record(evp[0], s));
        for (int64_t k = 0; k + 1 < nt; ++k) {
            if (k > 0) GPEX_TRY(wait(s, evr[(size_t)k - 1]));
            GPEX_TRY(launch_groups(k, GEMM_UPDATE, 1, s));
            GPEX_TRY(panel_work(k + 1));
            GPEX_TRY(record(evp[(size_t)k + 1], s));
            GPEX_TRY(wait(sb, evp[(size_t)k]));
            GPEX_TRY(launch_groups(k, GEMM_UPDATE, 0, sb));
            GPEX_TRY(record(evr[(size_t)k], sb));
        }
        // join: the context stream waits for the last bulk update
        if (nt > 1) GPEX_TRY(wait(s, evr[(size_t)nt - 2]));
        if (a->l16) {   // the diagonal tiles' two FP16 parts, beside their off-diagonal rows
            const unsigned nsub = (unsigned)((nb + D16_T - 1) / D16_T);
            hipLaunchKernelGGL(k_diag16, dim3(nsub, nsub, (unsigned)nt), dim3(256), 0, s, d_diag_tiles, nb, a->l16,
                               reinterpret_cast<unsigned long long*>(ctx->d_flags));
            GPEX_HIP(ctx, hipGetLastError());
        }
        return GPEX_OK;
    };
    int r = schedule();
    if (ctx->timing) {
        e_all1 = tm.next();
        (void)hipEventRecord(e_all1, s);
    }
    hipError_t se = hipStreamSynchronize(s);
    if (two && se == hipSuccess) se = hipStreamSynchronize(sb);
    if (r < 0) return r;
    if (se != hipSuccess) return set_err(ctx, GPEX_ERR_HIP, std::string("potrf sync: ") + hipGetErrorString(se));
    if (ctx->timing) {
        float ms = 0;
        (void)hipEventElapsedTime(&ms, e_all0, e_all1);
        ctx->timings[0] = ms;
        for (int p = 0; p < 3; ++p) {
            ctx->timings[1 + 3 * p] = 0;
            ctx->timings[2 + 3 * p] = 0;
            ctx->timings[3 + 3 * p] = upd_flops[(size_t)p];
            ctx->timings[12 + p] = upd_flops_exact[(size_t)p];
        }
        // per precision: summed launch durations and the busy time (union of the launch intervals,
        // which overlap where launches of two streams run together)
        std::vector<std::pair<double, double>> iv[3];
        for (auto& rc : recs) {
            float m = 0, b0 = 0, b1 = 0;
            (void)hipEventElapsedTime(&m, rc.b, rc.e);
            (void)hipEventElapsedTime(&b0, e_all0, rc.b);
            (void)hipEventElapsedTime(&b1, e_all0, rc.e);
            ctx->timings[1 + 3 * rc.prec] += m;
            ctx->timings[2 + 3 * rc.prec] += 1;
            iv[rc.prec].push_back({b0, b1});
        }
        for (int p = 0; p < 3; ++p) {
            std::sort(iv[p].begin(), iv[p].end());
            double busy = 0, cb = -1, ce = -1;
            for (auto& x : iv[p]) {
                if (x.first > ce) {
                    if (ce > cb) busy += ce - cb;
                    cb = x.first;
                    ce = x.second;
                } else {
                    ce = std::max(ce, x.second);
                }
            }
            if (ce > cb) busy += ce - cb;
            ctx->timings[15 + p] = busy;
        }
    }
    long long fl[FLAG_COUNT] = {};
    GPEX_HIP(ctx, hipMemcpy(fl, ctx->d_flags, sizeof(fl), hipMemcpyDeviceToHost));
    if (fl[FLAG_BADTASK]) return set_err(ctx, GPEX_ERR_STATE, "gpex_potrf_mp: internal task-type mismatch");
    *info = fl[FLAG_INFO];
    if (fl[FLAG_INFO] != 0) {
        // the tiles were overwritten in place up to the failing column: the handle is unusable
        a->failed = true;
        return set_err(ctx, GPEX_ERR_NOT_SPD, "gpex_potrf_mp: non-positive pivot at column " + std::to_string(fl[FLAG_INFO]));
    }
    a->factored = true;
    a->unscaled64 = false;
    if (fl[FLAG_FP16_OVF]) {
        // a value stored in FP16 (an FP16 tile update or the FP16 copy of the factor) became +-inf
        a->diag.fp16_overflow = 1;
        return set_err(ctx, GPEX_WARN_FP16_OVERFLOW, "gpex_potrf_mp: an FP16 value of the factor overflowed");
    }
    return GPEX_OK;
}

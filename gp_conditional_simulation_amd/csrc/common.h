// Internal declarations shared by the gfx950 HIP sources of libgpex.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "gpex.h"

namespace gpex {

// Storage / compute precision codes (same numbering as the public precision map).
enum : int { DT_F64 = 0, DT_F32 = 1, DT_F16 = 2 };
inline size_t dt_size(int dt) { return dt == DT_F64 ? 8 : (dt == DT_F32 ? 4 : 2); }

// Device-side flag words kept per context (zeroed by the entry points that use them).
enum : int { FLAG_INFO = 0, FLAG_FP16_OVF = 1, FLAG_MSPE = 2, FLAG_BADTASK = 3, FLAG_COUNT = 4 };

}  // namespace gpex

struct gpex_ctx_s {
    int device = 0;
    hipStream_t stream = nullptr;
    std::string err;
    long long* d_flags = nullptr;     // FLAG_COUNT device words
    bool timing = false;
    double timings[16] = {};          // layout documented at gpex_ctx_timings
    // simulation workspace (FP16/FP64 input B, padded M, norm partials), kept between calls and
    // grown when a call needs more
    void* sim_ws = nullptr;
    size_t sim_ws_bytes = 0;
    // side stream (default priority) for the ragged strips of a split GEMM launch, forked from and
    // joined to the launching stream through two events; created on first use
    hipStream_t side = nullptr;
    hipEvent_t side_fork = nullptr, side_join = nullptr;
};

struct gpex_tiled_s {
    int device = 0;
    int64_t n = 0, nt = 0;
    int nb = 0;
    std::vector<uint8_t> map;        // nt*nt, row-major, 255 above the diagonal
    std::vector<int64_t> off;        // byte offset of lower tile t = i(i+1)/2 + j in `base`
    uint8_t* base = nullptr;         // tile storage, each tile nb x nb column-major
    size_t bytes = 0;
    double s = 1.0;
    std::vector<double> stats;       // 3 per lower tile: sum of squares, min, max (unscaled)
    double* tinv = nullptr;          // nt tiles nb x nb FP64: inverse of each diagonal factor tile
    // FP16 copy of the off-diagonal factor for the simulation product (amp only): tile row i as one
    // row-major panel of nb x (i nb) at l16 + nb*nb*i(i-1)/2 (k contiguous, leading dim i nb)
    _Float16* l16 = nullptr;
    _Float16* l16_panel(int64_t i) const { return l16 + (size_t)nb * nb * (size_t)(i * (i - 1) / 2); }
    bool factored = false;
    gpex_prec_opts opts{};
    gpex_diag diag{};

    int64_t tidx(int64_t i, int64_t j) const { return i * (i + 1) / 2 + j; }
    int prec(int64_t i, int64_t j) const { return map[(size_t)(i * nt + j)]; }
    void* tile(int64_t i, int64_t j) const { return base + off[(size_t)tidx(i, j)]; }
    double* tinv_tile(int64_t k) const { return tinv + (size_t)k * nb * nb; }
};

namespace gpex {

int set_err(gpex_ctx_t ctx, int code, const std::string& msg);

#define GPEX_HIP(ctx, call)                                                                 \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return ::gpex::set_err((ctx), GPEX_ERR_HIP,                                     \
                                   std::string(#call) + ": " + hipGetErrorString(e_));      \
    } while (0)

#define GPEX_TRY(expr)               \
    do {                             \
        int r_ = (expr);             \
        if (r_ < 0) return r_;       \
    } while (0)

int dev_alloc(gpex_ctx_t ctx, void** p, size_t bytes, const char* what);
void dev_free(void* p);

// ---- batched mixed-precision GEMM engine (gemm.hip) ---------------------------------------
// One task: C (M x N) = alpha * op(A) * op(B) + beta * C.  op(A) is M x K, op(B) is K x N.
// Storage codes ta/tb/tc pick each operand's element type; trans flags pick the layout:
// transA = 0: A(m, k) at A[m + k*lda]; transA = 1: A(m, k) at A[k + m*lda];
// transB = 0: B(k, n) at B[k + n*ldb]; transB = 1: B(k, n) at B[n + k*ldb].
// With beta == 0 the old C is not read.
struct GemmTask {
    const void* A;
    const void* B;
    void* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int8_t ta, tb, tc, transA, transB;
    int8_t tri;   // TRI_* flags: triangular structure the kernels may exploit (results are unchanged)
    int8_t pad1, pad2;
    double alpha, beta;
    // Optional second output (typed kernels only): the stored result converted to FP16 and
    // written row-major, element (row, col) at C2[col + row * ldc2].
    _Float16* C2;
    int64_t ldc2;
};

// Triangular structure of a task.  TRI_C_LOWER: only the lower triangle of C is wanted (blocks
// strictly above the diagonal are skipped and keep their old contents).  TRI_A_LOWER: op(A) is
// lower triangular (zero for k > row), so a block of rows stops its K loop after its last row.
// TRI_B_UPPER: op(B) is upper triangular (zero for k > column), so a block of columns stops after
// its last column.  The skipped products are exact zeros.
enum : int { TRI_C_LOWER = 1, TRI_A_LOWER = 2, TRI_B_UPPER = 4 };

// compute: DT_F64 (FP64 matrix cores), DT_F32 (FP32 matrix cores) or DT_F16 (FP16 matrix cores,
// FP32 accumulation).  Either `d_tasks` (device array of ntasks tasks with identical M, N, K,
// element types and layout flags, those of `one`) or, when d_tasks is null, the single task
// `one` passed by value.  A task whose types differ from `one`'s sets flags[FLAG_BADTASK] and
// is skipped.
enum : int { GEMM_GENERIC = 0, GEMM_UPDATE = 1, GEMM_TRMM = 2 };
// role only names the kernel symbols (trailing updates, simulation product, the rest) so that
// kernel traces attribute their time; the launch choices follow the task types.
extern int g_f16_grid;   // wave grid of FP16 TRMM launches (-1 auto, 0: 2 x 2, otherwise 2 x 4)
int gemm_launch(gpex_ctx_t ctx, hipStream_t s, int compute, const GemmTask* d_tasks, int ntasks,
                const GemmTask& one, int role = GEMM_GENERIC);

// Convenience: single-task GEMM on the context stream.
int gemm1(gpex_ctx_t ctx, int compute, const void* A, int ta, int transA, int64_t lda,
          const void* B, int tb, int transB, int64_t ldb, void* C, int tc, int64_t ldc, int M,
          int N, int K, double alpha, double beta);

// ---- small helpers (chol.hip) ---------------------------------------------------------------
// Dense 2-D copy with element-type conversion (RNE on narrowing; FP16 overflow sets the flag).
int copy2d(gpex_ctx_t ctx, hipStream_t s, const void* src, int tsrc, int64_t lds, void* dst,
           int tdst, int64_t ldd, int64_t rows, int64_t cols, double scale);
// Set a rows x cols FP64 block to zero.
int zero2d(gpex_ctx_t ctx, hipStream_t s, double* dst, int64_t ldd, int64_t rows, int64_t cols);

// Factor the FP64 diagonal block A (n x n, leading dim lda) in place (lower, upper zeroed) and
// write its inverse into T (n x n, leading dim ldt, upper zeroed).  ws: FP64 scratch of at least
// n*n/4 elements + n*n (leading dim n).  col0 is the global 0-based column of A(0,0) (for info).
int potrf_inv(gpex_ctx_t ctx, hipStream_t s, double* A, int64_t lda, double* T, int64_t ldt,
              int n, double* ws, int64_t col0);

// ---- planner (planner.cpp) -------------------------------------------------------------------
void plan_precision(const std::vector<double>& stats, int64_t nt, const gpex_prec_opts& o,
                    std::vector<uint8_t>& map, gpex_diag& d);

}  // namespace gpex

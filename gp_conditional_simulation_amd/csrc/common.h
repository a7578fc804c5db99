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

// Grow-only device workspaces kept by a context, one per entry point that needs temporaries.  A
// call takes its slot's buffer (growing it when too small) and leaves it for the next call, so a
// steady run allocates nothing; the buffers go back through the context's allocator at destroy
// (or gpex_ctx_release_workspace).  Reuse is safe because every use is ordered on the context
// stream (work forked to the context's other streams is joined back before a call returns).
namespace gpex {
enum : int { WS_COV = 0, WS_POTRF = 1, WS_SIM = 2, WS_KRIGE = 3, WS_SCAN = 4, WS_COUNT = 5 };
}

struct gpex_ctx_s {
    int device = 0;
    hipStream_t stream = nullptr;
    std::string err;
    // device memory: the caller's allocator (e.g. torch's caching allocator), else hipMalloc
    void* (*alloc)(size_t, void*) = nullptr;
    void (*dealloc)(void*, void*) = nullptr;
    void* user = nullptr;
    long long* d_flags = nullptr;     // FLAG_COUNT device words
    bool timing = false;
    bool serial = false;              // every launch on the context stream, in program order
    double timings[32] = {};          // layout documented at gpex_ctx_timings
    struct Ws {
        void* p = nullptr;
        size_t bytes = 0;
    } ws[gpex::WS_COUNT];
    // side stream (default priority) for the ragged strips of a split GEMM launch, forked from and
    // joined to the launching stream through two events; created on first use
    hipStream_t side = nullptr;
    hipEvent_t side_fork = nullptr, side_join = nullptr;
    // look-ahead stream of the factorization and its event pool (created on first use, kept)
    hipStream_t ahead = nullptr;
    std::vector<hipEvent_t> events;
    // timing events of the simulation product's phase timings (created on first use, kept)
    std::vector<hipEvent_t> tevents;
    // pinned host words for the simulation product's end-of-call readback (flags, then ||B||^2),
    // allocated with the context
    long long* h_ret = nullptr;
};

struct gpex_tiled_s {
    int device = 0;
    // the allocator of the creating context (the handle may outlive the context)
    void* (*alloc)(size_t, void*) = nullptr;
    void (*dealloc)(void*, void*) = nullptr;
    void* user = nullptr;
    int64_t n = 0, nt = 0;
    int nb = 0;
    std::vector<uint8_t> map;        // nt*nt, row-major, 255 above the diagonal
    std::vector<int64_t> off;        // byte offset of lower tile t = i(i+1)/2 + j in `base`
    uint8_t* base = nullptr;         // tile storage, each tile nb x nb column-major
    size_t bytes = 0;
    double s = 1.0;
    std::vector<double> stats;       // 3 per lower tile: sum of squares, min, max (unscaled)
    double* tinv = nullptr;          // nt tiles nb x nb FP64: inverse of each diagonal factor tile
    // FP16 copy of the factor for the simulation product and the factorization's FP16 updates (amp
    // only, more than one tile row): tile row i as one row-major panel of nb x ((i + 2) nb), k
    // contiguous, at l16 + nb*nb*(i(i-1)/2 + 2i): columns [0, i nb) hold cast16 of the off-diagonal
    // tiles (i, 0..i-1), columns [i nb, (i+2) nb) the diagonal tile L_ii as two FP16 parts
    // (hi = cast16(L_ii), lo = cast16(L_ii - hi), zeros above the diagonal) in pairs of w-wide
    // slabs, w = l16_pair_w(nb): column c of L_ii has hi at i nb + 2 w (c / w) + c % w and lo w
    // further.
    _Float16* l16 = nullptr;
    _Float16* l16_panel(int64_t i) const { return l16 + (size_t)nb * nb * (size_t)(i * (i - 1) / 2 + 2 * i); }
    int64_t l16_ld(int64_t i) const { return (i + 2) * (int64_t)nb; }
    size_t l16_elems() const { return (size_t)nb * nb * (size_t)(nt * (nt - 1) / 2 + 2 * nt); }
    bool factored = false;
    bool failed = false;             // a factorization stopped at a non-positive pivot: tiles hold garbage
    // FP64 tiles hold V rather than s^2 V (reduced tiles hold s^2 V): the factorization applies s^2
    // to them in its first step
    bool unscaled64 = false;
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

// Device memory through the context's allocator (hipMalloc / hipFree without one).  The tiled
// variants use the allocator the handle recorded at creation.
int dev_alloc(gpex_ctx_t ctx, void** p, size_t bytes, const char* what);
void dev_free(gpex_ctx_t ctx, void* p);
int tiled_alloc(gpex_ctx_t ctx, gpex_tiled_t t, void** p, size_t bytes, const char* what);
void tiled_free(gpex_tiled_t t, void* p);
// Workspace slot `slot` of at least `bytes` bytes (grown when smaller).
int ws_get(gpex_ctx_t ctx, int slot, size_t bytes, void** out, const char* what);
inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }
// Consecutive 256-byte aligned pieces of one workspace buffer: size them with add(), then take
// them in the same order from the buffer.
// Slab width of the diagonal tiles' (hi, lo) pairs in the FP16 factor panels: 64 (the row-panel
// kernel's k slab) when it divides the tile order, else the whole tile (one pair).
__host__ __device__ inline int l16_pair_w(int nb) { return nb % 64 == 0 ? 64 : nb; }

struct Carve {
    size_t total = 0;
    std::vector<size_t> at;
    size_t add(size_t b) {
        at.push_back(total);
        total += al256(b ? b : 1);
        return at.size() - 1;
    }
    template <typename T> T* get(void* base, size_t piece) const {
        return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + at[piece]);
    }
};
// A timing-disabled event from the context's pool (index i, created on first use).
int ctx_event(gpex_ctx_t ctx, size_t i, hipEvent_t* out);
// A timing-enabled event from the context's second pool (index i, created on first use).
int ctx_timing_event(gpex_ctx_t ctx, size_t i, hipEvent_t* out);
// Device address of the fixed scratch array of the allocation-free entry points on `device`
// (NULL before a context was created on it).
constexpr size_t SCRATCH_BYTES = size_t(32) << 20;
void* scratch_ptr(int device);

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
    // Optional second output (typed FP64-compute kernels of the generic role only, i.e. the panel
    // solves): the stored result converted to FP16 and written row-major, element (row, col) at
    // C2[col + row * ldc2].
    _Float16* C2;
    int64_t ldc2;
    // Optional copies of the stored result in FP32 (C3) and FP64 (C4), column-major with leading
    // dimension ldc (the factorization's per-step operand copies of the panel tiles; same kernels
    // as C2).
    float* C3;
    double* C4;
    // FP16 destination storage between k-tasks (simulation product only, whole blocks): the
    // accumulator starts from beta C, is rounded to FP16 after every kround values of k and at the
    // end of the K loop, and alpha times it is stored.  0: off.
    int32_t kround;
    // Simulation product only: the caller's part of C, rows [0, m_store) and columns [0, n_store)
    // of the task's C (the tile padding beyond them is computed but not stored, and C is read
    // only inside it).  0: all of C.
    int32_t m_store, n_store;
    // Row panels of the simulation product only (the 256 x 256 FP16 kernel): the last 2 kdup values
    // of k are the diagonal tile (order kdup) as pairs of 64-wide slabs (hi, lo), both meeting the
    // same 64 rows of B: k = K - 2 kdup + 128 s + 64 h + t (h = 0, 1; t < 64) reads B row
    // K - 2 kdup + 64 s + t.  0: off.
    int32_t kdup;
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
extern int g_panel16;    // FP16 simulation-product row panels on 256 x 256 blocks when they fit (0: never)
extern int g_f16_grid;   // wave grid of FP16 TRMM launches (-1 auto, 0: 2 x 2, otherwise 2 x 4)
int gemm_launch(gpex_ctx_t ctx, hipStream_t s, int compute, const GemmTask* d_tasks, int ntasks,
                const GemmTask& one, int role = GEMM_GENERIC);

// Convenience: single-task GEMM on the context stream.
int gemm1(gpex_ctx_t ctx, int compute, const void* A, int ta, int transA, int64_t lda,
          const void* B, int tb, int transB, int64_t ldb, void* C, int tc, int64_t ldc, int M,
          int N, int K, double alpha, double beta);

// Whether the 256 x 256 FP16 row-panel kernel takes a launch of these tasks (the shape and
// alignment it needs, at least one workgroup per CU (256), the kernel enabled), and its launch.
bool panel16_takes(const GemmTask& one, int ntasks);
int panel16_launch(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one);

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

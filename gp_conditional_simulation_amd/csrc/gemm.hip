// Batched tile GEMM entry points: dispatch on the compute precision to the per-precision
// translation units (gemm_f64.hip, gemm_f32.hip, gemm_f16.hip), which hold the kernels of
// gemm_kernel.h.
#include "gemm_kernel.h"

namespace gpex {

// Wave grid of FP16 simulation-product launches: -1 = chosen per launch (2 x 4 waves when that
// still gives at least 2048 workgroups, else 2 x 2), 0 = 2 x 2 waves (128 x 128), otherwise 2 x 4
// (128 x 256).
int g_f16_grid = -1;
// Row panels of the FP16 simulation product on the 256 x 256 kernel (panel16.h) when their shape
// allows; 0 keeps them on the general kernel.
int g_panel16 = 1;

int gemm_launch(gpex_ctx_t ctx, hipStream_t s, int compute, const GemmTask* d_tasks, int ntasks,
                const GemmTask& one, int role) {
    if (compute == DT_F64) return gemm_launch_f64(ctx, s, d_tasks, ntasks, one, role);
    if (compute == DT_F32) return gemm_launch_f32(ctx, s, d_tasks, ntasks, one, role);
    return gemm_launch_f16(ctx, s, d_tasks, ntasks, one, role);
}

int gemm1(gpex_ctx_t ctx, int compute, const void* A, int ta, int transA, int64_t lda,
          const void* B, int tb, int transB, int64_t ldb, void* C, int tc, int64_t ldc, int M,
          int N, int K, double alpha, double beta) {
    GemmTask g{};
    g.A = A; g.B = B; g.C = C;
    g.lda = lda; g.ldb = ldb; g.ldc = ldc;
    g.M = M; g.N = N; g.K = K;
    g.ta = (int8_t)ta; g.tb = (int8_t)tb; g.tc = (int8_t)tc;
    g.transA = (int8_t)transA; g.transB = (int8_t)transB;
    g.alpha = alpha; g.beta = beta;
    if (K <= 0) {
        if (beta == 1.0) return GPEX_OK;
    }
    return gemm_launch(ctx, ctx->stream, compute, nullptr, 1, g);
}

}  // namespace gpex

// Batched tile GEMM launches with FP16 compute (FP32 accumulation) (kernels of gemm_kernel.h).
#include "gemm_kernel.h"

namespace gpex {

// At least one 256 x 256 workgroup per CU: from there the row-panel kernel beat the 128 x 128 /
// 128 x 256 kernels at every measured shape (N = 16,384, 2,048 columns: 512 workgroups, 1.41 ->
// 0.90 ms; N = 40,000 at tile 512, 1,000 columns: 632 workgroups, 2.68 -> 2.03 ms).
bool panel16_takes(const GemmTask& one, int ntasks) {
    return g_panel16 && ntasks > 0 && panel16_fits(one) && (int64_t)ntasks * (one.M / P16_BM) * (one.N / P16_BN) >= 256;
}

int panel16_launch(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one) {
    if (!d_tasks || !panel16_takes(one, ntasks))
        return set_err(ctx, GPEX_ERR_STATE, "panel16_launch: the row-panel kernel does not take these tasks");
    const int bmc = one.M / P16_BM, bnc = one.N / P16_BN, xcd = ntasks >= 8 ? 1 : 0;
    const int64_t grid = xcd ? (int64_t)8 * ((ntasks + 7) / 8) * bmc * bnc : (int64_t)ntasks * bmc * bnc;
    if (grid > 0x7fffffffLL) return set_err(ctx, GPEX_ERR_ARG, "panel16_launch: grid too large");
    hipLaunchKernelGGL(k_panel16<0>, dim3((unsigned)grid), dim3(P16_THR), 0, s, d_tasks, ntasks, bmc, bnc, xcd,
                       reinterpret_cast<unsigned long long*>(ctx->d_flags));
    GPEX_HIP(ctx, hipGetLastError());
    return GPEX_OK;
}

int gemm_launch_f16(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, int role) {
    return launch_precision<_Float16>(ctx, s, d_tasks, ntasks, one, role);
}

}  // namespace gpex

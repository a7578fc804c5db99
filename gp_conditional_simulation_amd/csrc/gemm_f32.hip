// Batched tile GEMM launches with FP32 compute (kernels of gemm_kernel.h).
#include "gemm_kernel.h"

namespace gpex {

int gemm_launch_f32(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, int role) {
    return launch_precision<float>(ctx, s, d_tasks, ntasks, one, role);
}

}  // namespace gpex

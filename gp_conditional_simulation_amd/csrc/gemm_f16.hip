// Batched tile GEMM launches with FP16 compute (FP32 accumulation) (kernels of gemm_kernel.h).
#include "gemm_kernel.h"

namespace gpex {

int gemm_launch_f16(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, int role) {
    return launch_precision<_Float16>(ctx, s, d_tasks, ntasks, one, role);
}

}  // namespace gpex

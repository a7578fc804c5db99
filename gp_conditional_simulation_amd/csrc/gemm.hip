// Batched mixed-precision tile GEMM on gfx950 matrix cores.
//
// This is the workhorse of the adaptive mixed-precision tile Cholesky ("Mixed-Precision GPU
// Acceleration for Confidence Regions of Spatial Excursion Sets", Sec. IV-B: each tile task runs
// in the precision of its output tile with the operands converted to it), of the panel solves,
// of kriging (Sec. V-A) and of the conditioning product (Eq. 7).
//
// Design (gfx950, wave64):
//   * 256 threads = 4 waves per workgroup, one 128 x 128 block of C per workgroup, each wave a
//     64 x 64 sub-block made of 4 x 4 matrix-core tiles of 16 x 16.
//   * FP64: v_mfma_f64_16x16x4 (lane l, acc r -> row l/16 + 4r, col l%16).
//     FP32: v_mfma_f32_16x16x4 (row 4(l/16) + r, col l%16).
//     FP16: v_mfma_f32_16x16x32_f16 with FP32 accumulation (row 4(l/16) + r, col l%16).
//   * Operands are staged through LDS with the reduction index contiguous ([row][k] + pad), so
//     every lane feeds four (FP32/FP64) or one (FP16) matrix-core step from one vector read.
//   * Global loads are coalesced along whichever index is contiguous in memory and converted on
//     the fly to the compute type (FP64 -> FP16 goes through round-to-odd FP32, which makes the
//     final FP16 rounding a correct round-to-nearest-even).
//   * The next K slab is prefetched into registers while the current one is multiplied.
//   * Batched launches place all workgroups of one task on one XCD (workgroups are dealt to the
//     8 XCDs round-robin by index), so a task's operand tiles stream through a single L2.
#include "common.h"
#include "devutil.h"

namespace gpex {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, NTHR = 256;

template <typename CT> struct Cfg;
template <> struct Cfg<double> { static constexpr int BK = 16, PAD = 2; };
template <> struct Cfg<float> { static constexpr int BK = 16, PAD = 4; };
template <> struct Cfg<_Float16> { static constexpr int BK = 32, PAD = 8; };

template <typename CT> __device__ __forceinline__ CT cvt_d(double v);
template <> __device__ __forceinline__ double cvt_d<double>(double v) { return v; }
template <> __device__ __forceinline__ float cvt_d<float>(double v) { return (float)v; }
template <> __device__ __forceinline__ _Float16 cvt_d<_Float16>(double v) { return f64_to_f16(v); }
template <typename CT> __device__ __forceinline__ CT cvt_f(float v);
template <> __device__ __forceinline__ double cvt_f<double>(float v) { return (double)v; }
template <> __device__ __forceinline__ float cvt_f<float>(float v) { return v; }
template <> __device__ __forceinline__ _Float16 cvt_f<_Float16>(float v) { return (_Float16)v; }
template <typename CT> __device__ __forceinline__ CT cvt_h(_Float16 v);
template <> __device__ __forceinline__ double cvt_h<double>(_Float16 v) { return (double)v; }
template <> __device__ __forceinline__ float cvt_h<float>(_Float16 v) { return (float)v; }
template <> __device__ __forceinline__ _Float16 cvt_h<_Float16>(_Float16 v) { return v; }

// Load 4 consecutive elements (index idx..idx+3, idx % 4 == 0, 16-byte aligned) of type dt.
template <typename CT>
__device__ __forceinline__ void load4(const void* p, int dt, int64_t idx, CT out[4]) {
    if (dt == DT_F64) {
        const double2* q = reinterpret_cast<const double2*>(static_cast<const double*>(p) + idx);
        double2 a = q[0], b = q[1];
        out[0] = cvt_d<CT>(a.x); out[1] = cvt_d<CT>(a.y);
        out[2] = cvt_d<CT>(b.x); out[3] = cvt_d<CT>(b.y);
    } else if (dt == DT_F32) {
        float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
        out[0] = cvt_f<CT>(a.x); out[1] = cvt_f<CT>(a.y);
        out[2] = cvt_f<CT>(a.z); out[3] = cvt_f<CT>(a.w);
    } else {
        h4 a = *reinterpret_cast<const h4*>(static_cast<const _Float16*>(p) + idx);
        out[0] = cvt_h<CT>(a[0]); out[1] = cvt_h<CT>(a[1]);
        out[2] = cvt_h<CT>(a[2]); out[3] = cvt_h<CT>(a[3]);
    }
}

template <typename CT>
__device__ __forceinline__ CT load1(const void* p, int dt, int64_t idx) {
    if (dt == DT_F64) return cvt_d<CT>(static_cast<const double*>(p)[idx]);
    if (dt == DT_F32) return cvt_f<CT>(static_cast<const float*>(p)[idx]);
    return cvt_h<CT>(static_cast<const _Float16*>(p)[idx]);
}

// Loads one BK x 128 slab of an operand into registers.  Rows r (block-local, 0..127) map to
// global row r0 + r; depth k to k0 + k.  contig_r: element (r, k) at base[r + k*ld], else at
// base[k + r*ld].
template <typename CT, bool EDGE>
struct SlabLoader {
    static constexpr int BK = Cfg<CT>::BK;
    static constexpr int VPT = (128 * BK / NTHR) / 4;  // 4-element vectors per thread
    CT v[VPT][4];

    __device__ __forceinline__ void load(const void* base, int dt, int64_t ld, bool contig_r,
                                         int r0, int k0, int R, int K, int t) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            int r, k;
            if (contig_r) {
                r = (t % 32) * 4;
                k = t / 32 + 8 * q;
            } else {
                constexpr int TPR = BK / 4;
                r = t / TPR + (NTHR / TPR) * q;
                k = (t % TPR) * 4;
            }
            int gr = r0 + r, gk = k0 + k;
            if (!EDGE) {
                int64_t idx = contig_r ? (int64_t)gr + (int64_t)gk * ld : (int64_t)gk + (int64_t)gr * ld;
                load4<CT>(base, dt, idx, v[q]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    int rr = contig_r ? gr + e : gr;
                    int kk = contig_r ? gk : gk + e;
                    v[q][e] = (rr < R && kk < K)
                                  ? load1<CT>(base, dt, (contig_r ? (int64_t)rr + (int64_t)kk * ld
                                                                  : (int64_t)kk + (int64_t)rr * ld))
                                  : CT(0);
                }
            }
        }
    }

    __device__ __forceinline__ void store(CT* sm, bool contig_r, int t) {
        constexpr int LDK = BK + Cfg<CT>::PAD;
#pragma unroll
        for (int q = 0; q < VPT; ++q) {
            if (contig_r) {
                int r = (t % 32) * 4, k = t / 32 + 8 * q;
#pragma unroll
                for (int e = 0; e < 4; ++e) sm[(r + e) * LDK + k] = v[q][e];
            } else {
                constexpr int TPR = BK / 4;
                int r = t / TPR + (NTHR / TPR) * q, k = (t % TPR) * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) sm[r * LDK + k + e] = v[q][e];
            }
        }
    }
};

template <typename CT> struct AccT { typedef f4 type; };
template <> struct AccT<double> { typedef d4 type; };

__device__ __forceinline__ void mma(d4& c, double a, double b) {
    c = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4& c, float a, float b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f4& c, h8 a, h8 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Row of accumulator element r held by lane l inside a 16 x 16 matrix-core tile.
template <typename CT> __device__ __forceinline__ int acc_row(int l, int r) { return 4 * (l / 16) + r; }
template <> __device__ __forceinline__ int acc_row<double>(int l, int r) { return l / 16 + 4 * r; }

// ROLE only separates the symbols of the trailing-update (1) and TRMM (2) launches from the other
// uses (0) so that kernel traces attribute their time; the code is identical.
template <typename CT, bool EDGE, int ROLE>
__global__ __launch_bounds__(NTHR) void k_gemm(const GemmTask* __restrict__ tasks, GemmTask one,
                                               int ntasks, int bmc, int bnc, int xcd_map,
                                               unsigned long long* flags) {
    constexpr int BK = Cfg<CT>::BK;
    constexpr int LDK = BK + Cfg<CT>::PAD;
    __shared__ __attribute__((aligned(16))) CT As[BM * LDK];
    __shared__ __attribute__((aligned(16))) CT Bs[BN * LDK];

    const int bpt = bmc * bnc;
    int64_t b = blockIdx.x;
    int task, blk;
    if (xcd_map) {
        int x = (int)(b % 8);
        int64_t slot = b / 8;
        task = x + 8 * (int)(slot / bpt);
        blk = (int)(slot % bpt);
        if (task >= ntasks) return;
    } else {
        task = (int)(b / bpt);
        blk = (int)(b % bpt);
    }
    const GemmTask& T = tasks ? tasks[task] : one;
    const int m0 = (blk % bmc) * BM, n0 = (blk / bmc) * BN;
    const int t = threadIdx.x, l = t % 64, w = t / 64;
    const int wm = w / 2, wn = w % 2;
    const bool a_contig_r = T.transA == 0;   // A(m, k) at A[m + k*lda]
    const bool b_contig_r = T.transB != 0;   // op(B)(k, n) at B[n + k*ldb]

    typedef typename AccT<CT>::type Acc;
    Acc acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    SlabLoader<CT, EDGE> la, lb;
    const int nk = (T.K + BK - 1) / BK;
    la.load(T.A, T.ta, T.lda, a_contig_r, m0, 0, T.M, T.K, t);
    lb.load(T.B, T.tb, T.ldb, b_contig_r, n0, 0, T.N, T.K, t);
    for (int kb = 0; kb < nk; ++kb) {
        la.store(As, a_contig_r, t);
        lb.store(Bs, b_contig_r, t);
        __syncthreads();
        if (kb + 1 < nk) {
            la.load(T.A, T.ta, T.lda, a_contig_r, m0, (kb + 1) * BK, T.M, T.K, t);
            lb.load(T.B, T.tb, T.ldb, b_contig_r, n0, (kb + 1) * BK, T.N, T.K, t);
        }
        if constexpr (sizeof(CT) == 2) {
            h8 af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                af[i] = *reinterpret_cast<const h8*>(&As[(wm * 64 + i * 16 + l % 16) * LDK + 8 * (l / 16)]);
                bf[i] = *reinterpret_cast<const h8*>(&Bs[(wn * 64 + i * 16 + l % 16) * LDK + 8 * (l / 16)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) mma(acc[i][j], af[i], bf[j]);
        } else {
            CT af[4][4], bf[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    af[i][e] = As[(wm * 64 + i * 16 + l % 16) * LDK + 4 * (l / 16) + e];
                    bf[i][e] = Bs[(wn * 64 + i * 16 + l % 16) * LDK + 4 * (l / 16) + e];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mma(acc[i][j], af[i][e], bf[j][e]);
        }
        __syncthreads();
    }

    // Epilogue: C = alpha * acc + beta * C in the output's precision.
    bool ovf = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int row = m0 + wm * 64 + i * 16 + acc_row<CT>(l, r);
                int col = n0 + wn * 64 + j * 16 + l % 16;
                if (EDGE && (row >= T.M || col >= T.N)) continue;
                int64_t ci = (int64_t)row + (int64_t)col * T.ldc;
                if (T.tc == DT_F64) {
                    double* C = static_cast<double*>(T.C);
                    double v = T.alpha * (double)acc[i][j][r];
                    if (T.beta != 0.0) v += T.beta * C[ci];
                    C[ci] = v;
                } else if (T.tc == DT_F32) {
                    float* C = static_cast<float*>(T.C);
                    float v = (float)T.alpha * (float)acc[i][j][r];
                    if (T.beta != 0.0) v += (float)T.beta * C[ci];
                    C[ci] = v;
                } else if constexpr (sizeof(CT) == 8) {
                    _Float16* C = static_cast<_Float16*>(T.C);
                    double v = T.alpha * acc[i][j][r];
                    if (T.beta != 0.0) v += T.beta * (double)C[ci];
                    _Float16 h = f64_to_f16(v);
                    if (__builtin_isinf((float)h) && !__builtin_isinf(v)) ovf = true;
                    C[ci] = h;
                } else {
                    _Float16* C = static_cast<_Float16*>(T.C);
                    float v = (float)T.alpha * (float)acc[i][j][r];
                    if (T.beta != 0.0) v += (float)T.beta * (float)C[ci];
                    _Float16 h = (_Float16)v;
                    if (__builtin_isinf((float)h) && !__builtin_isinf(v)) ovf = true;
                    C[ci] = h;
                }
            }
    if (ovf && flags) atomicOr(&flags[FLAG_FP16_OVF], 1ull);
}

template <typename CT, int ROLE>
static int launch_ct(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks,
                     const GemmTask& one) {
    constexpr int BK = Cfg<CT>::BK;
    const int M = one.M, N = one.N, K = one.K;
    if (M <= 0 || N <= 0 || ntasks <= 0) return GPEX_OK;
    const int bmc = (M + BM - 1) / BM, bnc = (N + BN - 1) / BN;
    // The vector path needs whole blocks, leading dimensions that keep 4-element groups
    // 16-byte aligned, and aligned base pointers (checked on the representative task).
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    bool fast = (M % BM == 0) && (N % BN == 0) && (K % BK == 0) && (one.lda % 4 == 0) &&
                (one.ldb % 4 == 0) && al(one.A) && al(one.B);
    const int bpt = bmc * bnc;
    int xcd = ntasks >= 8 ? 1 : 0;
    int64_t grid = xcd ? (int64_t)8 * ((ntasks + 7) / 8) * bpt : (int64_t)ntasks * bpt;
    if (grid > 0x7fffffffLL) return set_err(ctx, GPEX_ERR_ARG, "gemm grid too large");
    unsigned long long* fl = reinterpret_cast<unsigned long long*>(ctx->d_flags);
    if (fast)
        hipLaunchKernelGGL((k_gemm<CT, false, ROLE>), dim3((unsigned)grid), dim3(NTHR), 0, s, d_tasks, one,
                           ntasks, bmc, bnc, xcd, fl);
    else
        hipLaunchKernelGGL((k_gemm<CT, true, ROLE>), dim3((unsigned)grid), dim3(NTHR), 0, s, d_tasks, one,
                           ntasks, bmc, bnc, xcd, fl);
    GPEX_HIP(ctx, hipGetLastError());
    return GPEX_OK;
}

template <int ROLE>
static int launch_role(gpex_ctx_t ctx, hipStream_t s, int compute, const GemmTask* d_tasks, int ntasks,
                       const GemmTask& one) {
    if (compute == DT_F64) return launch_ct<double, ROLE>(ctx, s, d_tasks, ntasks, one);
    if (compute == DT_F32) return launch_ct<float, ROLE>(ctx, s, d_tasks, ntasks, one);
    return launch_ct<_Float16, ROLE>(ctx, s, d_tasks, ntasks, one);
}

int gemm_launch(gpex_ctx_t ctx, hipStream_t s, int compute, const GemmTask* d_tasks, int ntasks,
                const GemmTask& one, int role) {
    if (role == GEMM_UPDATE) return launch_role<GEMM_UPDATE>(ctx, s, compute, d_tasks, ntasks, one);
    if (role == GEMM_TRMM) return launch_role<GEMM_TRMM>(ctx, s, compute, d_tasks, ntasks, one);
    return launch_role<GEMM_GENERIC>(ctx, s, compute, d_tasks, ntasks, one);
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

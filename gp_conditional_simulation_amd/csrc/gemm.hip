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
#include <type_traits>
#include "common.h"
#include "devutil.h"

namespace gpex {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, NTHR = 256;

// Wave grid of FP16 TRMM launches: -1 = chosen per launch (2 x 4 waves when that still gives at
// least 2048 workgroups, else 2 x 2), 0 = 2 x 2 waves (128 x 128), 1 = 4 x 2, 2 = 2 x 4.
int g_f16_grid = -1;
int g_gemm_interleave = 1;

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

// Register fragment of one matrix-core step: one element per lane (FP64/FP32), 8 (FP16).
template <typename CT> struct FragT { typedef CT type; };
template <> struct FragT<_Float16> { typedef h8 type; };

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
    if ((T.tri & TRI_C_LOWER) && n0 >= m0 + BM) return;   // block strictly above the diagonal
    int kend = T.K;                                       // products beyond kend are exact zeros
    if (T.tri & TRI_A_LOWER) kend = min(kend, m0 + BM);
    if (T.tri & TRI_B_UPPER) kend = min(kend, n0 + BN);
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
    const int nk = (kend + BK - 1) / BK;
    la.load(T.A, T.ta, T.lda, a_contig_r, m0, 0, T.M, kend, t);
    lb.load(T.B, T.tb, T.ldb, b_contig_r, n0, 0, T.N, kend, t);
    for (int kb = 0; kb < nk; ++kb) {
        la.store(As, a_contig_r, t);
        lb.store(Bs, b_contig_r, t);
        __syncthreads();
        if (kb + 1 < nk) {
            la.load(T.A, T.ta, T.lda, a_contig_r, m0, (kb + 1) * BK, T.M, kend, t);
            lb.load(T.B, T.tb, T.ldb, b_contig_r, n0, (kb + 1) * BK, T.N, kend, t);
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

// ---------------------------------------------------------------------------------------------
// Typed kernel: operand element types fixed at compile time (the hot launches: trailing updates
// and TRMM with uniform operand types), global-address-space operand pointers, K slabs of 32
// (FP64/FP32) or 64 (FP16) staged through two LDS buffers, one barrier per slab.
template <typename T> struct DtOf;
template <> struct DtOf<double> { static constexpr int v = DT_F64; };
template <> struct DtOf<float> { static constexpr int v = DT_F32; };
template <> struct DtOf<_Float16> { static constexpr int v = DT_F16; };

template <typename T> using gptr = const __attribute__((address_space(1))) T*;
template <typename T> using gptr_mut = __attribute__((address_space(1))) T*;

template <typename CT> struct TCfg;
template <> struct TCfg<double> { static constexpr int BK = 16, PAD = 2, KSTEP = 4; };
template <> struct TCfg<float> { static constexpr int BK = 32, PAD = 4, KSTEP = 4; };
template <> struct TCfg<_Float16> { static constexpr int BK = 64, PAD = 8, KSTEP = 32; };

template <typename CT, typename T> __device__ __forceinline__ CT to_ct(T v);
template <> __device__ __forceinline__ double to_ct<double, double>(double v) { return v; }
template <> __device__ __forceinline__ double to_ct<double, float>(float v) { return (double)v; }
template <> __device__ __forceinline__ double to_ct<double, _Float16>(_Float16 v) { return (double)v; }
template <> __device__ __forceinline__ float to_ct<float, double>(double v) { return (float)v; }
template <> __device__ __forceinline__ float to_ct<float, float>(float v) { return v; }
template <> __device__ __forceinline__ float to_ct<float, _Float16>(_Float16 v) { return (float)v; }
template <> __device__ __forceinline__ _Float16 to_ct<_Float16, double>(double v) { return f64_to_f16(v); }
template <> __device__ __forceinline__ _Float16 to_ct<_Float16, float>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ _Float16 to_ct<_Float16, _Float16>(_Float16 v) { return v; }

template <typename T, int N> struct VN { typedef T __attribute__((ext_vector_type(N))) type; };

// One operand slab (128 rows x BK) of the typed kernel.  CR: the row index is contiguous in
// global memory.  LDS layout: FP64/FP32 operands with CR are kept as [k][row] (row stride LDR,
// padded so that the four lane groups of a fragment read hit different banks; stores are plain
// vector writes); all other operands as [row][k] (k contiguous, the FP16 fragments need 8
// consecutive k per lane).
template <typename CT, typename T, bool CR, bool EDGE, int ROWS = 128, int THREADS = NTHR>
struct TSlab {
    static constexpr int BK = TCfg<CT>::BK;
    static constexpr bool KROW = CR && sizeof(CT) >= 4;        // [k][row] layout
    static constexpr int LDK = BK + TCfg<CT>::PAD;               // [row][k] row stride
    static constexpr int LDR = ROWS + (sizeof(CT) == 8 ? 4 : 8); // [k][row] k stride
    static constexpr int ELEMS = KROW ? BK * LDR : ROWS * LDK;
    // Micro-block path (FP16 compute, row index contiguous): each thread loads MR consecutive rows
    // in each of KB consecutive k and writes them transposed, KB consecutive k per row, so that the
    // [row][k] LDS layout the FP16 fragments need is filled with 2 KB-byte stores instead of
    // 2-byte ones.  Consecutive lanes take consecutive k groups of one row block: their stores
    // cover a row contiguously (no bank conflicts) and their loads 64-byte column segments.
    static constexpr bool MB = CR && sizeof(CT) == 2;
    static constexpr int MR = 8;
    static constexpr int KB = MB ? ROWS * BK / (MR * THREADS) : 1;
    static constexpr int KG = BK / KB;                            // k groups per slab (MB)
    static_assert(!MB || (KB >= 2 && ROWS * BK == MR * KB * THREADS), "micro-blocks must tile the slab");
    // elements per vector: 16-byte loads for k-contiguous FP16 operands, MR rows on the
    // micro-block path, else 4 elements
    static constexpr int VE = MB ? MR : (!CR && sizeof(T) == 2 && sizeof(CT) == 2) ? 8 : 4;
    static constexpr int VPT = MB ? 1 : (ROWS * BK / THREADS) / VE;
    static constexpr int TPK = ROWS / VE;                         // threads per k-row (CR)
    static_assert(MB || (VPT >= 1 && (ROWS * BK) % (THREADS * VE) == 0), "slab must split evenly over the threads");
    CT v[MB ? KB : VPT][VE];

    __device__ __forceinline__ static int idx(int row, int k) { return KROW ? k * LDR + row : row * LDK + k; }

    // Vector q of this thread's share of the slab at (r0, k0), from global memory into registers.
    __device__ __forceinline__ void load_q(int q, gptr<T> base, int64_t ld, int r0, int k0, int R, int K, int t) {
        if constexpr (MB) {
            const int r = (t / KG) * MR, k = (t % KG) * KB;
            const int gr = r0 + r;
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int gk = k0 + k + kk;
                if (!EDGE) {
                    typedef typename VN<T, MR>::type VT;
                    VT x = *reinterpret_cast<const __attribute__((address_space(1))) VT*>(base + (int64_t)gr + (int64_t)gk * ld);
#pragma unroll
                    for (int e = 0; e < MR; ++e) v[kk][e] = to_ct<CT, T>(x[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < MR; ++e)
                        v[kk][e] = (gr + e < R && gk < K) ? to_ct<CT, T>(base[(int64_t)(gr + e) + (int64_t)gk * ld]) : CT(0);
                }
            }
            return;
        }
        int r, k;
        if (CR) {
            r = (t % TPK) * VE;
            k = t / TPK + (THREADS / TPK) * q;
        } else {
            constexpr int TPR = BK / VE;
            r = t / TPR + (THREADS / TPR) * q;
            k = (t % TPR) * VE;
        }
        int gr = r0 + r, gk = k0 + k;
        if (!EDGE) {
            int64_t id = CR ? (int64_t)gr + (int64_t)gk * ld : (int64_t)gk + (int64_t)gr * ld;
            typedef typename VN<T, VE>::type VT;
            VT x = *reinterpret_cast<const __attribute__((address_space(1))) VT*>(base + id);
#pragma unroll
            for (int e = 0; e < VE; ++e) v[q][e] = to_ct<CT, T>(x[e]);
        } else {
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                int rr = CR ? gr + e : gr;
                int kk = CR ? gk : gk + e;
                v[q][e] = (rr < R && kk < K)
                              ? to_ct<CT, T>(base[CR ? (int64_t)rr + (int64_t)kk * ld : (int64_t)kk + (int64_t)rr * ld])
                              : CT(0);
            }
        }
    }

    __device__ __forceinline__ void load(gptr<T> base, int64_t ld, int r0, int k0, int R, int K, int t) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) load_q(q, base, ld, r0, k0, R, K, t);
    }

    // Vector q of the registers into the LDS slab.
    __device__ __forceinline__ void store_q(int q, CT* sm, int t) {
        if constexpr (MB) {
            const int r = (t / KG) * MR, k = (t % KG) * KB;
            typedef typename VN<CT, KB>::type WT;
#pragma unroll
            for (int e = 0; e < MR; ++e) {
                WT w;
#pragma unroll
                for (int kk = 0; kk < KB; ++kk) w[kk] = v[kk][e];
                *reinterpret_cast<WT*>(&sm[idx(r + e, k)]) = w;
            }
            return;
        }
        if (CR) {
            int r = (t % TPK) * VE, k = t / TPK + (THREADS / TPK) * q;
#pragma unroll
            for (int e = 0; e < VE; ++e) sm[idx(r + e, k)] = v[q][e];
        } else {
            constexpr int TPR = BK / VE;
            int r = t / TPR + (THREADS / TPR) * q, k = (t % TPR) * VE;
#pragma unroll
            for (int e = 0; e < VE; ++e) sm[idx(r, k + e)] = v[q][e];
        }
    }

    __device__ __forceinline__ void store(CT* sm, int t) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) store_q(q, sm, t);
    }
};

// WMW x WNW waves of 64 x (16 FJ) each: a block of (64 WMW) x (16 FJ WNW) outputs per workgroup,
// two waves per SIMD (accumulators in vector registers: with FJ = 4 they take 128 of them).
template <typename CT, typename TA, typename TB, typename TC, int TRA, int TRB, bool EDGE, int ROLE,
          int WMW = 2, int WNW = 2, int FJ = 4, int INTERLEAVE = 0>
__global__ __launch_bounds__(64 * WMW * WNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_t(const GemmTask* __restrict__ tasks, GemmTask one, int ntasks, int bmc, int bnc, int xcd_map,
              unsigned long long* flags) {
    constexpr int BK = TCfg<CT>::BK;
    constexpr int TBM = 64 * WMW, WTN = 16 * FJ, TBN = WTN * WNW, THR = 64 * WMW * WNW;
    constexpr bool a_contig_r = TRA == 0;
    constexpr bool b_contig_r = TRB != 0;
    typedef TSlab<CT, TA, a_contig_r, EDGE, TBM, THR> SA;
    typedef TSlab<CT, TB, b_contig_r, EDGE, TBN, THR> SB;
    __shared__ __attribute__((aligned(16))) CT As[2][SA::ELEMS];
    __shared__ __attribute__((aligned(16))) CT Bs[2][SB::ELEMS];

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
    const GemmTask T = tasks ? tasks[task] : one;
    if (T.ta != DtOf<TA>::v || T.tb != DtOf<TB>::v || T.tc != DtOf<TC>::v || T.transA != TRA ||
        (T.transB != 0) != (TRB != 0)) {
        if (threadIdx.x == 0 && flags) atomicOr(&flags[FLAG_BADTASK], 1ull);
        return;
    }
    gptr<TA> Ap = (gptr<TA>)T.A;
    gptr<TB> Bp = (gptr<TB>)T.B;
    gptr_mut<TC> Cp = (gptr_mut<TC>)T.C;
    const int m0 = (blk % bmc) * TBM, n0 = (blk / bmc) * TBN;
    if ((T.tri & TRI_C_LOWER) && n0 >= m0 + TBM) return;   // block strictly above the diagonal
    int kend = T.K;                                        // products beyond kend are exact zeros
    if (T.tri & TRI_A_LOWER) kend = min(kend, m0 + TBM);
    if (T.tri & TRI_B_UPPER) kend = min(kend, n0 + TBN);
    const int t = threadIdx.x, l = t % 64, w = t / 64;
    const int wm = w % WMW, wn = w / WMW;
    typedef typename AccT<CT>::type Acc;
    Acc acc[4][FJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = Acc{0, 0, 0, 0};

    SA la;
    SB lb;
    const int nk = (kend + BK - 1) / BK;
    // Operand slabs are prefetched two ahead: slab 0 goes to LDS and slab 1 stays in registers;
    // during slab kb each register vector is stored into the other LDS buffer (slab kb + 1) and
    // then reloaded from global memory with slab kb + 2, spread over the slab's steps.
    la.load(Ap, T.lda, m0, 0, T.M, kend, t);
    lb.load(Bp, T.ldb, n0, 0, T.N, kend, t);
    la.store(As[0], t);
    lb.store(Bs[0], t);
    if (nk > 1) {
        la.load(Ap, T.lda, m0, BK, T.M, kend, t);
        lb.load(Bp, T.ldb, n0, BK, T.N, kend, t);
    }
    __syncthreads();

    // Matrix-core steps: 4 k per step for FP64/FP32 (lane group g supplies k = 4 g + e of a 16-k
    // group), 32 k per step for FP16 (8 consecutive k per lane group).  Fragments are double
    // buffered in registers: step st + 1 is read from LDS while step st's products run, and at the
    // end of a slab the next slab's first fragments are read right after the barrier, before the
    // slab's last products, so the barrier wait does not drain the matrix-core pipe.
    constexpr int KST = sizeof(CT) == 2 ? 32 : 4;
    constexpr int NST = BK / KST;
    static_assert(NST % 2 == 0, "the register double buffer needs an even step count per slab");
    constexpr int NV = SA::VPT + SB::VPT;   // register vectors per thread per slab
    constexpr bool IL = INTERLEAVE != 0;
    typedef typename FragT<CT>::type FT;
    FT fa[2][4], fb[2][FJ];
    auto rd = [&](const CT* as, const CT* bs, int st, FT* af, FT* bf) {
        if constexpr (sizeof(CT) == 2) {
            const int ks = st * 32;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const h8*>(&as[SA::idx(wm * 64 + i * 16 + l % 16, ks + 8 * (l / 16))]);
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                bf[j] = *reinterpret_cast<const h8*>(&bs[SB::idx(wn * WTN + j * 16 + l % 16, ks + 8 * (l / 16))]);
        } else {
            const int kk = (st / 4) * 16 + 4 * (l / 16) + st % 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = as[SA::idx(wm * 64 + i * 16 + l % 16, kk)];
#pragma unroll
            for (int j = 0; j < FJ; ++j) bf[j] = bs[SB::idx(wn * WTN + j * 16 + l % 16, kk)];
        }
    };

    // One slab.  WR: slab kb + 1 exists (its registers are stored and the barrier is taken);
    // LD: slab kb + 2 exists (reloaded into the freed registers).  The last two slabs are peeled
    // off so that every path is straight-line code: the compiler's wait counts then let the
    // deferred products run while the new fragments are in flight.  Scheduling fences keep the
    // order per step: next fragments' LDS reads, this step's share of the register vectors
    // (store, reload), the products; in the last step the barrier and the next slab's first reads
    // come ahead of the deferred products.
    auto slab = [&](int kb, auto wr_t, auto ld_t) {
        constexpr bool WR = decltype(wr_t)::value;
        constexpr bool LD = decltype(ld_t)::value;
        const int cur = kb & 1;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const int p = st & 1, q = p ^ 1;
            if (st + 1 < NST) {
                rd(As[cur], Bs[cur], st + 1, fa[q], fb[q]);
                if constexpr (!IL) __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (WR) {
                // this step's share of the vectors, spread over all but the last step
#pragma unroll
                for (int vq = 0; vq < NV; ++vq) {
                    if (vq * (NST - 1) / NV != st) continue;
                    if (vq < SA::VPT) {
                        la.store_q(vq, As[cur ^ 1], t);
                        if constexpr (LD) la.load_q(vq, Ap, T.lda, m0, (kb + 2) * BK, T.M, kend, t);
                    } else {
                        lb.store_q(vq - SA::VPT, Bs[cur ^ 1], t);
                        if constexpr (LD) lb.load_q(vq - SA::VPT, Bp, T.ldb, n0, (kb + 2) * BK, T.N, kend, t);
                    }
                }
                if (st + 1 == NST) {
                    __syncthreads();
                    rd(As[cur ^ 1], Bs[cur ^ 1], 0, fa[q], fb[q]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j) mma(acc[i][j], fb[p][j], fa[p][i]);
            if constexpr (IL) {
                // one product, then one LDS or global-memory instruction, in turn
#pragma unroll
                for (int g = 0; g < 12; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x0A0, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4 * FJ, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    rd(As[0], Bs[0], 0, fa[0], fb[0]);
    for (int kb = 0; kb + 2 < nk; ++kb) slab(kb, std::true_type{}, std::true_type{});
    if (nk >= 2) slab(nk - 2, std::true_type{}, std::false_type{});
    slab(nk - 1, std::false_type{}, std::false_type{});

    // Epilogue.  The operands went into the matrix cores as (B, A), so fragment (i, j) holds the
    // transposed 16 x 16 block: lane l is row l % 16 and register r is column acc_row(l, r).  The 16
    // lanes of a column then cover 16 consecutive rows of the column-major C (whole cache lines), and
    // each row group's old C values are all loaded before any store, so their latencies overlap.
    bool ovf = false;
    _Float16* __restrict__ C2 = T.C2;
    const bool use_beta = T.beta != 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + i * 16 + l % 16;
        TC cold[FJ][4];
        if (use_beta) {
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = n0 + wn * WTN + j * 16 + acc_row<CT>(l, r);
                    cold[j][r] = (!EDGE || (row < T.M && col < T.N)) ? Cp[(int64_t)row + (int64_t)col * T.ldc]
                                                                     : TC(0);
                }
        }
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = n0 + wn * WTN + j * 16 + acc_row<CT>(l, r);
                if (EDGE && (row >= T.M || col >= T.N)) continue;
                const int64_t ci = (int64_t)row + (int64_t)col * T.ldc;
                double sv;   // the stored value, exactly, for the optional FP16 copy
                if constexpr (sizeof(TC) == 8) {
                    double v = T.alpha * (double)acc[i][j][r];
                    if (use_beta) v += T.beta * (double)cold[j][r];
                    Cp[ci] = v;
                    sv = v;
                } else if constexpr (sizeof(TC) == 4) {
                    float v = (float)T.alpha * (float)acc[i][j][r];
                    if (use_beta) v += (float)T.beta * (float)cold[j][r];
                    Cp[ci] = v;
                    sv = (double)v;
                } else if constexpr (sizeof(CT) == 8) {
                    double v = T.alpha * acc[i][j][r];
                    if (use_beta) v += T.beta * (double)cold[j][r];
                    _Float16 h = f64_to_f16(v);
                    if (__builtin_isinf((float)h) && !__builtin_isinf(v)) ovf = true;
                    Cp[ci] = h;
                    sv = (double)h;
                } else {
                    float v = (float)T.alpha * (float)acc[i][j][r];
                    if (use_beta) v += (float)T.beta * (float)cold[j][r];
                    _Float16 h = (_Float16)v;
                    if (__builtin_isinf((float)h) && !__builtin_isinf(v)) ovf = true;
                    Cp[ci] = h;
                    sv = (double)h;
                }
                if (C2) {
                    _Float16 h2 = f64_to_f16(sv);
                    C2[(int64_t)col + (int64_t)row * T.ldc2] = h2;
                    if (__builtin_isinf((float)h2) && !__builtin_isinf(sv)) ovf = true;
                }
            }
    }
    if (ovf && flags) atomicOr(&flags[FLAG_FP16_OVF], 1ull);
}

// Launch the typed kernel when (ta, tb, tc, transA, transB) match; returns 1 if launched.
template <typename CT, typename TA, typename TB, typename TC, int TRA, int TRB, int ROLE>
static int try_typed(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one,
                     bool fast, int64_t grid, int bmc, int bnc, int xcd, unsigned long long* fl) {
    if (one.ta != DtOf<TA>::v || one.tb != DtOf<TB>::v || one.tc != DtOf<TC>::v) return 0;
    if (one.transA != TRA || (one.transB != 0) != (TRB != 0)) return 0;
    if constexpr (sizeof(CT) == 2 && ROLE == GEMM_TRMM && TRA == 1 && TRB == 0) {
        int choice = g_f16_grid;
        if (choice < 0)
            choice = (one.N % 256 == 0 && (int64_t)ntasks * (one.M / 128) * (one.N / 256) >= 2048) ? 2 : 0;
        if (fast && choice != 0 && one.M % 256 == 0 && one.N % 256 == 0) {
            const bool tall = choice == 1;   // 1: 4 x 2 waves (256 x 128), 2: 2 x 4 waves (128 x 256)
            const int bm = tall ? 256 : 128, bn = tall ? 128 : 256;
            const int bmc2 = one.M / bm, bnc2 = one.N / bn, bpt2 = bmc2 * bnc2;
            int64_t grid2 = xcd ? (int64_t)8 * ((ntasks + 7) / 8) * bpt2 : (int64_t)ntasks * bpt2;
            if (tall && g_gemm_interleave)
                hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 4, 2, 4, 1>), dim3((unsigned)grid2),
                                   dim3(512), 0, s, d_tasks, one, ntasks, bmc2, bnc2, xcd, fl);
            else if (tall)
                hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 4, 2>), dim3((unsigned)grid2),
                                   dim3(512), 0, s, d_tasks, one, ntasks, bmc2, bnc2, xcd, fl);
            else if (g_gemm_interleave)
                hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 4, 4, 1>), dim3((unsigned)grid2),
                                   dim3(512), 0, s, d_tasks, one, ntasks, bmc2, bnc2, xcd, fl);
            else
                hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 4>), dim3((unsigned)grid2),
                                   dim3(512), 0, s, d_tasks, one, ntasks, bmc2, bnc2, xcd, fl);
            return 1;
        }
    }
    if (fast && g_gemm_interleave)
        hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 2, 4, 1>), dim3((unsigned)grid),
                           dim3(NTHR), 0, s, d_tasks, one, ntasks, bmc, bnc, xcd, fl);
    else if (fast)
        hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE>), dim3((unsigned)grid), dim3(NTHR), 0, s,
                           d_tasks, one, ntasks, bmc, bnc, xcd, fl);
    else
        hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, true, ROLE>), dim3((unsigned)grid), dim3(NTHR), 0, s,
                           d_tasks, one, ntasks, bmc, bnc, xcd, fl);
    return 1;
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
    // typed fast kernels for the operand-type combinations of the hot launches
    bool tfast = (M % BM == 0) && (N % BN == 0) && (K % TCfg<CT>::BK == 0) && (one.lda % 8 == 0) &&
                 (one.ldb % 8 == 0) && al(one.A) && al(one.B);
    // NT form (trailing updates, panel solves), NN form (TRMM, blocked solves) and TN form with uniform
    // types, and the TRMM/TRSM operand mixes
    int done = try_typed<CT, CT, CT, CT, 0, 1, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
    if (!done) done = try_typed<CT, CT, CT, CT, 0, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
    // TN form (conditioning product W^T R, transposed blocked solves)
    if (!done) done = try_typed<CT, CT, CT, CT, 1, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
    if constexpr (sizeof(CT) == 2) {
        if (!done) done = try_typed<CT, _Float16, _Float16, double, 1, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
        if (!done) done = try_typed<CT, double, _Float16, double, 0, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
        if (!done) done = try_typed<CT, float, _Float16, double, 0, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
        if (!done) done = try_typed<CT, _Float16, _Float16, double, 0, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
    }
    if constexpr (sizeof(CT) == 4) {
        if (!done) done = try_typed<CT, double, _Float16, double, 0, 0, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
    }
    if constexpr (sizeof(CT) == 8) {
        if (!done) done = try_typed<CT, float, double, float, 0, 1, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
        if (!done) done = try_typed<CT, _Float16, double, _Float16, 0, 1, ROLE>(ctx, s, d_tasks, ntasks, one, tfast, grid, bmc, bnc, xcd, fl);
    }
    if (done) {
        GPEX_HIP(ctx, hipGetLastError());
        return GPEX_OK;
    }
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

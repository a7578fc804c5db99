// Batched mixed-precision tile GEMM on gfx950 matrix cores: the kernel template and its launch
// logic, shared by one translation unit per compute precision (gemm_f64.hip, gemm_f32.hip,
// gemm_f16.hip) so that the three compile in parallel.
//
// This is the workhorse of the adaptive mixed-precision tile Cholesky ("Mixed-Precision GPU
// Acceleration for Confidence Regions of Spatial Excursion Sets", Sec. IV-B: each tile task runs
// in the precision of its output tile with the operands converted to it), of the panel solves,
// of kriging (Sec. V-A), of the simulation product (Algorithm 1) and of the conditioning product
// (Eq. 7).
//
// Design (gfx950, wave64):
//   * A workgroup computes one block of C: 2 x 2 waves of 64 x 64 (128 x 128, 256 threads), or
//     2 x 4 waves (128 x 256) for large simulation products.  Each wave's 64 x 64 sub-block is
//     4 x 4 matrix-core tiles of 16 x 16, accumulated in vector registers.  Large FP16 row panels
//     of the simulation product go to a dedicated 256 x 256 kernel instead (panel16.h).
//   * FP64: v_mfma_f64_16x16x4 (lane l, acc r -> row l/16 + 4r, col l%16).
//     FP32: v_mfma_f32_16x16x4 (row 4(l/16) + r, col l%16).
//     FP16: v_mfma_f32_16x16x32_f16 with FP32 accumulation (row 4(l/16) + r, col l%16).
//   * Operand slabs (K = 16 FP64, 32 FP32, 64 FP16) are staged through two LDS buffers and
//     prefetched two slabs ahead through registers; global loads are coalesced along whichever
//     index is contiguous in memory and converted on the fly to the compute type (FP64 -> FP16
//     goes through round-to-odd FP32, which makes the final FP16 rounding a correct
//     round-to-nearest-even).
//   * Element types are template parameters; the hot launches (uniform types, and the operand
//     mixes of the mixed-precision factorization and the simulation product) run fully typed
//     kernels, and one variant that reads the types from the task at run time covers everything
//     else (ragged shapes with mixed types, unaligned operands).
//   * Batched launches place all workgroups of one task on one XCD (workgroups are dealt to the
//     8 XCDs round-robin by index), so a task's operand tiles stream through a single L2.
#pragma once
#include <type_traits>
#include "common.h"
#include "devutil.h"

namespace gpex {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, NTHR = 256;

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

// Element type tag "read from the task at run time" (operand or output).
struct DynT {};
template <typename T> constexpr bool is_dyn = std::is_same<T, DynT>::value;

template <typename T> struct DtOf;
template <> struct DtOf<double> { static constexpr int v = DT_F64; };
template <> struct DtOf<float> { static constexpr int v = DT_F32; };
template <> struct DtOf<_Float16> { static constexpr int v = DT_F16; };

// Whether a task's type code dt is what a kernel built for element type T reads.
template <typename T> __device__ __forceinline__ bool type_ok(int dt) {
    if constexpr (is_dyn<T>) return dt == DT_F64 || dt == DT_F32 || dt == DT_F16;
    else return dt == DtOf<T>::v;
}

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

// One operand slab (ROWS rows x BK) of the kernel.  T: the operand's element type in global
// memory (DynT: read from dt, element by element, ragged-shape kernels only).  CR: the row index
// is contiguous in global memory.  LDS layout: FP64/FP32 operands with CR are kept as [k][row] (row stride LDR,
// padded so that the four lane groups of a fragment read hit different banks; stores are plain
// vector writes); all other operands as [row][k] (k contiguous, the FP16 fragments need 8
// consecutive k per lane).  FP16 rows are not padded: their 16-byte chunks of 8 k are stored in
// the order chunk ^ (row mod 8), so the 16 rows that one fragment read touches at one chunk
// index fall on 8 different chunk positions (with a padded row stride they took 2-way bank
// conflicts).
template <typename CT, typename T, bool CR, bool EDGE, int ROWS = 128, int THREADS = NTHR>
struct TSlab {
    static constexpr int BK = TCfg<CT>::BK;
    static constexpr bool KROW = CR && sizeof(CT) >= 4;        // [k][row] layout
    static constexpr bool SWZ = !KROW && sizeof(CT) == 2;       // [row][k] with XOR-swizzled 16-byte chunks
    static_assert(!SWZ || BK == 64, "the FP16 chunk swizzle assumes 8 chunks of 8 k per row");
    static constexpr int LDK = SWZ ? BK : BK + TCfg<CT>::PAD;    // [row][k] row stride
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
    static_assert(EDGE || !is_dyn<T>, "run-time element types are read element by element");
    CT v[MB ? KB : VPT][VE];
    int dt = 0;   // element type code of a DynT operand

    // Element i of the operand, converted to the compute type.
    __device__ __forceinline__ CT get(gptr<T> base, int64_t i) const {
        if constexpr (is_dyn<T>) {
            if (dt == DT_F64) return to_ct<CT, double>(((gptr<double>)base)[i]);
            if (dt == DT_F32) return to_ct<CT, float>(((gptr<float>)base)[i]);
            return to_ct<CT, _Float16>(((gptr<_Float16>)base)[i]);
        } else {
            return to_ct<CT, T>(base[i]);
        }
    }

    __device__ __forceinline__ static int idx(int row, int k) {
        if constexpr (KROW) return k * LDR + row;
        if constexpr (SWZ) return row * LDK + ((((k >> 3) ^ (row & 7)) << 3) | (k & 7));
        return row * LDK + k;
    }

    // Vector q of this thread's share of the slab at (r0, k0), from global memory into registers.
    __device__ __forceinline__ void load_q(int q, gptr<T> base, int64_t ld, int r0, int k0, int R, int K, int t) {
        if constexpr (MB) {
            const int r = (t / KG) * MR, k = (t % KG) * KB;
            const int gr = r0 + r;
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int gk = k0 + k + kk;
                if constexpr (!EDGE) {
                    typedef typename VN<T, MR>::type VT;
                    VT x = *reinterpret_cast<const __attribute__((address_space(1))) VT*>(base + (int64_t)gr + (int64_t)gk * ld);
#pragma unroll
                    for (int e = 0; e < MR; ++e) v[kk][e] = to_ct<CT, T>(x[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < MR; ++e)
                        v[kk][e] = (gr + e < R && gk < K) ? get(base, (int64_t)(gr + e) + (int64_t)gk * ld) : CT(0);
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
        if constexpr (!EDGE) {
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
                              ? get(base, CR ? (int64_t)rr + (int64_t)kk * ld : (int64_t)kk + (int64_t)rr * ld)
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
            if constexpr (SWZ) {
                // VE consecutive k (a whole or half 16-byte chunk) stay together under the swizzle
                typedef typename VN<CT, VE>::type WT;
                WT w;
#pragma unroll
                for (int e = 0; e < VE; ++e) w[e] = v[q][e];
                *reinterpret_cast<WT*>(&sm[idx(r, k)]) = w;
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) sm[idx(r, k + e)] = v[q][e];
            }
        }
    }

    __device__ __forceinline__ void store(CT* sm, int t) {
#pragma unroll
        for (int q = 0; q < VPT; ++q) store_q(q, sm, t);
    }
};

// A launch covers bmc x bnc blocks of every task, the block grid starting at row m_off and column
// n_off of C (a launch may cover only part of C: the whole-block part and its ragged strips go to
// separate launches).
// WMW x WNW waves of 64 x (16 FJ) each: a block of (64 WMW) x (16 FJ WNW) outputs per workgroup,
// two waves per SIMD (accumulators in vector registers: with FJ = 4 they take 128 of them; the
// run-time-typed variant may drop to one wave per SIMD for the registers its loads need).
// INTERLEAVE: products and memory instructions issued one by one (whole-block launches).  ROLE
// only separates the symbols of trailing updates (1) and the simulation product (2) from the
// other uses (0) so that kernel traces attribute their time.
// EMU: FP16 destination storage between k-tasks (GemmTask::kround; FP32-accumulating compute
// types, FP64 output, whole blocks only).
template <typename CT, typename TA, typename TB, typename TC, int TRA, int TRB, bool EDGE, int ROLE,
          int WMW = 2, int WNW = 2, int FJ = 4, int INTERLEAVE = 0, bool EMU = false>
__global__ __launch_bounds__(64 * WMW * WNW)
__attribute__((amdgpu_waves_per_eu(is_dyn<TA> ? 1 : 2, 2)))
void k_gemm_t(const GemmTask* __restrict__ tasks, GemmTask one, int ntasks, int bmc, int bnc, int m_off,
              int n_off, int xcd_map, unsigned long long* flags) {
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
    // The task through the scalar data cache in one go (the index is the same for the whole
    // workgroup): field-by-field loads through the vector path waited for each other in turn.
    GemmTask T = one;
    if (tasks) {
        static_assert(sizeof(GemmTask) % 8 == 0, "task read as 8-byte words");
        const __attribute__((address_space(4))) uint64_t* src =
            (const __attribute__((address_space(4))) uint64_t*)(tasks + task);
        uint64_t w[sizeof(GemmTask) / 8];
#pragma unroll
        for (int i = 0; i < (int)(sizeof(GemmTask) / 8); ++i) w[i] = src[i];
        __builtin_memcpy(&T, w, sizeof(GemmTask));
    }
    if (!type_ok<TA>(T.ta) || !type_ok<TB>(T.tb) || !type_ok<TC>(T.tc) || T.transA != TRA ||
        (T.transB != 0) != (TRB != 0) || T.kdup != 0) {
        if (threadIdx.x == 0 && flags) atomicOr(&flags[FLAG_BADTASK], 1ull);
        return;
    }
    gptr<TA> Ap = (gptr<TA>)T.A;
    gptr<TB> Bp = (gptr<TB>)T.B;
    const int m0 = m_off + (blk % bmc) * TBM, n0 = n_off + (blk / bmc) * TBN;   // block origin in the task
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

    static_assert(!EMU || (!EDGE && sizeof(CT) <= 4 && std::is_same<TC, double>::value),
                  "FP16 destination emulation: typed whole-block kernels with FP64 output");
    // stored part of C (simulation product: the caller's rows and columns; else all of C)
    const int m_st = (ROLE == GEMM_TRMM && T.m_store) ? T.m_store : T.M;
    const int n_st = (ROLE == GEMM_TRMM && T.n_store) ? T.n_store : T.N;
    if constexpr (EMU) {
        // the destination enters the accumulator (it holds FP16 values: exact in FP32)
        if (T.beta != 0.0) {
            gptr<double> Cq = (gptr<double>)T.C;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = m0 + wm * 64 + i * 16 + l % 16;
                        const int col = n0 + wn * WTN + j * 16 + acc_row<CT>(l, r);
                        // clamped, in-bounds reads outside the stored part (never written back)
                        acc[i][j][r] = (float)(T.beta * Cq[(int64_t)min(row, m_st - 1) + (int64_t)min(col, n_st - 1) * T.ldc]);
                    }
        }
    }
    // round the accumulator to FP16 (the destination store of one k-task).  The lambdas that touch
    // the accumulator are forced inline: when the FP16-destination variant grew past the inliner's
    // threshold, the accumulators went to scratch memory and that kernel ran 16x slower.
    auto round16 = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][r] = (float)(_Float16)acc[i][j][r];
    };
    auto task_end = [&](int kb) __attribute__((always_inline)) {
        if constexpr (EMU) {
            if (((kb + 1) * BK) % T.kround == 0) round16();
        }
    };

    SA la;
    SB lb;
    la.dt = T.ta;
    lb.dt = T.tb;
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
    auto rd = [&](const CT* as, const CT* bs, int st, FT* af, FT* bf) __attribute__((always_inline)) {
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
    auto slab = [&](int kb, auto wr_t, auto ld_t) __attribute__((always_inline)) {
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
    for (int kb = 0; kb + 2 < nk; ++kb) {
        slab(kb, std::true_type{}, std::true_type{});
        task_end(kb);
    }
    if (nk >= 2) {
        slab(nk - 2, std::true_type{}, std::false_type{});
        task_end(nk - 2);
    }
    slab(nk - 1, std::false_type{}, std::false_type{});
    if constexpr (EMU) round16();   // the end of the K loop ends the last task

    // Epilogue.  The operands went into the matrix cores as (B, A), so fragment (i, j) holds the
    // transposed 16 x 16 block: lane l is row l % 16 and register r is column acc_row(l, r).  The 16
    // lanes of a column then cover 16 consecutive rows of the column-major C (whole cache lines), and
    // each row group's old C values are all loaded before any store, so their latencies overlap.
    bool ovf = false;
    _Float16* __restrict__ C2 = T.C2;
    float* __restrict__ C3 = T.C3;
    double* __restrict__ C4 = T.C4;
    const bool use_beta = !EMU && T.beta != 0.0;   // EMU: the destination is in the accumulator
    auto epilogue = [&](auto out_tag) {   // out_tag: a value of the output element type
        typedef decltype(out_tag) TO;
        gptr_mut<TO> Cp = (gptr_mut<TO>)T.C;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = m0 + wm * 64 + i * 16 + l % 16;
            TO cold[FJ][4];
            if (use_beta) {
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int col = n0 + wn * WTN + j * 16 + acc_row<CT>(l, r);
                        if constexpr (ROLE == GEMM_TRMM && !EDGE) {
                            // outside the stored part (never written back) read a clamped, in-bounds
                            // element: the loads stay unconditional and issue together
                            cold[j][r] = Cp[(int64_t)min(row, m_st - 1) + (int64_t)min(col, n_st - 1) * T.ldc];
                        } else {
                            bool in = !EDGE || (row < T.M && col < T.N);
                            if constexpr (ROLE == GEMM_TRMM) in = in && row < m_st && col < n_st;
                            cold[j][r] = in ? Cp[(int64_t)row + (int64_t)col * T.ldc] : TO(0);
                        }
                    }
            }
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = n0 + wn * WTN + j * 16 + acc_row<CT>(l, r);
                    if (EDGE && (row >= T.M || col >= T.N)) continue;
                    if constexpr (ROLE == GEMM_TRMM) {
                        if (row >= m_st || col >= n_st) continue;
                    }
                    const int64_t ci = (int64_t)row + (int64_t)col * T.ldc;
                    double sv;   // the stored value, exactly, for the optional copies
                    if constexpr (sizeof(TO) == 8) {
                        double v = T.alpha * (double)acc[i][j][r];
                        if (use_beta) v += T.beta * (double)cold[j][r];
                        Cp[ci] = v;
                        sv = v;
                    } else if constexpr (sizeof(TO) == 4) {
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
                    if constexpr (ROLE == GEMM_GENERIC && sizeof(CT) == 8) {
                        // extra outputs of the panel solves (FP64 compute, generic role)
                        if (C2) {
                            _Float16 h2 = f64_to_f16(sv);
                            C2[(int64_t)col + (int64_t)row * T.ldc2] = h2;
                            if (__builtin_isinf((float)h2) && !__builtin_isinf(sv)) ovf = true;
                        }
                        if (C3) C3[ci] = (float)sv;            // the values the update kernels convert on load
                        if (C4) C4[ci] = sv;
                    }
                }
        }
    };
    if constexpr (is_dyn<TC>) {
        if (T.tc == DT_F64) epilogue(double{});
        else if (T.tc == DT_F32) epilogue(float{});
        else epilogue(_Float16{});
    } else {
        epilogue(TC{});
    }
    if (ovf && flags) atomicOr(&flags[FLAG_FP16_OVF], 1ull);
}

}  // namespace gpex

#include "panel16.h"

namespace gpex {

__attribute__((unused)) static __global__ void k_flag_badtask(unsigned long long* flags) {
    if (flags) atomicOr(&flags[FLAG_BADTASK], 1ull);
}

// Part of the output of a launch: bmc x bnc blocks of 128 x 128 from (m_off, n_off), in every task.
struct Part {
    int m_off, n_off, bmc, bnc;
    bool fast;   // whole blocks and slabs with aligned operands: vector loads, no bounds checks
};

static inline int64_t part_grid(const Part& p, int ntasks, int xcd) {
    const int64_t bpt = (int64_t)p.bmc * p.bnc;
    return xcd ? (int64_t)8 * ((ntasks + 7) / 8) * bpt : (int64_t)ntasks * bpt;
}

// Launch the typed kernel on one part when (ta, tb, tc, transA, transB) match; returns 1 if
// launched.  A part that needs bounds checks runs the bounds-checked variant when RAGGED
// instantiates it, and otherwise returns 0 (the run-time-typed kernel takes it).
template <typename CT, typename TA, typename TB, typename TC, int TRA, int TRB, int ROLE, bool RAGGED = false>
static int try_typed(hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, const Part& p, int xcd,
                     unsigned long long* fl) {
    if (one.ta != DtOf<TA>::v || one.tb != DtOf<TB>::v || one.tc != DtOf<TC>::v) return 0;
    if (one.transA != TRA || (one.transB != 0) != (TRB != 0)) return 0;
    const unsigned grid = (unsigned)part_grid(p, ntasks, xcd);
    if constexpr (sizeof(CT) == 2 && ROLE == GEMM_TRMM && TRA == 1 && TRB == 0 && std::is_same<TA, _Float16>::value &&
                  std::is_same<TB, _Float16>::value && std::is_same<TC, double>::value) {
        // row panels of the simulation product: 256 x 256 blocks (panel16.h) when the part is all
        // of C and that still leaves at least one workgroup per CU
        const bool whole = p.fast && p.m_off == 0 && p.n_off == 0 && p.bmc * BM == one.M && p.bnc * BN == one.N;
        if (whole && panel16_takes(one, ntasks)) {
            const Part w{0, 0, one.M / P16_BM, one.N / P16_BN, true};
            hipLaunchKernelGGL(k_panel16<0>, dim3((unsigned)part_grid(w, ntasks, xcd)), dim3(P16_THR), 0, s, d_tasks,
                               ntasks, w.bmc, w.bnc, xcd, fl);
            return 1;
        }
    }
    if constexpr (ROLE == GEMM_TRMM && sizeof(CT) <= 4 && std::is_same<TC, double>::value) {
        if (one.kround) {   // FP16 destination emulation: 128 x 128 blocks, whole blocks only
            if (!p.fast) return 0;
            hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 2, 4, 1, true>), dim3(grid), dim3(NTHR),
                               0, s, d_tasks, one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
            return 1;
        }
    }
    if (!p.fast) {
        if constexpr (RAGGED) {
            hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, true, ROLE>), dim3(grid), dim3(NTHR), 0, s, d_tasks,
                               one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
            return 1;
        }
        return 0;
    }
    if constexpr (sizeof(CT) == 2 && ROLE == GEMM_TRMM && TRA == 1 && TRB == 0) {
        // 2 x 4 waves (128 x 256 blocks) when the part is all of C and that still leaves at least
        // 2048 workgroups
        const bool whole = p.m_off == 0 && p.n_off == 0 && p.bmc * 128 == one.M && p.bnc * 128 == one.N;
        const bool wide = whole && one.N % 256 == 0 &&
                          (g_f16_grid < 0 ? (int64_t)ntasks * (one.M / 128) * (one.N / 256) >= 2048 : g_f16_grid != 0);
        if (wide) {
            const Part w{0, 0, one.M / 128, one.N / 256, true};
            hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 4, 4, 1>),
                               dim3((unsigned)part_grid(w, ntasks, xcd)), dim3(512), 0, s, d_tasks, one, ntasks, w.bmc,
                               w.bnc, 0, 0, xcd, fl);
            return 1;
        }
    }
    if constexpr (sizeof(CT) == 4 && ROLE == GEMM_TRMM && TRA == 0 && TRB == 0 && sizeof(TA) == 8) {
        // diagonal tiles of the simulation product: 2 x 4 waves (128 x 256 blocks) read each FP64
        // tile half as often as 128 x 128 blocks
        const bool whole = p.m_off == 0 && p.n_off == 0 && p.bmc * 128 == one.M && p.bnc * 128 == one.N;
        if (whole && one.N % 256 == 0) {
            const Part w{0, 0, one.M / 128, one.N / 256, true};
            hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 4, 4, 1>),
                               dim3((unsigned)part_grid(w, ntasks, xcd)), dim3(512), 0, s, d_tasks, one, ntasks, w.bmc,
                               w.bnc, 0, 0, xcd, fl);
            return 1;
        }
    }
    hipLaunchKernelGGL((k_gemm_t<CT, TA, TB, TC, TRA, TRB, false, ROLE, 2, 2, 4, 1>), dim3(grid), dim3(NTHR), 0, s,
                       d_tasks, one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
    return 1;
}

// Trailing-update operand mixes of the mixed-precision factorization: C (type CT) -= A B^T with A
// and B in any of the three tile precisions.
template <typename CT, typename TA>
static int try_update_row(hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, const Part& p,
                          int xcd, unsigned long long* fl) {
    int done = try_typed<CT, TA, double, CT, 0, 1, GEMM_UPDATE>(s, d_tasks, ntasks, one, p, xcd, fl);
    if (!done) done = try_typed<CT, TA, float, CT, 0, 1, GEMM_UPDATE>(s, d_tasks, ntasks, one, p, xcd, fl);
    if (!done) done = try_typed<CT, TA, _Float16, CT, 0, 1, GEMM_UPDATE>(s, d_tasks, ntasks, one, p, xcd, fl);
    return done;
}

// One part of a launch: the typed kernel of the task signature if there is one, else the
// run-time-typed kernel.
template <typename CT, int ROLE>
static void launch_part(hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, const Part& p,
                        int xcd, unsigned long long* fl) {
    // uniform types: NT form (trailing updates, panel solves), NN form (simulation product, blocked
    // solves), TN form (conditioning product W^T R, transposed blocked solves)
    int done = try_typed<CT, CT, CT, CT, 0, 1, ROLE, true>(s, d_tasks, ntasks, one, p, xcd, fl);
    if (!done) done = try_typed<CT, CT, CT, CT, 0, 0, ROLE, true>(s, d_tasks, ntasks, one, p, xcd, fl);
    if (!done) done = try_typed<CT, CT, CT, CT, 1, 0, ROLE, true>(s, d_tasks, ntasks, one, p, xcd, fl);
    if constexpr (ROLE == GEMM_TRMM && sizeof(CT) == 2) {
        // simulation product: FP16 row panels (transposed), or tiles of any precision, times FP16 Z/s
        if (!done) done = try_typed<CT, _Float16, _Float16, double, 1, 0, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
        if (!done) done = try_typed<CT, double, _Float16, double, 0, 0, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
        if (!done) done = try_typed<CT, float, _Float16, double, 0, 0, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
        if (!done) done = try_typed<CT, _Float16, _Float16, double, 0, 0, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
    }
    if constexpr (ROLE == GEMM_TRMM && sizeof(CT) == 4) {
        // simulation product, diagonal tiles: FP64 tile times FP16 Z/s in FP32
        if (!done) done = try_typed<CT, double, _Float16, double, 0, 0, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
    }
    if constexpr (ROLE == GEMM_GENERIC && sizeof(CT) == 8) {
        // panel solves of reduced-precision tiles: L_ik = A_ik T_kk^T in FP64, stored back in the tile's type
        if (!done) done = try_typed<CT, float, double, float, 0, 1, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
        if (!done) done = try_typed<CT, _Float16, double, _Float16, 0, 1, ROLE>(s, d_tasks, ntasks, one, p, xcd, fl);
    }
    if constexpr (ROLE == GEMM_UPDATE) {
        if (!done) done = try_update_row<CT, double>(s, d_tasks, ntasks, one, p, xcd, fl);
        if (!done) done = try_update_row<CT, float>(s, d_tasks, ntasks, one, p, xcd, fl);
        if (!done) done = try_update_row<CT, _Float16>(s, d_tasks, ntasks, one, p, xcd, fl);
    }
    if (done) return;
    if (one.kround) {   // no kernel emulates FP16 destinations for this shape: flag it, compute nothing
        hipLaunchKernelGGL(k_flag_badtask, dim3(1), dim3(1), 0, s, fl);
        return;
    }
    // everything else: element types read from the tasks, bounds-checked element loads
    const dim3 grid((unsigned)part_grid(p, ntasks, xcd));
    if constexpr (ROLE == GEMM_TRMM) {
        // the simulation product stores only the caller's part of C (GemmTask::m_store / n_store),
        // which only the kernels of its own role honour
        switch ((one.transA ? 2 : 0) | (one.transB ? 1 : 0)) {
            case 0:
                hipLaunchKernelGGL((k_gemm_t<CT, DynT, DynT, DynT, 0, 0, true, GEMM_TRMM>), grid, dim3(NTHR), 0, s,
                                   d_tasks, one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
                break;
            case 2:
                hipLaunchKernelGGL((k_gemm_t<CT, DynT, DynT, DynT, 1, 0, true, GEMM_TRMM>), grid, dim3(NTHR), 0, s,
                                   d_tasks, one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
                break;
            default:   // the simulation product has no transposed B
                hipLaunchKernelGGL(k_flag_badtask, dim3(1), dim3(1), 0, s, fl);
                break;
        }
        return;
    }
    switch ((one.transA ? 2 : 0) | (one.transB ? 1 : 0)) {
        case 0:
            hipLaunchKernelGGL((k_gemm_t<CT, DynT, DynT, DynT, 0, 0, true, GEMM_GENERIC>), grid, dim3(NTHR), 0, s, d_tasks,
                               one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
            break;
        case 1:
            hipLaunchKernelGGL((k_gemm_t<CT, DynT, DynT, DynT, 0, 1, true, GEMM_GENERIC>), grid, dim3(NTHR), 0, s, d_tasks,
                               one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
            break;
        case 2:
            hipLaunchKernelGGL((k_gemm_t<CT, DynT, DynT, DynT, 1, 0, true, GEMM_GENERIC>), grid, dim3(NTHR), 0, s, d_tasks,
                               one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
            break;
        default:
            hipLaunchKernelGGL((k_gemm_t<CT, DynT, DynT, DynT, 1, 1, true, GEMM_GENERIC>), grid, dim3(NTHR), 0, s, d_tasks,
                               one, ntasks, p.bmc, p.bnc, p.m_off, p.n_off, xcd, fl);
            break;
    }
}

template <typename CT, int ROLE>
static int launch_ct(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one) {
    const int M = one.M, N = one.N, K = one.K;
    if (M <= 0 || N <= 0 || ntasks <= 0) return GPEX_OK;
    const int bmc = (M + BM - 1) / BM, bnc = (N + BN - 1) / BN;
    const int xcd = ntasks >= 8 ? 1 : 0;
    if (part_grid(Part{0, 0, bmc, bnc, false}, ntasks, xcd) > 0x7fffffffLL)
        return set_err(ctx, GPEX_ERR_ARG, "gemm grid too large");
    unsigned long long* fl = reinterpret_cast<unsigned long long*>(ctx->d_flags);
    // The vector path needs whole slabs, leading dimensions that keep 16-byte groups aligned, and
    // aligned base pointers (checked on the representative task).  When only M or N is ragged, the
    // whole 128-blocks run the vector path and the leftover strips (fewer than 128 rows at the
    // bottom, fewer than 128 columns at the right) the bounds-checked one.
    auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    const bool kfast = (K % TCfg<CT>::BK == 0) && (one.lda % 8 == 0) && (one.ldb % 8 == 0) && al(one.A) && al(one.B);
    const int mw = kfast ? M / BM : 0, nw = kfast ? N / BN : 0;   // whole block rows / columns
    if (mw == bmc && nw == bnc) {
        launch_part<CT, ROLE>(s, d_tasks, ntasks, one, Part{0, 0, mw, nw, true}, xcd, fl);
    } else if ((int64_t)mw * nw * ntasks < 512) {
        // few whole blocks: one bounds-checked launch costs less than three on the critical path
        launch_part<CT, ROLE>(s, d_tasks, ntasks, one, Part{0, 0, bmc, bnc, false}, xcd, fl);
    } else if (ctx->serial) {
        // serial mode: the same three launches, one after the other on the launching stream
        if (mw < bmc) launch_part<CT, ROLE>(s, d_tasks, ntasks, one, Part{mw * BM, 0, 1, bnc, false}, xcd, fl);
        if (nw < bnc) launch_part<CT, ROLE>(s, d_tasks, ntasks, one, Part{0, nw * BN, mw, 1, false}, xcd, fl);
        launch_part<CT, ROLE>(s, d_tasks, ntasks, one, Part{0, 0, mw, nw, true}, xcd, fl);
    } else {
        // the strips run beside the whole blocks on the context's side stream
        if (!ctx->side) {
            GPEX_HIP(ctx, hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking));
            GPEX_HIP(ctx, hipEventCreateWithFlags(&ctx->side_fork, hipEventDisableTiming));
            GPEX_HIP(ctx, hipEventCreateWithFlags(&ctx->side_join, hipEventDisableTiming));
        }
        GPEX_HIP(ctx, hipEventRecord(ctx->side_fork, s));
        GPEX_HIP(ctx, hipStreamWaitEvent(ctx->side, ctx->side_fork, 0));
        if (mw < bmc)   // bottom strip, every column
            launch_part<CT, ROLE>(ctx->side, d_tasks, ntasks, one, Part{mw * BM, 0, 1, bnc, false}, xcd, fl);
        if (nw < bnc)   // right strip, the whole block rows
            launch_part<CT, ROLE>(ctx->side, d_tasks, ntasks, one, Part{0, nw * BN, mw, 1, false}, xcd, fl);
        GPEX_HIP(ctx, hipEventRecord(ctx->side_join, ctx->side));
        launch_part<CT, ROLE>(s, d_tasks, ntasks, one, Part{0, 0, mw, nw, true}, xcd, fl);
        GPEX_HIP(ctx, hipStreamWaitEvent(s, ctx->side_join, 0));
    }
    GPEX_HIP(ctx, hipGetLastError());
    return GPEX_OK;
}

// All launches of one compute precision (one translation unit each).
template <typename CT>
static int launch_precision(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks,
                            const GemmTask& one, int role) {
    if (role == GEMM_UPDATE) return launch_ct<CT, GEMM_UPDATE>(ctx, s, d_tasks, ntasks, one);
    if (role == GEMM_TRMM) return launch_ct<CT, GEMM_TRMM>(ctx, s, d_tasks, ntasks, one);
    return launch_ct<CT, GEMM_GENERIC>(ctx, s, d_tasks, ntasks, one);
}

int gemm_launch_f64(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, int role);
int gemm_launch_f32(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, int role);
int gemm_launch_f16(gpex_ctx_t ctx, hipStream_t s, const GemmTask* d_tasks, int ntasks, const GemmTask& one, int role);

}  // namespace gpex

// FP16 simulation product on 256 x 256 blocks with operands loaded straight into LDS.
// C (FP64, column-major) = alpha A B + beta C with A a row-major FP16 factor panel (M x K, lda) and
// B = Z / s in FP16 (column-major K x N, ldb): the GEMM16 tasks of one tile row of L summed as one
// product ("Mixed-Precision GPU Acceleration for Confidence Regions of Spatial Excursion Sets",
// Algorithm 1).  A task may carry the row's diagonal tile too, as 64-wide slab pairs of its two
// FP16 parts (hi, lo) at the end of the panel (GemmTask::kdup), both parts meeting the same rows
// of B, so the whole tile row is one product summed in FP32.  Included by gemm_kernel.h (fragment
// types, matrix-core wrappers, GemmTask).
//
// The general kernel's 128 x 256 blocks move (128 + 256) x 64 operand halves through LDS per
// 2 x 128 x 256 x 64 products; a 256 x 256 block moves (256 + 256) x 64 for twice the products,
// a third less global and LDS-write traffic per product, and its 64 x 128 wave tiles read a
// quarter less from LDS per product than 64 x 64 ones.  The operands skip the registers: 16-byte
// direct loads put them into one of two LDS stages (128 KB), the loads of slab kb + 1 issued at
// the start of slab kb into the stage slab kb - 1 used.  Layout of a stage: A's 256 rows, then
// B's 256 rows (B's rows are the block's columns), 64 k each, unpadded, the 16-byte chunk c of row
// r at position c ^ (r mod 8).  A direct load writes lane l's 16 bytes at the instruction's LDS
// base + 16 l, so one wave instruction fills 8 whole rows: lane l writes row l / 8 at position
// l % 8 and so loads chunk (l % 8) ^ (l / 8) of that row.  Waves: 4 x 2 of 64 x 128 (4 x 8 tiles of
// v_mfma_f32_16x16x32_f16, operands in as (B, A) as in the general kernel).
#pragma once

namespace gpex {

constexpr int P16_BM = 256, P16_BN = 256, P16_BK = 64, P16_THR = 512;
constexpr int P16_STAGE = (P16_BM + P16_BN) * P16_BK;   // halves per stage (64 KB)

// Wait until no vector-memory operation and no LDS access of this wave is outstanding (export
// counter left alone).  s_waitcnt fields: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
__device__ __forceinline__ void p16_wait_all() { __builtin_amdgcn_s_waitcnt((0x7 << 4)); }

// Workgroup barrier without the memory fence of __syncthreads (the fence is the explicit wait
// before it); the empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void p16_barrier() {
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

// Whether the 256 x 256 kernel can run a task: FP16 operands (A row-major, B column-major), FP64
// output, no FP16 destination emulation, whole 256 x 256 blocks, whole 64-k slabs, 16-byte
// aligned rows, diagonal slab pairs (kdup) of whole slabs within K.
inline bool panel16_fits(const GemmTask& g) {
    return g.ta == DT_F16 && g.tb == DT_F16 && g.tc == DT_F64 && g.transA == 1 && g.transB == 0 && g.kround == 0 &&
           g.M % P16_BM == 0 && g.N % P16_BN == 0 && g.K % P16_BK == 0 && g.K >= P16_BK && g.lda % 8 == 0 &&
           g.ldb % 8 == 0 && reinterpret_cast<uintptr_t>(g.A) % 16 == 0 && reinterpret_cast<uintptr_t>(g.B) % 16 == 0 &&
           g.kdup >= 0 && g.kdup % P16_BK == 0 && 2 * (int64_t)g.kdup <= g.K;
}

// (a template so that the several sources including this header share one definition)
template <int UNUSED = 0>
__global__ __launch_bounds__(P16_THR) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_panel16(const GemmTask* __restrict__ tasks, int ntasks, int bmc, int bnc, int xcd_map,
               unsigned long long* flags) {
    __shared__ __attribute__((aligned(16))) _Float16 S[2 * P16_STAGE];
    const int bpt = bmc * bnc;
    const int64_t b = blockIdx.x;
    int task, blk;
    if (xcd_map) {   // every block of a task on one XCD (workgroups are dealt round-robin)
        const int x = (int)(b % 8);
        const int64_t slot = b / 8;
        task = x + 8 * (int)(slot / bpt);
        blk = (int)(slot % bpt);
        if (task >= ntasks) return;
    } else {
        task = (int)(b / bpt);
        blk = (int)(b % bpt);
    }
    GemmTask T;
    {   // the task through the scalar data cache
        const __attribute__((address_space(4))) uint64_t* src =
            (const __attribute__((address_space(4))) uint64_t*)(tasks + task);
        uint64_t wds[sizeof(GemmTask) / 8];
#pragma unroll
        for (int i = 0; i < (int)(sizeof(GemmTask) / 8); ++i) wds[i] = src[i];
        __builtin_memcpy(&T, wds, sizeof(GemmTask));
    }
    if (T.ta != DT_F16 || T.tb != DT_F16 || T.tc != DT_F64 || T.transA != 1 || T.transB != 0 || T.kround != 0 ||
        T.K % P16_BK != 0 || T.K < P16_BK || T.M != bmc * P16_BM || T.N != bnc * P16_BN || T.lda % 8 != 0 ||
        T.ldb % 8 != 0 || reinterpret_cast<uintptr_t>(T.A) % 16 != 0 || reinterpret_cast<uintptr_t>(T.B) % 16 != 0 ||
        T.kdup < 0 || T.kdup % P16_BK != 0 || 2 * (int64_t)T.kdup > T.K) {
        if (threadIdx.x == 0 && flags) atomicOr(&flags[FLAG_BADTASK], 1ull);
        return;
    }
    const int m0 = (blk % bmc) * P16_BM, n0 = (blk / bmc) * P16_BN;
    const int t = threadIdx.x, l = t % 64, w = t / 64, wm = w % 4, wn = w / 4;
    // the diagonal tile's (hi, lo) slab pairs start at k = kd.  (Stopping a block after the last
    // pair that meets its rows, past which the pairs hold zeros, made the launch 1.4% slower.)
    const int kd = T.K - 2 * T.kdup;
    const int nk = T.K / P16_BK;

    // Direct loads of one slab: wave w fills A rows [32 w, 32 w + 32) and B rows [32 w, 32 w + 32),
    // four instructions each; lane l: row offset l / 8, chunk (l % 8) ^ (l / 8).
    const int lrow = l / 8, lchunk = (l % 8) ^ lrow;
    const gptr<_Float16> a_src = (gptr<_Float16>)T.A + (int64_t)(m0 + 32 * w + lrow) * T.lda + 8 * lchunk;
    const gptr<_Float16> b_src = (gptr<_Float16>)T.B + (int64_t)(n0 + 32 * w + lrow) * T.ldb + 8 * lchunk;
    const int64_t a_step8 = 8 * T.lda, b_step8 = 8 * T.ldb;   // 8 rows further
    auto issue = [&](int kb) {
        _Float16* st = S + (kb & 1) * P16_STAGE;
        const int k0 = kb * P16_BK;
        const int kb0 = k0 >= kd ? kd + (((k0 - kd) >> 1) & ~(P16_BK - 1)) : k0;   // B's k of this slab
#pragma unroll
        for (int a = 0; a < 4; ++a)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a_src + a * a_step8 + k0),
                                             (__attribute__((address_space(3))) void*)(st + (32 * w + 8 * a) * P16_BK),
                                             16, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(b_src + q * b_step8 + kb0),
                                             (__attribute__((address_space(3))) void*)(st + (P16_BM + 32 * w + 8 * q) * P16_BK),
                                             16, 0, 0);
    };
    // fragments of step s (k = 32 s + [0, 32)) of a stage: row l % 16 of each 16-row tile, chunk
    // 4 s + l / 16 (8 consecutive k), swizzled
    auto frag = [&](const _Float16* st, int row, int s) {
        const int kc = 4 * s + l / 16;
        return *reinterpret_cast<const h8*>(&st[row * P16_BK + ((kc ^ (row & 7)) << 3)]);
    };
    auto rd_a = [&](const _Float16* st, int s, h8* fa) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = frag(st, wm * 64 + i * 16 + l % 16, s);
    };
    f4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0, 0, 0, 0};
    // products of column tiles [j0, j0 + 4) of one step
    auto products = [&](const h8* fa, const h8* fb, int j0) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) mma(acc[i][j0 + j], fb[j], fa[i]);
    };
    // Fragments in registers: A double buffered across the two steps of a slab; B in two halves
    // (column tiles 0-3 and 4-7), each read one half-step ahead of its products (a whole second B
    // set would not fit the 256 registers of two waves per SIMD).
    h8 fa[2][4], fb0[4], fb1[4];
    auto rd_b = [&](const _Float16* st, int s, int j0, h8* fb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = frag(st, P16_BM + wn * 128 + (j0 + j) * 16 + l % 16, s);
    };

    issue(0);
    p16_wait_all();
    p16_barrier();
    rd_a(S, 0, fa[0]);
    rd_b(S, 0, 0, fb0);
    for (int kb = 0; kb < nk; ++kb) {
        const _Float16* st = S + (kb & 1) * P16_STAGE;
        const bool more = kb + 1 < nk;
        // into the other stage: every wave finished reading it (slab kb - 1) before the last barrier
        if (more) issue(kb + 1);
        // step 0
        rd_b(st, 0, 4, fb1);
        rd_a(st, 1, fa[1]);
        products(fa[0], fb0, 0);
        rd_b(st, 1, 0, fb0);
        products(fa[0], fb1, 4);
        // step 1
        rd_b(st, 1, 4, fb1);
        products(fa[1], fb0, 0);
        if (more) {
            // this wave's part of slab kb + 1 has landed and its reads of slab kb are done; after
            // the barrier every wave's part is there and the stage of slab kb may be refilled
            p16_wait_all();
            p16_barrier();
            const _Float16* nx = S + ((kb + 1) & 1) * P16_STAGE;
            rd_a(nx, 0, fa[0]);
            rd_b(nx, 0, 0, fb0);
        }
        products(fa[1], fb1, 4);
    }

    // Epilogue: fragment (i, j) holds the transposed 16 x 16 block (lane l: row l % 16, register
    // r: column 4 (l / 16) + r); only the caller's rows and columns (m_store, n_store) are stored.
    // Old C outside them is read at a clamped position, so the loads of a row group are
    // unconditional and issue together; all values are formed before the guarded stores.
    const int m_st = T.m_store ? T.m_store : T.M, n_st = T.n_store ? T.n_store : T.N;
    const gptr_mut<double> Cp = (gptr_mut<double>)T.C;
    const bool use_beta = T.beta != 0.0;
    const bool full = m0 + P16_BM <= m_st && n0 + P16_BN <= n_st;   // the block lies inside the stored part
    // (in groups of one row tile and four column tiles: 16 old values, 16 results)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + wm * 64 + i * 16 + l % 16;
#pragma unroll
        for (int jh = 0; jh < 2; ++jh) {
            double v[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[j][r] = T.alpha * (double)acc[i][4 * jh + j][r];
            if (use_beta) {
                double cold[4][4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int col = n0 + wn * 128 + (4 * jh + j) * 16 + 4 * (l / 16) + r;
                        cold[j][r] = Cp[(int64_t)min(row, m_st - 1) + (int64_t)min(col, n_st - 1) * T.ldc];
                    }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[j][r] += T.beta * cold[j][r];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int col = n0 + wn * 128 + (4 * jh + j) * 16 + 4 * (l / 16) + r;
                    if (full || (row < m_st && col < n_st)) Cp[(int64_t)row + (int64_t)col * T.ldc] = v[j][r];
                }
        }
    }
}

}  // namespace gpex

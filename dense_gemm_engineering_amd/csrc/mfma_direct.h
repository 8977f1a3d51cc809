// Direct-to-LDS macro-tile GEMM for fp16/bf16 on gfx950 (full tiles).
//
// Same decomposition as gemm_mfma_kernel (BM x BN workgroup tile, WM x WN
// waves, 16x16x32 MFMA blocks, 128-byte K stages, two LDS buffers), with the
// operand traffic moved off the vector registers:
//
//  * Global -> LDS with global_load_lds_dwordx4: each instruction moves 16
//    bytes per lane straight into LDS at (wave-uniform base + 16 * lane), so
//    no staging registers and no ds_write.  The LDS layout is chosen by which
//    global chunk each lane fetches: for a K-contiguous operand, lane L of an
//    instruction fills row (L / 8) of an 8-row, 1 KB block at physical
//    chunk L % 8 and fetches logical chunk (L % 8) ^ (row & 7), which is the
//    XOR swizzle the fragment reads expect.  This is gfx950's counterpart of
//    the bulk-copy engines of "Optimizing GEMMs using tcgen05 - Part 2" §5.1
//    and of cp.async in "02 · 8m/8m② — Tiled wmma f16 prefill GEMM" §2.4:
//    the copy runs while the MFMAs of the previous stage execute.
//  * A K x N row-major B (the headline layout) is stored in LDS as it sits in
//    memory, n-contiguous, and its MFMA fragments are read with
//    ds_read_b64_tr_b16: within each 16-lane group, lane t points at 4
//    consecutive n of k-row (kbase + t / 4); lane i then receives the 4
//    values of column i for k = kbase .. kbase + 3.  Two such reads give the
//    8 consecutive k one MFMA operand register quad holds.  The 16-byte
//    chunks of k-row k are XOR-swizzled by 2 (k & 3) + 8 ((k >> 3) & 1) so
//    the four k-rows a group reads fall in different 32-byte bank groups.
//  * Software pipeline, one barrier per stage: the fragment reads of the
//    next k-block are interleaved with the MFMAs of the current one (the LDS
//    counter can track 15 outstanding reads, so they are issued a few at a
//    time between MFMAs); the barrier sits before the last quarter of a
//    stage's MFMAs, and right after it each wave issues the direct loads two
//    stages ahead and the first reads of the next stage, so the MFMA pipe
//    keeps busy across the barrier.
#pragma once

#include "mfma_gemm.h"

namespace dge {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define DGE_LDS __attribute__((address_space(3)))

__device__ inline int swz_b(int k) { return ((k & 3) << 1) | (((k >> 3) & 1) << 3); }

// One global_load_lds_dwordx4: 16 bytes per lane from g to LDS address
// (l + 16 * lane).  Issued as inline assembly on purpose: the compiler then
// does not count it in its memory-wait bookkeeping, and every wait for these
// loads is explicit in the kernel (s_waitcnt vmcnt before the barrier that
// publishes a stage).  Left to the compiler, each later transposed LDS read
// (whose intrinsic carries no address information) would be preceded by a
// wait for ALL outstanding loads, serialising every stage with its loads.
// M0 (the LDS base of the copy) is set inside the same statement; these
// kernels have no other M0 user, so the clobber of that reserved register is
// safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void lds_dma16(const void* g, DGE_LDS void* l) {
    const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline uint2 ds_read_tr(const DGE_LDS char* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DGE_LDS s16x4*)p);
    return __builtin_bit_cast(uint2, v);
}

template <int DT, int BM, int BN, int WM, int WN, bool TRANS_B>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_direct_kernel(MfmaArgs p) {
    static_assert(DT == IN_F16 || DT == IN_BF16, "16-bit inputs only");
    constexpr int NW = WM * WN;
    constexpr int BK = 64;
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;  // one stage
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int IA = A_BYTES / 1024 / NW;  // direct-load instructions per wave per stage
    constexpr int IB = B_BYTES / 1024 / NW;
    static_assert(IA * 1024 * NW == A_BYTES && IB * 1024 * NW == B_BYTES, "stage split");
    static_assert(TRANS_B || BN >= 128, "transposed-read layout needs 16+ chunks per k-row");
    constexpr int CPR_B = BN / 8;             // 16-byte chunks per k-row of a K x N B tile
    constexpr int RPI_B = 1024 / (BN * 2);    // k-rows per 1 KB direct-load instruction
    static_assert(TRANS_B || RPI_B * BN * 2 == 1024, "whole k-rows per instruction");

    __shared__ __attribute__((aligned(1024))) char lds[2][A_BYTES + B_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

    const int ntiles = p.tiles_m * p.tiles_n;
    const int lin = remap_xcd(blockIdx.x, ntiles * p.splits);
    const int split = lin / ntiles;
    int tm, tn;
    grouped_tile(lin % ntiles, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.k_per_split;
    const int kend = min(kbeg + p.k_per_split, p.K);
    const int nk = (kend - kbeg) / BK;

    // ---- per-lane global source offsets (elements) for the direct loads
    // A: instruction i of this wave fills rows 8 * (wave * IA + i) + lane / 8.
    const int a_row = 8 * wave * IA + (lane >> 3);
    const int a_chunk = (lane & 7) ^ ((lane >> 3) & 7);
    const uint16_t* a_src = (const uint16_t*)p.A + (int64_t)(m0 + a_row) * p.lda + a_chunk * 8 + kbeg;
    const int64_t a_step = (int64_t)8 * p.lda;  // next instruction: 8 rows down
    const uint16_t* b_src;
    int64_t b_step;
    if constexpr (TRANS_B) {
        const int b_row = 8 * wave * IB + (lane >> 3);
        b_src = (const uint16_t*)p.B + (int64_t)(n0 + b_row) * p.ldb + a_chunk * 8 + kbeg;
        b_step = (int64_t)8 * p.ldb;
    } else {
        // instruction i fills k-rows RPI * (wave * IB + i) + lane / CPR; the
        // chunk swizzle depends on the k-row, so it is applied per instruction
        const int krow = RPI_B * wave * IB + lane / CPR_B;
        b_src = (const uint16_t*)p.B + (int64_t)(kbeg + krow) * p.ldb + n0;
        b_step = (int64_t)RPI_B * p.ldb;
    }
    const int b_lane_chunk = lane % CPR_B;
    const int b_krow0 = RPI_B * wave * IB + lane / CPR_B;
    const int64_t a_kstep = BK;                                        // A per stage
    const int64_t b_kstep = TRANS_B ? (int64_t)BK : (int64_t)BK * p.ldb;  // B per stage

    auto issue_loads = [&](int st, int kt) {
        DGE_LDS char* la = (DGE_LDS char*)&lds[st][0] + wave * IA * 1024;
        DGE_LDS char* lb = (DGE_LDS char*)&lds[st][A_BYTES] + wave * IB * 1024;
        const uint16_t* ga = a_src + kt * a_kstep;
        const uint16_t* gb = b_src + kt * b_kstep;
#pragma unroll
        for (int i = 0; i < IA; ++i) lds_dma16(ga + i * a_step, la + i * 1024);
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            if constexpr (TRANS_B) {
                lds_dma16(gb + i * b_step, lb + i * 1024);
            } else {
                const int chunk = b_lane_chunk ^ swz_b(b_krow0 + RPI_B * i);
                lds_dma16(gb + i * b_step + chunk * 8, lb + i * 1024);
            }
        }
    };

    // ---- fragment reads
    // A (and K-contiguous B): row r = base + (lane & 15), chunk (kb*4 + lane/16) ^ (r & 7).
    auto read_rows = [&](const DGE_LDS char* base, int row0, int kb, int ntile, u32x4* f) {
        const int r = row0 + (lane & 15);
        const DGE_LDS char* q = base + r * 128 + (((kb * 4 + (lane >> 4)) ^ (r & 7)) << 4);
#pragma unroll
        for (int i = 0; i < ntile; ++i) f[i] = *(const DGE_LDS u32x4*)(q + i * 16 * 128);
    };
    // K x N B via transposed reads: k = kb*32 + 8*(lane/16) + 4h + (t/4), n = wn0 + 16j + 4(t%4).
    auto read_bt = [&](const DGE_LDS char* base, int kb, u32x4* f) {
        const int t = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kb * 32 + 8 * (lane >> 4) + 4 * h + (t >> 2);
            const int nloc = wn0 + 4 * (t & 3);  // + 16 j
            const DGE_LDS char* rowp = base + k * (BN * 2);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = nloc + 16 * j;
                const int c = (n >> 3) ^ swz_b(k);
                const uint2 v = ds_read_tr(rowp + (c << 4) + ((n & 7) << 1));
                f[j][2 * h] = v.x;
                f[j][2 * h + 1] = v.y;
            }
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    auto read_kblock = [&](int st, int kb, u32x4* fa, u32x4* fb) {
        const DGE_LDS char* la = (const DGE_LDS char*)&lds[st][0];
        const DGE_LDS char* lb = (const DGE_LDS char*)&lds[st][A_BYTES];
        read_rows(la, wm0, kb, TM, fa);
        if constexpr (TRANS_B)
            read_rows(lb, wn0, kb, TN, fb);
        else
            read_bt(lb, kb, fb);
    };
    // MFMAs [lo, hi) of one k-block, row-major over the TM x TN blocks.
    auto mma_range = [&](const u32x4* fa, const u32x4* fb, int lo, int hi) {
#pragma unroll
        for (int x = 0; x < TM * TN; ++x)
            if (x >= lo && x < hi) mma_chunk<DT>(acc[x / TN][x % TN], fa[x / TN], fb[x % TN]);
    };

    // Instruction counts of one stage, for the interleaving below.
    constexpr int NMF = TM * TN;                         // MFMAs per k-block
    constexpr int NRD = TM + (TRANS_B ? TN : 2 * TN);    // LDS fragment reads per k-block
    constexpr int NDMA = IA + IB;                        // direct loads per stage
    constexpr int TAIL = NMF / 4;                        // k-block-1 MFMAs after the barrier
    constexpr int Q1 = NMF / NRD > 0 ? NMF / NRD : 1;    // MFMAs per read in phase 1

    // Prologue: stages 0 and 1 in flight, wait for stage 0, read its k-block 0.
    issue_loads(0, 0);
    issue_loads(1, nk > 1 ? 1 : 0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((NDMA & 15) | ((NDMA >> 4) << 14)));  // vmcnt(NDMA)
    __syncthreads();
    read_kblock(0, 0, fa0, fb0);

    // Steady state, stage kt (buffer kt & 1):
    //   phase 1: MFMAs of k-block 0, with the reads of k-block 1 interleaved;
    //   phase 2: the first 3/4 of k-block 1's MFMAs;
    //   barrier: stage kt + 1 has landed and nobody reads buffer kt & 1 any more;
    //   phase 3: direct loads of stage kt + 2 into buffer kt & 1 and the reads
    //            of stage kt + 1's k-block 0, interleaved with the last MFMAs.
    // Past the last stage the loads re-fetch the last stage (never read) so
    // the body has no branch and the scheduling groups cover all of it.
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        read_kblock(st, 1, fa1, fb1);
        mma_range(fa0, fb0, 0, NMF);
#pragma unroll
        for (int r = 0; r < NRD; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, Q1, 0); // Q1 MFMAs
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
        mma_range(fa1, fb1, 0, NMF - TAIL);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - TAIL, 0);

        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of stage kt + 1
        __syncthreads();

        issue_loads(st, min(kt + 2, nk - 1));
        read_kblock(st ^ 1, 0, fa0, fb0);
        mma_range(fa1, fb1, NMF - TAIL, NMF);
#pragma unroll
        for (int r = 0; r < TAIL; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x020, (NDMA + TAIL - 1) / TAIL, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, (NRD + TAIL - 1) / TAIL, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    epilogue_tile<DT, BM, BN, WM, WN, LOAD_FAST>(p, acc, (float*)&lds[0][0], m0, n0, split);
}

}  // namespace dge


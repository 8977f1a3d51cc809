// Direct-to-LDS macro-tile GEMM for fp16/bf16 on gfx950 (full tiles).
//
// BM x BN workgroup tile, WM x WN waves, 128-byte K stages in two LDS
// buffers, accumulators in MS x MS MFMA blocks.
//
//  * Block size per wave count: one wave issuing independent 32x32x16 MFMAs
//    back to back keeps its SIMD's matrix unit ~98% busy on gfx950, one
//    wave of 16x16x32 MFMAs only ~60% (two waves per SIMD ~91%).  So the
//    4-wave tiles (one wave per SIMD) use 32x32x16 blocks (MS = 32); the
//    8-wave 256 x 256 tile, with two waves per SIMD, measured faster with
//    16x16x32 blocks (MS = 16: 119 vs 124 us at 4096^3, K x N B).
//    Operand layouts: lane l supplies row (l % MS) of A and column (l % MS)
//    of B, each with 8 consecutive k (chunk l / MS of the k-block, which is
//    32 deep for MS = 16 and 16 deep for MS = 32).  A 16x16 block gives lane
//    l rows 4 (l / 16) + e, e = 0..3, of column l % 16; a 32x32 block gives
//    it rows 8 (r / 4) + 4 (l / 32) + r % 4, r = 0..15, of column l % 32.
//  * Global -> LDS with global_load_lds_dwordx4: each instruction moves 16
//    bytes per lane straight into LDS at (wave-uniform base + 16 * lane), so
//    no staging registers and no ds_write.  The LDS layout is chosen by which
//    global chunk each lane fetches: for a K-contiguous operand, lane L of an
//    instruction fills row (L / 8) of an 8-row, 1 KB block at physical
//    chunk L % 8 and fetches logical chunk (L % 8) ^ swz_k(row), which is
//    the XOR swizzle the fragment reads expect.  For 32-row operand reads
//    swz_k(row) = (row & 7) ^ ((row >> 4) & 1), which spreads the 32 rows
//    over all banks (with (row & 7) alone, rows r and r + 16 collide and a
//    read takes ~1.8x as long, measured); 16-row reads use (row & 7).  This is gfx950's counterpart of
//    the bulk-copy engines of "Optimizing GEMMs using tcgen05 - Part 2" §5.1
//    and of cp.async in "02 · 8m/8m② — Tiled wmma f16 prefill GEMM" §2.4:
//    the copy runs while the MFMAs of the previous stage execute.
//  * A K x N row-major B (the headline layout) is stored in LDS as it sits in
//    memory, n-contiguous, and its MFMA fragments are read with
//    ds_read_b64_tr_b16: within each 16-lane group, lane t points at 4
//    consecutive n of k-row (kbase + t / 4); lane i then receives the 4
//    values of column i for k = kbase .. kbase + 3.  Two such reads give the
//    8 consecutive k one operand register quad holds.  The 16-byte chunks of
//    k-row k are XOR-swizzled (swz_b<MS>) so that the k-rows and columns
//    the lane groups of one read cover fall in different bank groups.
//  * Software pipeline, one barrier per stage: the fragment reads of the
//    next k-block are interleaved with the MFMAs of the current one (the LDS
//    counter can track 15 outstanding reads, so they are issued a few at a
//    time between MFMAs); the barrier sits before the last MFMAs of a stage,
//    and right after it each wave issues the first part of the direct loads
//    two stages ahead and the first reads of the next stage, so the MFMA
//    pipe keeps busy across the barrier; the rest of those loads go out
//    between the MFMAs of the following k-blocks.
#pragma once

#include "mfma_gemm.h"

namespace dge {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define DGE_LDS __attribute__((address_space(3)))

template <int MS>
__device__ inline int swz_b(int k) {
    if constexpr (MS == 32) return (k & 3) << 2;
    return ((k & 3) << 1) | (((k >> 3) & 1) << 3);
}
// (bit 4 of the row only matters for 32-row reads; 16-row reads step across
// it between blocks, so they keep the plain (row & 7))
template <int MS>
__device__ inline int swz_k(int row) {
    if constexpr (MS == 32) return (row & 7) ^ ((row >> 4) & 1);
    return row & 7;
}

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

// Scheduling pattern for one k-block: its NMF MFMAs spread evenly between
// the NRD fragment reads of the next k-block (one read, then its share of
// MFMAs), so that every group matches instructions of this k-block only.
template <int NRD, int NMF, int R = 0>
__device__ inline void interleave_reads() {
    if constexpr (R < NRD) {
        constexpr int m = (R + 1) * NMF / NRD - R * NMF / NRD;
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);  // m MFMAs
        interleave_reads<NRD, NMF, R + 1>();
    }
}

template <int DT>
__device__ inline void mma32(f32x16& acc, const u32x4& a, const u32x4& b) {
    if constexpr (DT == IN_F16)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    else
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <int MS> struct AccBlock;
template <> struct AccBlock<16> { typedef f32x4 T; };
template <> struct AccBlock<32> { typedef f32x16 T; };

template <int DT, int BM, int BN, int WM, int WN, bool TRANS_B, int MS>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_direct_kernel(MfmaArgs p) {
    static_assert(DT == IN_F16 || DT == IN_BF16, "16-bit inputs only");
    static_assert(MS == 16 || MS == 32, "MFMA block size");
    constexpr int NW = WM * WN;
    constexpr int BK = 64;
    constexpr int KBLK = 512 / MS;   // k per k-block: 32 (16x16x32) or 16 (32x32x16)
    constexpr int KB = BK / KBLK;    // k-blocks per stage
    constexpr int CPK = KBLK / 8;    // 16-byte chunks per row per k-block
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;  // one stage
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / MS, TN = WTN / MS;
    static_assert(TM * MS == WTM && TN * MS == WTN, "wave tile must be a multiple of the block");
    constexpr int IA = A_BYTES / 1024 / NW;  // direct-load instructions per wave per stage
    constexpr int IB = B_BYTES / 1024 / NW;
    static_assert(IA * 1024 * NW == A_BYTES && IB * 1024 * NW == B_BYTES, "stage split");
    static_assert(TRANS_B || BN >= 128, "transposed-read layout needs 16+ chunks per k-row");
    constexpr int CPR_B = BN / 8;             // 16-byte chunks per k-row of a K x N B tile
    constexpr int RPI_B = 1024 / (BN * 2);    // k-rows per 1 KB direct-load instruction
    static_assert(TRANS_B || RPI_B * BN * 2 == 1024, "whole k-rows per instruction");
    static_assert(NW * MS * (WTN + 8) * 4 <= 2 * (A_BYTES + B_BYTES), "epilogue staging fits");

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
    // A: instruction i of this wave fills rows 8 * (wave * IA + i) + lane / 8;
    // its chunk swizzle depends on the row block, so it is applied per instruction
    const int a_row = 8 * wave * IA + (lane >> 3);
    const int k_lane_chunk = lane & 7;
    const uint16_t* a_src = (const uint16_t*)p.A + (int64_t)(m0 + a_row) * p.lda + kbeg;
    const int64_t a_step = (int64_t)8 * p.lda;  // next instruction: 8 rows down
    const uint16_t* b_src;
    int64_t b_step;
    if constexpr (TRANS_B) {
        const int b_row = 8 * wave * IB + (lane >> 3);
        b_src = (const uint16_t*)p.B + (int64_t)(n0 + b_row) * p.ldb + kbeg;
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

    // Direct loads [lo, hi) of the IA + IB of stage kt, into buffer st.
    auto issue_part = [&](int st, int kt, int lo, int hi) {
        DGE_LDS char* la = (DGE_LDS char*)&lds[st][0] + wave * IA * 1024;
        DGE_LDS char* lb = (DGE_LDS char*)&lds[st][A_BYTES] + wave * IB * 1024;
        const uint16_t* ga = a_src + kt * a_kstep;
        const uint16_t* gb = b_src + kt * b_kstep;
#pragma unroll
        for (int i = 0; i < IA; ++i) {
            if (i < lo || i >= hi) continue;
            const int chunk = k_lane_chunk ^ swz_k<MS>(a_row + 8 * i);
            lds_dma16(ga + i * a_step + chunk * 8, la + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            if (IA + i < lo || IA + i >= hi) continue;
            if constexpr (TRANS_B) {
                const int chunk = k_lane_chunk ^ swz_k<MS>(8 * wave * IB + (lane >> 3) + 8 * i);
                lds_dma16(gb + i * b_step + chunk * 8, lb + i * 1024);
            } else {
                const int chunk = b_lane_chunk ^ swz_b<MS>(b_krow0 + RPI_B * i);
                lds_dma16(gb + i * b_step + chunk * 8, lb + i * 1024);
            }
        }
    };

    // ---- fragment reads of k-block kb
    // A (and K-contiguous B): row r = base + (lane % MS), chunk
    // (CPK kb + lane / MS) ^ swz_k(r) (the same swizzle for every block of rows).
    auto read_rows = [&](const DGE_LDS char* base, int row0, int kb, int ntile, u32x4* f) {
        const int r = row0 + (lane % MS);
        const DGE_LDS char* q = base + r * 128 + (((kb * CPK + lane / MS) ^ swz_k<MS>(r)) << 4);
#pragma unroll
        for (int i = 0; i < ntile; ++i) f[i] = *(const DGE_LDS u32x4*)(q + i * MS * 128);
    };
    // K x N B via transposed reads.  Lane group g = lane / 16 covers k-rows
    // kb KBLK + 8 (g / (MS / 16)) + 4 h + (t / 4) and columns
    // wn0 + MS j + 16 (g % (MS / 16)) + 4 (t % 4).
    auto read_bt = [&](const DGE_LDS char* base, int kb, u32x4* f) {
        const int t = lane & 15, g = lane >> 4;
        const int kofs = MS == 16 ? 8 * g : 8 * (g >> 1);
        const int nofs = MS == 16 ? 0 : 16 * (g & 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kb * KBLK + kofs + 4 * h + (t >> 2);
            const int nloc = wn0 + nofs + 4 * (t & 3);  // + MS j
            const DGE_LDS char* rowp = base + k * (BN * 2);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = nloc + MS * j;
                const int c = (n >> 3) ^ swz_b<MS>(k);
                const uint2 v = ds_read_tr(rowp + (c << 4) + ((n & 7) << 1));
                f[j][2 * h] = v.x;
                f[j][2 * h + 1] = v.y;
            }
        }
    };

    typedef typename AccBlock<MS>::T Acc;
    constexpr int NACC = MS * MS / 64;  // accumulator elements per lane per block
    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.f;

    u32x4 fa[2][TM], fb[2][TN];
    auto read_kblock = [&](int st, int kb, u32x4* a, u32x4* b) {
        const DGE_LDS char* la = (const DGE_LDS char*)&lds[st][0];
        const DGE_LDS char* lb = (const DGE_LDS char*)&lds[st][A_BYTES];
        read_rows(la, wm0, kb, TM, a);
        if constexpr (TRANS_B)
            read_rows(lb, wn0, kb, TN, b);
        else
            read_bt(lb, kb, b);
    };
    // MFMAs [lo, hi) of one k-block, row-major over the TM x TN blocks.
    auto mma_range = [&](const u32x4* a, const u32x4* b, int lo, int hi) {
#pragma unroll
        for (int x = 0; x < TM * TN; ++x)
            if (x >= lo && x < hi) {
                if constexpr (MS == 32)
                    mma32<DT>(acc[x / TN][x % TN], a[x / TN], b[x % TN]);
                else
                    mma_chunk<DT>(acc[x / TN][x % TN], a[x / TN], b[x % TN]);
            }
    };

    // Instruction counts of one k-block, for the interleaving below.
    constexpr int NMF = TM * TN;                         // MFMAs per k-block
    constexpr int NRD = TM + (TRANS_B ? TN : 2 * TN);    // LDS fragment reads per k-block
    constexpr int NDMA = IA + IB;                        // direct loads per stage
    // A stage's direct loads go out in DPART parts: the first right after the
    // barrier that frees its buffer, the others between the MFMAs of the next
    // k-blocks.  Issued as one burst they stall the wave's MFMA issue while
    // the address unit works through them (measured: ~2960 -> ~2680 cycles
    // per stage for the 8-wave tile).
    constexpr int DPART = KB - 1 < 3 ? KB - 1 : 3;  // 1 (all after the barrier) for MS = 16
    constexpr int NP0 = NDMA / DPART;                    // loads in the first part
    constexpr int TAIL = NMF / (MS == 16 ? 4 : 2) > 0 ? NMF / (MS == 16 ? 4 : 2) : 1;  // after the barrier

    // Prologue: stages 0 and 1 in flight, wait for stage 0, read its k-block 0.
    issue_part(0, 0, 0, NDMA);
    issue_part(1, nk > 1 ? 1 : 0, 0, NP0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((NP0 & 15) | ((NP0 >> 4) << 14)));  // vmcnt(NP0)
    __syncthreads();
    read_kblock(0, 0, fa[0], fb[0]);

    // Steady state, stage kt (buffer kt & 1), k-blocks 0 .. KB-1 with their
    // fragments alternating between two register sets:
    //   k-blocks 0 .. KB-2: MFMAs, with the reads of the next k-block interleaved;
    //   k-block KB-1: the first MFMAs, then the barrier (stage kt + 1 has landed
    //   and nobody reads buffer kt & 1 any more), then the direct loads of
    //   stage kt + 2 into buffer kt & 1 and the reads of stage kt + 1's
    //   k-block 0, interleaved with the last TAIL MFMAs.
    // Past the last stage the loads re-fetch the last stage (never read) so
    // the body has no branch and the scheduling groups cover all of it.
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
#pragma unroll
        for (int kb = 0; kb < KB - 1; ++kb) {
            read_kblock(st, kb + 1, fa[(kb + 1) & 1], fb[(kb + 1) & 1]);
            mma_range(fa[kb & 1], fb[kb & 1], 0, NMF);
            // the remaining parts of stage kt + 1's loads (its buffer was freed
            // by the barrier that ended the previous stage)
            if (kb + 1 < DPART)
                issue_part(st ^ 1, min(kt + 1, nk - 1), (kb + 1) * NDMA / DPART,
                           (kb + 2) * NDMA / DPART);
            interleave_reads<NRD, NMF>();
        }
        constexpr int L = (KB - 1) & 1;
        mma_range(fa[L], fb[L], 0, NMF - TAIL);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - TAIL, 0);
        // nothing moves across the barrier (the MFMAs above would otherwise
        // drift past it, leaving the matrix unit idle while the wave waits)
        __builtin_amdgcn_sched_barrier(0);

        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of stage kt + 1
        __syncthreads();

        issue_part(st, min(kt + 2, nk - 1), 0, NP0);
        read_kblock(st ^ 1, 0, fa[0], fb[0]);
        mma_range(fa[L], fb[L], NMF - TAIL, NMF);
#pragma unroll
        for (int r = 0; r < TAIL; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x020, (NDMA + TAIL - 1) / TAIL, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, (NRD + TAIL - 1) / TAIL, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if constexpr (MS == 32)
        epilogue_tile32<DT, BM, BN, WM, WN, LOAD_FAST>(p, acc, (float*)&lds[0][0], m0, n0, split);
    else
        epilogue_tile<DT, BM, BN, WM, WN, LOAD_FAST>(p, acc, (float*)&lds[0][0], m0, n0, split);
}

}  // namespace dge

// Direct-to-LDS macro-tile GEMM for fp16/bf16 on gfx950 (full tiles).
//
// BM x BN workgroup tile, WM x WN waves, 128-byte K stages in two LDS
// buffers (three for the 8-wave 256 x 128 tile), accumulators in MS x MS
// MFMA blocks.
//
//  * Block size per wave count: one wave issuing independent 32x32x16 MFMAs
//    back to back keeps its SIMD's matrix unit ~98% busy on gfx950, one
//    wave of 16x16x32 MFMAs only ~60% (two waves per SIMD ~91%).  So the
//    4-wave tiles (one wave per SIMD) use 32x32x16 blocks (MS = 32); the
//    8-wave tiles (256 x 256 as 2 x 4 waves, 256 x 128 as 4 x 2), with two
//    waves per SIMD, measured faster with 16x16x32 blocks (MS = 16: 119 vs
//    124 us at 4096^3, K x N B; 2048 x 4096 x 4096 with 256 x 128 tiles
//    64.6 us against 70.4 for the 4-wave 32x32x16 tile).
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
//  * Fused q4 weights (Q4 = true, N x K weights as 18-byte blocks: a binary16
//    scale d, then 16 code bytes, byte i holding element i in its low nibble
//    and element i + 16 in its high nibble, value d (q - 8); "02 · 8m/8m② —
//    Tiled wmma f16 prefill GEMM" §3.2): the B tile is not copied but made.
//    After the barrier that frees a buffer, each thread loads the 20
//    4-byte-aligned bytes holding one 32-weight block of the stage two ahead
//    into registers; before the next barrier it decodes them and writes four
//    16-byte rows chunks into the swizzled k-contiguous B layout.  Decoding
//    uses packed binary16 arithmetic: (0x6400 | q) is 1024 + q exactly,
//    minus 1032 gives q - 8 exactly, and one packed multiply by d rounds
//    d (q - 8) once to nearest-even, the value the two-pass path stores.
//    The fp16 weight matrix is never written (the dequant pass and its
//    re-read, 90 of the 115.5 MB a 11008 x 4096 projection moves, go away).
//  * Software pipeline, one barrier per stage: the fragment reads of the
//    next k-block are interleaved with the MFMAs of the current one (the LDS
//    counter can track 15 outstanding reads, so they are issued a few at a
//    time between MFMAs); the barrier sits before the last MFMAs of a stage,
//    and right after it each wave issues the first part of the direct loads
//    two stages ahead and the first reads of the next stage, one load and
//    its share of the reads per remaining MFMA (not as a burst: 4096^3 NN
//    109.8 -> 109.1 us, NT 108.7 -> 107.6 us), so the MFMA pipe keeps busy
//    across the barrier; the rest of those loads go out between the MFMAs of
//    the following k-blocks.
#pragma once

#include "mfma_gemm.h"

namespace dge {

// Diagnostic build (-DGEMM_DIAG_EXTRA_BARRIERS, libdge_gemm_diag.so): after
// every group of direct loads, fragment reads, q4 decode writes and epilogue
// staging writes, each wave waits for all its memory operations and meets
// every other wave at a barrier.  Nothing then overlaps, so a missing wait
// or barrier in the pipelined kernel (one wave's loads overwriting a buffer
// another still reads) shows up as a difference between the two builds'
// bit-exact results.  Every place it is used is reached by all waves of the
// workgroup the same number of times.
#if defined(GEMM_DIAG_EXTRA_BARRIERS)
#define DGE_DIAG_SYNC()                     \
    do {                                    \
        __builtin_amdgcn_s_waitcnt(0);      \
        __syncthreads();                    \
    } while (0)
#else
#define DGE_DIAG_SYNC() \
    do {                \
    } while (0)
#endif

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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
// The same with the address split into a wave-uniform 64-bit base (scalar
// registers) and a 32-bit per-lane byte offset: a stage's advance is then
// scalar arithmetic on the base, and the per-lane offsets stay constant.
__device__ inline void lds_dma16_s(const void* sbase, uint32_t voff, DGE_LDS void* l) {
    const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(la)
                 : "memory", "m0");
}
// One global_load_lds_dword: 4 bytes per lane from sbase + voff to LDS
// address (l + 4 * lane), with the same wait discipline as lds_dma16.
__device__ inline void lds_dma4_s(const void* sbase, uint32_t voff, DGE_LDS void* l) {
    const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(la)
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

// Scheduling pattern of a stage's last NM MFMAs after the barrier: each MFMA
// followed by its share of the NRD fragment reads of the next k-block.
template <int NM, int NRD, int R = 0>
__device__ inline void tail_reads() {
    if constexpr (R < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        constexpr int n = (R + 1) * NRD / NM - R * NRD / NM;
        if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);  // n LDS reads
        tail_reads<NM, NRD, R + 1>();
    }
}

// Scheduling pattern for NM MFMAs interleaved with VALU work: after each
// MFMA up to V VALU instructions, and NW LDS writes spread evenly.
template <int NM, int V, int NW, int R = 0>
__device__ inline void interleave_valu() {
    if constexpr (R < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // V VALU
        constexpr int w = (R + 1) * NW / NM - R * NW / NM;
        if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);  // LDS writes
        interleave_valu<NM, V, NW, R + 1>();
    }
}

// Scheduling pattern of a fused q4 stage's first k-block: each of its NM
// MFMAs followed by its share of NRD LDS reads (fragments of the next
// k-block and raw q4 blocks), NV VALU instructions (the decode) and NW LDS
// writes (the decoded B tile).
template <int NM, int NRD, int NV, int NW, int R = 0>
__device__ inline void interleave_q4() {
    if constexpr (R < NM) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        constexpr int r = (R + 1) * NRD / NM - R * NRD / NM;
        if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
        constexpr int v = (R + 1) * NV / NM - R * NV / NM;
        if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x002, v, 0);
        constexpr int w = (R + 1) * NW / NM - R * NW / NM;
        if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);
        interleave_q4<NM, NRD, NV, NW, R + 1>();
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

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Eight q4 codes (nib: the low or high nibbles of 4 code bytes, one per
// byte) as eight binary16 weights d * (q - 8), packed in pairs: v_perm_b32
// puts byte 0x64 above each code, giving 1024 + q exactly, minus 1032 is
// q - 8 exactly, and one packed multiply by d rounds once.
__device__ inline void q4_decode4(uint32_t nib, h2v d2, uint32_t* o) {
    const h2v off = {(_Float16)1032.0f, (_Float16)1032.0f};
    // selector bytes: 0-3 pick bytes of nib, 4-7 bytes of 0x64646464
    const uint32_t v01 = __builtin_amdgcn_perm(0x64646464u, nib, 0x04010400u);  // q0, q1
    const uint32_t v23 = __builtin_amdgcn_perm(0x64646464u, nib, 0x04030402u);  // q2, q3
    o[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(h2v, v01) - off) * d2);
    o[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(h2v, v23) - off) * d2);
}

// Epilogue of a tile held as transposed MS x MS blocks (the MFMA operands
// swapped, so each block is C^T): lane l holds, of block (i, j), row
// MS i + (l % MS) and NG groups of 4 consecutive columns, group g at column
// MS j + CG g + 4 (l / MS) (MS = 16: one group, CG unused; MS = 32: four
// groups, CG = 8), accumulator elements 4 g .. 4 g + 3.  alpha, beta (4
// consecutive old values), bias, GELU and the rounding run in registers;
// the results go through the wave's own part of LDS (IP row blocks at a
// time, 16-byte chunks XOR-swizzled by row) and leave as 16-byte pieces of
// whole rows of the wave tile: no workgroup barrier.  (fp32 results stored
// straight from registers left as 64-byte row pieces, and drained slower.)
// Split-K partials leave straight from registers, 16 bytes per lane.  Full
// tiles, 16-byte aligned rows.  The final C stores are non-temporal (streamed towards memory rather
// than left dirty in L2 for the end-of-kernel write-back: 4096^3 NN 113.1 ->
// 111.5 us, NT 113.0 -> 108.7 us, 4096 x 4096 x 256 21.5 -> 19.6 us);
// split-K partials, which the fixup reads back, are ordinary stores.
template <int MS> struct TLayout;
template <> struct TLayout<16> { static constexpr int NG = 1, CG = 0; };
template <> struct TLayout<32> { static constexpr int NG = 4, CG = 8; };

// Epilogue modes, fixed per instance so that no work of an unused option is
// done: the flags are uniform, but left to the compiler the per-element
// branches become selects, and every element then pays for the GELU, the
// beta term and the bias whether asked for or not (and with a run-time beta
// each group's old values are waited for one load at a time).  Bits: alpha
// and bias, GELU, beta; no bit set = the accumulator as it is.
enum : int { EM_PLAIN = 0, EM_AFFINE = 1, EM_GELU = 2, EM_BETA = 4 };

template <int DT, int OT, int EM, int MS, int WTM, int WTN, int TM, int TN, int PW>
__device__ __attribute__((always_inline)) inline void epilogue_tile_t_ot(
    const MfmaArgs& p, typename AccBlock<MS>::T (&acc)[TM][TN], DGE_LDS char* stg, int m0, int n0,
    int wm0, int wn0, int lane) {
    typedef typename OutType<OT>::T T;
    constexpr int NG = TLayout<MS>::NG, CG = TLayout<MS>::CG;
    const int rl = lane % MS, cl = 4 * (lane / MS);
    // the lane's bias values: held in registers when few (16 for the 8-wave
    // tile), else loaded per group of 4 columns (the 4-wave tiles keep 256
    // accumulators live)
    constexpr bool PRE_BIAS = EM != EM_PLAIN && TN * NG * 4 <= 16;
    const bool has_bias = EM != EM_PLAIN && p.ep.epi != EPI_NONE;
    constexpr bool beta = (EM & EM_BETA) != 0;
    float bias[PRE_BIAS ? TN : 1][PRE_BIAS ? NG : 1][4];
    if constexpr (PRE_BIAS) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bias[j][g][e] =
                        has_bias ? load_elem<DT>(p.ep.bias, n0 + wn0 + MS * j + CG * g + cl + e) : 0.0f;
    }
    auto finish4 = [&](int i, int j, int g, float* t) __attribute__((always_inline)) {
        if constexpr (EM == EM_PLAIN) {
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = acc[i][j][4 * g + e];
            return;
        }
        const int64_t row = m0 + wm0 + MS * i + rl, col = n0 + wn0 + MS * j + CG * g + cl;
        float old[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (beta) {
            const T* c = (const T*)p.C + row * p.ldc + col;
#pragma unroll
            for (int e = 0; e < 4; ++e) old[e] = OutType<OT>::to_f32(c[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = p.ep.alpha * acc[i][j][4 * g + e];
            if constexpr (beta) v += p.ep.beta * old[e];
            if constexpr (PRE_BIAS)
                v += bias[j][g][e];
            else if (has_bias)
                v += load_elem<DT>(p.ep.bias, col + e);
            t[e] = (EM & EM_GELU) ? gelu_tanh(v) : v;
        }
    };
    // the wave's staging (PW bytes) holds IP row blocks of its tile at a time
    constexpr int EB = OutType<OT>::BYTES;
    constexpr int RB = WTN * EB;   // bytes of a staged row
    constexpr int CPR = RB / 16;   // 16-byte chunks per row (a power of two)
    constexpr int IP0 = PW / (MS * RB);
    constexpr int IP = IP0 >= TM ? TM : (IP0 >= 4 ? 4 : (IP0 >= 2 ? 2 : 1));
    static_assert(IP0 >= 1, "a row block of the wave tile fits the staging");
    static_assert((CPR & (CPR - 1)) == 0 && CPR >= 4 && TM % IP == 0, "staging layout");
#pragma unroll
    for (int i0 = 0; i0 < TM; i0 += IP) {
#pragma unroll
        for (int i = i0; i < i0 + IP; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    float t[4];
                    finish4(i, j, g, t);
                    const int r = MS * (i - i0) + rl;
                    const int cb = (MS * j + CG * g + cl) * EB;  // byte column in the row
                    DGE_LDS char* d = stg + r * RB + (((cb >> 4) ^ (r & (CPR - 1))) << 4) + (cb & 15);
                    if constexpr (EB == 4)
                        *(DGE_LDS f32x4*)d = (f32x4){t[0], t[1], t[2], t[3]};
                    else
                        *(DGE_LDS u32x2*)d = (u32x2){OutType<OT>::pack2(t[0], t[1]),
                                                     OutType<OT>::pack2(t[2], t[3])};
                }
        DGE_DIAG_SYNC();
        // this wave's rows back as 16-byte pieces (the wave's own LDS
        // operations complete in order: no barrier); each store addresses
        // a wave-uniform row base plus a 32-bit lane offset (leading
        // dimensions are below 2^24, so 16 rows stay below 2^31)
        const uint32_t loff = (uint32_t)(((lane / CPR) * p.ldc + n0 + wn0) * EB + 16 * (lane % CPR));
#pragma unroll
        for (int q = 0; q < IP * MS * CPR / 64; ++q) {
            const int r = q * (64 / CPR) + lane / CPR, ch = lane % CPR;
            const u32x4 v = *(const DGE_LDS u32x4*)(stg + r * RB + ((ch ^ (r & (CPR - 1))) << 4));
            const char* rb = (const char*)p.C + (int64_t)(m0 + wm0 + MS * i0 + q * (64 / CPR)) * p.ldc * EB;
            __builtin_nontemporal_store(v, (u32x4*)(rb + loff));
        }
    }
}

template <int DT, int EM, int MS, int WTM, int WTN, int TM, int TN, int PW>
__device__ __attribute__((always_inline)) inline void epilogue_tile_t_em(
    const MfmaArgs& p, typename AccBlock<MS>::T (&acc)[TM][TN], DGE_LDS char* stg, int m0, int n0,
    int wm0, int wn0, int lane) {
    if (p.c_type == OUT_F16)
        epilogue_tile_t_ot<DT, OUT_F16, EM, MS, WTM, WTN, TM, TN, PW>(p, acc, stg, m0, n0, wm0, wn0, lane);
    else if (p.c_type == OUT_BF16)
        epilogue_tile_t_ot<DT, OUT_BF16, EM, MS, WTM, WTN, TM, TN, PW>(p, acc, stg, m0, n0, wm0, wn0, lane);
    else
        epilogue_tile_t_ot<DT, OUT_F32, EM, MS, WTM, WTN, TM, TN, PW>(p, acc, stg, m0, n0, wm0, wn0, lane);
}

// STG: LDS bytes the staging may use (it starts at stg_all); each wave gets
// STG / waves, and as many row blocks per pass as fit.
template <int DT, int BM, int BN, int WM, int WN, int MS, int TM, int TN, int STG>
__device__ __attribute__((always_inline)) inline void epilogue_tile_t(
    const MfmaArgs& p, typename AccBlock<MS>::T (&acc)[TM][TN], DGE_LDS char* stg_all, int m0,
    int n0, int split) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    static_assert(TM * MS == WTM && TN * MS == WTN, "wave tile");
    constexpr int NG = TLayout<MS>::NG, CG = TLayout<MS>::CG;
    constexpr int PER_WAVE = STG / (WM * WN);
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
    if (p.ws) {  // split-K partial sums: fp32, no epilogue
        const int rl = lane % MS, cl = 4 * (lane / MS);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const int64_t row = m0 + wm0 + MS * i + rl;
                    float* w = p.ws + ((int64_t)split * p.M + row) * p.N + n0 + wn0 + MS * j + CG * g + cl;
                    *(f32x4*)w = (f32x4){acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                         acc[i][j][4 * g + 3]};
                }
        return;
    }
    DGE_LDS char* stg = stg_all + wave * PER_WAVE;
    constexpr int AB = EM_AFFINE | EM_BETA;
    const bool gelu = p.ep.epi == EPI_BIAS_GELU;
    if (p.ep.beta != 0.0f) {
        if (gelu)
            epilogue_tile_t_em<DT, AB | EM_GELU, MS, WTM, WTN, TM, TN, PER_WAVE>(p, acc, stg, m0, n0, wm0, wn0, lane);
        else
            epilogue_tile_t_em<DT, AB, MS, WTM, WTN, TM, TN, PER_WAVE>(p, acc, stg, m0, n0, wm0, wn0, lane);
    } else if (gelu) {
        epilogue_tile_t_em<DT, EM_AFFINE | EM_GELU, MS, WTM, WTN, TM, TN, PER_WAVE>(p, acc, stg, m0, n0, wm0, wn0, lane);
    } else if (p.ep.epi != EPI_NONE || p.ep.alpha != 1.0f) {
        epilogue_tile_t_em<DT, EM_AFFINE, MS, WTM, WTN, TM, TN, PER_WAVE>(p, acc, stg, m0, n0, wm0, wn0, lane);
    } else {
        epilogue_tile_t_em<DT, EM_PLAIN, MS, WTM, WTN, TM, TN, PER_WAVE>(p, acc, stg, m0, n0, wm0, wn0, lane);
    }
}

template <int DT, int BM, int BN, int WM, int WN, bool TRANS_B, int MS, bool Q4 = false,
          bool SK = false>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_direct_kernel(MfmaArgs p) {
    static_assert(DT == IN_F16 || DT == IN_BF16, "16-bit inputs only");
    static_assert(MS == 16 || MS == 32, "MFMA block size");
    static_assert(!Q4 || (TRANS_B && DT == IN_F16), "q4 weights are N x K, with fp16 A");
    static_assert(!(SK && Q4), "the stream-K schedule runs the 16-bit B path");
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
    constexpr int IB = Q4 ? 0 : B_BYTES / 1024 / NW;
    static_assert(IA * 1024 * NW == A_BYTES && (Q4 || IB * 1024 * NW == B_BYTES), "stage split");
    static_assert(TRANS_B || BN >= 128, "transposed-read layout needs 16+ chunks per k-row");
    constexpr int CPR_B = BN / 8;             // 16-byte chunks per k-row of a K x N B tile
    constexpr int RPI_B = 1024 / (BN * 2);    // k-rows per 1 KB direct-load instruction
    static_assert(TRANS_B || RPI_B * BN * 2 == 1024, "whole k-rows per instruction");

    // LDS stages: a third one where it fits (the 8-wave 256 x 128 tile, 144 KB)
    // so each stage's loads have two stages to land.  With q4 weights each
    // buffer also holds the stage's raw blocks: a weight row's 64-weight
    // slice of a stage is two 18-byte blocks, 36 bytes at a 4-byte aligned
    // address, brought in by dword direct loads with consecutive lanes on
    // consecutive dwords (a load covers about 7 rows' slices, so it touches
    // few cache lines) into a row-major image of 36 bytes per row;
    // 3 x (32 + 16 + 4.75) KB fits the 160 KB.
    constexpr int NRAW = BN * 9 / 64;                         // raw dword loads per stage
    constexpr int RAW_BYTES = (NRAW * 256 + 255) / 256 * 256;
    constexpr bool Q4_3 = Q4 && !SK && MS == 16 && NW == 8 && BN % 64 == 0 &&
                          3 * (A_BYTES + B_BYTES + RAW_BYTES) <= 160 * 1024;
    constexpr int NBUF = ((!Q4 && !SK && MS == 16 && NW == 8 &&
                           3 * (A_BYTES + B_BYTES) <= 160 * 1024) || Q4_3) ? 3 : 2;
    constexpr int BUF_BYTES = A_BYTES + B_BYTES + (Q4_3 ? RAW_BYTES : 0);
    __shared__ __attribute__((aligned(1024))) char lds[NBUF][BUF_BYTES];
    __shared__ int sk_flag;  // stream-K: a counter value broadcast to the workgroup

    const int tid = threadIdx.x;
    // the wave index is uniform: in a scalar register, the per-wave LDS
    // bases of the direct loads need no per-stage readfirstlane
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

    // ---- per-lane global source offsets (elements) for the direct loads
    // A: instruction i of this wave fills rows 8 * (wave * IA + i) + lane / 8;
    // its chunk swizzle depends on the row block, so it is applied per instruction
    const int a_row = 8 * wave * IA + (lane >> 3);
    const int k_lane_chunk = lane & 7;
    // B (K x N): instruction i fills k-rows RPI * (wave * IB + i) + lane / CPR;
    // the chunk swizzle depends on the k-row, so it is applied per instruction
    const int b_lane_chunk = lane % CPR_B;
    const int b_krow0 = RPI_B * wave * IB + lane / CPR_B;
    // per-lane byte offsets of each direct load from the wave's base (row or
    // k-row within the wave's block, swizzled chunk); constant for the kernel
    // (the host keeps them below 2^31: leading dimensions under 2^24)
    uint32_t a_off[IA > 0 ? IA : 1], b_off[IB > 0 ? IB : 1];
#pragma unroll
    for (int i = 0; i < IA; ++i)
        a_off[i] = (uint32_t)((((lane >> 3) + 8 * i) * p.lda +
                               (k_lane_chunk ^ swz_k<MS>(a_row + 8 * i)) * 8) * 2);
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        if constexpr (TRANS_B)
            b_off[i] = (uint32_t)((((lane >> 3) + 8 * i) * p.ldb +
                                   (k_lane_chunk ^ swz_k<MS>(8 * wave * IB + (lane >> 3) + 8 * i)) * 8) * 2);
        else
            b_off[i] = (uint32_t)(((lane / CPR_B + RPI_B * i) * p.ldb +
                                   (b_lane_chunk ^ swz_b<MS>(b_krow0 + RPI_B * i)) * 8) * 2);
    }
    // the current tile: origin (m0, n0), first k kbeg, and the wave-uniform
    // bases of its direct loads (A: the wave's first row at kbeg; B: the
    // wave's first row (N x K) or k-row (K x N))
    int m0 = 0, n0 = 0, kbeg = 0;
    const char* a_base = nullptr;
    const char* b_base = nullptr;
    const char* q_base = nullptr;  // fused q4, three stages: the tile's blocks at kbeg
    auto start_tile = [&](int tm0, int tn0, int tk0) __attribute__((always_inline)) {
        m0 = tm0;
        n0 = tn0;
        kbeg = tk0;
        a_base = (const char*)p.A + ((int64_t)(m0 + 8 * wave * IA) * p.lda + kbeg) * 2;
        if constexpr (TRANS_B)
            b_base = (const char*)p.B + ((int64_t)(n0 + 8 * wave * IB) * p.ldb + kbeg) * 2;
        else
            b_base = (const char*)p.B + ((int64_t)(kbeg + RPI_B * wave * IB) * p.ldb + n0) * 2;
        if constexpr (Q4_3)
            q_base = (const char*)p.B + 18 * ((int64_t)n0 * (p.K / 32) + kbeg / 32);
    };
    const int64_t a_kstep = BK;                                        // A per stage
    const int64_t b_kstep = TRANS_B ? (int64_t)BK : (int64_t)BK * p.ldb;  // B per stage

    // Direct loads [lo, hi) of the IA + IB of stage kt, into buffer st.
    auto issue_part = [&](int st, int kt, int lo, int hi) __attribute__((always_inline)) {
        DGE_LDS char* la = (DGE_LDS char*)&lds[st][0] + wave * IA * 1024;
        DGE_LDS char* lb = (DGE_LDS char*)&lds[st][A_BYTES] + wave * IB * 1024;
        const char* ga = a_base + kt * a_kstep * 2;
        const char* gb = b_base + kt * b_kstep * 2;
#pragma unroll
        for (int i = 0; i < IA; ++i) {
            if (i < lo || i >= hi) continue;
            lds_dma16_s(ga, a_off[i], la + i * 1024);
        }
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            if (IA + i < lo || IA + i >= hi) continue;
            lds_dma16_s(gb, b_off[i], lb + i * 1024);
        }
        DGE_DIAG_SYNC();
    };

    // ---- q4 B producer: task t = (tile row t / 2, block t % 2 of the stage)
    constexpr int NTHR = NW * 64;
    constexpr int QT = Q4 ? (2 * BN + NTHR - 1) / NTHR : 1;  // tasks per thread per stage
    static_assert(!Q4 || (2 * BN) % NTHR == 0 || 2 * BN < NTHR, "q4 task split");
    uint32_t qraw[QT][5];
    const int64_t qnb = p.K / 32;  // blocks per weight row (even: K % 64 == 0)
    auto q4_load = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < QT; ++i) {
            const int t = tid + i * NTHR;
            if ((2 * BN) % NTHR != 0 && t >= 2 * BN) continue;  // folds away when tasks divide evenly
            const int row = t >> 1, j = t & 1;
            // block (n0 + row, kbeg / 32 + 2 kt + j) sits at 18 x its index; the
            // index of j = 0 is even, so that block starts 4-byte aligned and
            // j = 1 starts 2 bytes past the 16th byte: both read 20 aligned bytes
            const int64_t blk = (int64_t)(n0 + row) * qnb + kbeg / 32 + 2 * kt;
            const uint32_t* src = (const uint32_t*)((const uint8_t*)p.B + 18 * blk + 16 * j);
#pragma unroll
            for (int e = 0; e < 5; ++e) qraw[i][e] = src[e];
        }
    };
    auto q4_store = [&](int st) __attribute__((always_inline)) {
        DGE_LDS char* lb = (DGE_LDS char*)&lds[st][A_BYTES];
#pragma unroll
        for (int i = 0; i < QT; ++i) {
            const int t = tid + i * NTHR;
            if ((2 * BN) % NTHR != 0 && t >= 2 * BN) continue;  // folds away when tasks divide evenly
            const int row = t >> 1, j = t & 1;
            const uint32_t* w = qraw[i];
            const uint16_t dbits = (uint16_t)(j ? (w[0] >> 16) : (w[0] & 0xFFFFu));
            const _Float16 d = __builtin_bit_cast(_Float16, dbits);
            const h2v d2 = {d, d};
            uint32_t c[4];  // the 16 code bytes
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] = j ? w[e + 1] : (w[e] >> 16) | (w[e + 1] << 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {  // chunk q: elements 8q .. 8q + 7 of the block
                const int shift = q < 2 ? 0 : 4, base = (q & 1) * 2;
                uint32_t o[4];
                q4_decode4((c[base] >> shift) & 0x0F0F0F0Fu, d2, o);
                q4_decode4((c[base + 1] >> shift) & 0x0F0F0F0Fu, d2, o + 2);
                *(DGE_LDS u32x4*)(lb + row * 128 + (((4 * j + q) ^ swz_k<MS>(row)) << 4)) =
                    (u32x4){o[0], o[1], o[2], o[3]};
            }
        }
        DGE_DIAG_SYNC();
    };

    // ---- q4 with three stages: raw blocks by direct dword loads, decoded
    // from LDS by all threads
    // raw load i of this wave (i < NRW; instruction r = (wave NRW + i) mod
    // NRAW, the surplus repeating earlier ones with the same bytes into the
    // same place): lane L fetches dword D = 64 r + L of the stage's image,
    // dword D % 9 of row D / 9's slice
    constexpr int NRW = Q4_3 ? (NRAW + NW - 1) / NW : 1;
    uint32_t raw_off[NRW], raw_lds[NRW];
    if constexpr (Q4_3) {
#pragma unroll
        for (int i = 0; i < NRW; ++i) {
            const int r = (wave * NRW + i) % NRAW, D = 64 * r + lane;
            raw_off[i] = (uint32_t)((D / 9) * 18 * (p.K / 32) + 4 * (D % 9));
            raw_lds[i] = (uint32_t)(A_BYTES + B_BYTES + 256 * r);
        }
    }
    // raw loads [lo, hi) of stage s into buffer buf's raw area
    auto issue_raw = [&](int buf, int s, int lo, int hi) __attribute__((always_inline)) {
        if constexpr (Q4_3) {
            const char* g = q_base + 36 * s;
#pragma unroll
            for (int i = 0; i < NRW; ++i) {
                if (i < lo || i >= hi) continue;
                lds_dma4_s(g, raw_off[i], (DGE_LDS char*)&lds[buf][0] + raw_lds[i]);
            }
            DGE_DIAG_SYNC();
        }
    };
    // the B tile of the stage whose raw blocks sit in buffer buf, decoded into
    // it: thread task t = (row t % BN, block j and half h from t / BN), eight
    // code bytes (16 weights) and the scale each.  A wave's lanes take
    // consecutive rows with the same (j, h): its raw-image reads fall in
    // distinct banks (a row is 9 dwords, 9 is odd), and each 16-lane group of
    // its decoded-chunk writes covers 16 rows of one logical chunk, the
    // pattern the fragment reads of the swizzled layout are conflict-free for.
    // In two steps: the raw dwords into registers (q4_raw_read, issued a
    // k-block ahead of their use, ahead of that k-block's fragment reads, so
    // that waiting for them never waits for the fragments), then the decode
    // and the LDS writes (q4_decode_write).
    constexpr int QP = Q4_3 ? (4 * BN + NTHR - 1) / NTHR : 1;  // tasks per thread
    uint32_t rawv[QP][4];
    auto q4_raw_read = [&](int buf) __attribute__((always_inline)) {
        if constexpr (Q4_3) {
            const DGE_LDS char* raw = (const DGE_LDS char*)&lds[buf][A_BYTES + B_BYTES];
#pragma unroll
            for (int pass = 0; pass < QP; ++pass) {
                const int t = tid + pass * NTHR;
                const int row = t % BN, j = (t / BN) >> 1, h = (t / BN) & 1;
                // dword c of the row's 36 bytes
                const DGE_LDS uint32_t* rr = (const DGE_LDS uint32_t*)(raw + 36 * row);
                const int c0 = (18 * j + 2 + 8 * h) >> 2;  // dword of the half's first code byte
                rawv[pass][0] = rr[4 * j];                 // scale: bytes 0-1 or 18-19
                rawv[pass][1] = rr[c0];
                rawv[pass][2] = rr[c0 + 1];
                rawv[pass][3] = rr[min(c0 + 2, 8)];
            }
        }
    };
    auto q4_decode_write = [&](int buf) __attribute__((always_inline)) {
        if constexpr (Q4_3) {
            DGE_LDS char* lb = (DGE_LDS char*)&lds[buf][A_BYTES];
#pragma unroll
            for (int pass = 0; pass < QP; ++pass) {
                const int t = tid + pass * NTHR;
                const int row = t % BN, j = (t / BN) >> 1, h = (t / BN) & 1;
                const uint32_t sh = (uint32_t)((18 * j + 2 + 8 * h) & 2) * 8;  // 16: mid-dword start
                const uint32_t* w = rawv[pass];
                const uint32_t c01 = __builtin_amdgcn_alignbit(w[2], w[1], sh);  // code bytes 0-3
                const uint32_t c23 = __builtin_amdgcn_alignbit(w[3], w[2], sh);  // code bytes 4-7
                const _Float16 d =
                    __builtin_bit_cast(_Float16, (uint16_t)(j ? w[0] >> 16 : w[0] & 0xFFFFu));
                const h2v d2 = {d, d};
                uint32_t o8[8];
                q4_decode4(c01 & 0x0F0F0F0Fu, d2, o8);             // weights 8h .. 8h + 3
                q4_decode4(c23 & 0x0F0F0F0Fu, d2, o8 + 2);         // 8h + 4 .. 8h + 7
                q4_decode4((c01 >> 4) & 0x0F0F0F0Fu, d2, o8 + 4);  // 16 + 8h ..
                q4_decode4((c23 >> 4) & 0x0F0F0F0Fu, d2, o8 + 6);
                DGE_LDS char* brow = lb + row * 128;
                *(DGE_LDS u32x4*)(brow + (((4 * j + h) ^ swz_k<MS>(row)) << 4)) =
                    (u32x4){o8[0], o8[1], o8[2], o8[3]};
                *(DGE_LDS u32x4*)(brow + (((4 * j + 2 + h) ^ swz_k<MS>(row)) << 4)) =
                    (u32x4){o8[4], o8[5], o8[6], o8[7]};
            }
            DGE_DIAG_SYNC();
        }
    };

    // ---- fragment reads of k-block kb
    // A (and K-contiguous B): row r = base + (lane % MS), chunk
    // (CPK kb + lane / MS) ^ swz_k(r) (the same swizzle for every block of rows).
    // (lo, hi: only reads lo .. hi - 1 of the ones listed, for spreading a
    // k-block's reads over several MFMAs)
    auto read_rows = [&](const DGE_LDS char* base, int row0, int kb, int ntile, u32x4* f,
                         int lo = 0, int hi = 1 << 20) __attribute__((always_inline)) {
        const int r = row0 + (lane % MS);
        const DGE_LDS char* q = base + r * 128 + (((kb * CPK + lane / MS) ^ swz_k<MS>(r)) << 4);
#pragma unroll
        for (int i = 0; i < ntile; ++i)
            if (i >= lo && i < hi) f[i] = *(const DGE_LDS u32x4*)(q + i * MS * 128);
    };
    // K x N B via transposed reads.  Lane group g = lane / 16 covers k-rows
    // kb KBLK + 8 (g / (MS / 16)) + 4 h + (t / 4) and columns
    // wn0 + MS j + 16 (g % (MS / 16)) + 4 (t % 4).
    auto read_bt = [&](const DGE_LDS char* base, int kb, u32x4* f, int lo = 0,
                       int hi = 1 << 20) __attribute__((always_inline)) {
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
                if (h * TN + j < lo || h * TN + j >= hi) continue;
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
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < NACC; ++r) acc[i][j][r] = 0.f;
    };

    u32x4 fa[2][TM], fb[2][TN];
    // reads lo .. hi - 1 of k-block kb's fragment reads (A's TM first, then B's)
    auto read_kblock = [&](int st, int kb, u32x4* a, u32x4* b, int lo = 0,
                           int hi = 1 << 20) __attribute__((always_inline)) {
        const DGE_LDS char* la = (const DGE_LDS char*)&lds[st][0];
        const DGE_LDS char* lb = (const DGE_LDS char*)&lds[st][A_BYTES];
        read_rows(la, wm0, kb, TM, a, lo, hi);
        if constexpr (TRANS_B)
            read_rows(lb, wn0, kb, TN, b, lo - TM, hi - TM);
        else
            read_bt(lb, kb, b, lo - TM, hi - TM);
        DGE_DIAG_SYNC();
    };
    // MFMAs [lo, hi) of one k-block over the TM x TN blocks in serpentine
    // order (row i left to right, row i + 1 right to left), so consecutive
    // MFMAs share an operand fragment also where the rows change: fewer input
    // bits toggle in the matrix unit, which is power-bound here (measured
    // ~1.6% faster with an N x K B, no change with K x N).
    auto mma_range = [&](const u32x4* a, const u32x4* b, int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < TM * TN; ++x)
            if (x >= lo && x < hi) {
                const int i = x / TN, j = (i & 1) ? TN - 1 - x % TN : x % TN;
                // operands swapped: the block is C^T (the epilogue's layout)
                if constexpr (MS == 32)
                    mma32<DT>(acc[i][j], b[j], a[i]);
                else
                    mma_chunk<DT>(acc[i][j], b[j], a[i]);
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
    // 1 (all after the barrier) for MS = 16 and for q4 (whose decode waits
    // for all outstanding loads and must not meet fresh ones)
    constexpr int DPART = Q4 ? 1 : (KB - 1 < 3 ? KB - 1 : 3);
    constexpr int NP0 = NDMA / DPART;                    // loads in the first part
    // MFMAs of a stage's last k-block left after the barrier (measured, same
    // machine, alternating processes): the 256 x 256 8-wave tile runs 4096^3 in
    // 105.7 us with 24 of its 32 after the barrier against 112.3 with 8 (NN;
    // NT 110.5 -> 104.5); the 256 x 128 8-wave tile with three LDS stages
    // runs best with all 16 after it (2048 x 4096 x 11008: 153.3 us with 4,
    // 147.2 with 12, 145.2 with 16); the fused q4 kernel keeps a quarter (its
    // decode runs between the MFMAs before the barrier)
    constexpr int TAIL = MS == 16 ? (Q4 && !Q4_3 ? NMF / 4 : NBUF == 3 ? NMF : NMF >= 32 ? NMF * 3 / 4 : NMF / 4)
                                  : (NMF / 2 > 0 ? NMF / 2 : 1);

    // Main loop over the nk stages of the current tile, stage kt in buffer
    // (kt + par) & 1; pre: stage 0's loads into buffer par are already in
    // flight.  Ends with every load landed and both buffers free.
    // Prologue: stages 0 and 1 in flight, wait for stage 0, read its k-block 0.
    auto mainloop = [&](int nk, int par, bool pre) __attribute__((always_inline)) {
    // (zeroed accumulators are pinned ahead of the first wait below: left
    // alone the compiler sinks the moves behind it, so they run after the
    // data has landed instead of while it is in flight; 8-wave tiles only,
    // whose accumulators sit in VGPRs)
    if (!pre) issue_part(par, 0, 0, NDMA);
    if constexpr (Q4 && !Q4_3) q4_load(0);
    issue_part(par ^ 1, nk > 1 ? 1 : 0, 0, NP0);
    if constexpr (Q4 && !Q4_3) q4_store(par);
    if constexpr (NW == 8 && MS == 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[i][j]));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((NP0 & 15) | ((NP0 >> 4) << 14)));  // vmcnt(NP0)
    __syncthreads();
    if constexpr (Q4 && !Q4_3) q4_load(nk > 1 ? 1 : 0);
    read_kblock(par, 0, fa[0], fb[0]);

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
        const int st = (kt + par) & 1;
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
        if constexpr (Q4 && !Q4_3) {
            // q4: stage kt + 1's B tile (buffer kt + 1 & 1, free since the last
            // barrier), from the blocks loaded a stage ago, decoded between
            // this k-block's MFMAs: each MFMA is followed by a share of the
            // decode's VALU work and, now and then, one of its LDS writes
            q4_store(st ^ 1);
            interleave_valu<NMF - TAIL, (QT * 72 + NMF - TAIL - 1) / (NMF - TAIL), QT * 4>();
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, NMF - TAIL, 0);
        }
        // nothing moves across the barrier (the MFMAs above would otherwise
        // drift past it, leaving the matrix unit idle while the wave waits)
        __builtin_amdgcn_sched_barrier(0);

        // vmcnt(0): this wave's loads of stage kt + 1 have landed; lgkmcnt(0):
        // its fragment reads of this stage are done before the barrier lets
        // other waves load into this buffer (whatever MFMAs precede it)
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();

        if constexpr (Q4 && !Q4_3) {
            issue_part(st, min(kt + 2, nk - 1), 0, NP0);
            q4_load(min(kt + 2, nk - 1));
            read_kblock(st ^ 1, 0, fa[0], fb[0]);
            mma_range(fa[L], fb[L], NMF - TAIL, NMF);
#pragma unroll
            for (int r = 0; r < TAIL; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x100, (NRD + TAIL - 1) / TAIL, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
        } else {
            // the direct loads and the next k-block's reads in TAIL steps, each
            // after one of the last MFMAs: the matrix unit restarts right
            // after the barrier instead of after a burst of loads (the loads
            // are ordered with the LDS reads in program order, so the steps
            // are written out one by one)
#pragma unroll
            for (int r = 0; r < TAIL; ++r) {
                issue_part(st, min(kt + 2, nk - 1), r * NP0 / TAIL, (r + 1) * NP0 / TAIL);
                read_kblock(st ^ 1, 0, fa[0], fb[0], r * NRD / TAIL, (r + 1) * NRD / TAIL);
            }
            mma_range(fa[L], fb[L], NMF - TAIL, NMF);
            tail_reads<TAIL, NRD>();
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    };

    // Main loop over three LDS stages (NBUF = 3): stage kt in buffer kt % 3.
    // The barrier that ends stage kt needs only stage kt + 1 landed (the
    // loads of stage kt + 2, issued a stage later, stay in flight:
    // vmcnt(NDMA)); after it the loads of stage kt + 3 go into buffer kt % 3,
    // one per remaining MFMA, with the reads of stage kt + 1's k-block 0.
    auto mainloop3 = [&](int nk) __attribute__((always_inline)) {
    issue_part(0, 0, 0, NDMA);
    issue_part(1, nk > 1 ? 1 : nk - 1, 0, NDMA);
    issue_part(2, nk > 2 ? 2 : nk - 1, 0, NDMA);
    if constexpr (NW == 8 && MS == 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(acc[i][j]));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70 | (((2 * NDMA) & 15) | (((2 * NDMA) >> 4) << 14)));  // vmcnt(2 NDMA)
    __syncthreads();
    read_kblock(0, 0, fa[0], fb[0]);
    int st = 0;  // buffer of stage kt
    for (int kt = 0; kt < nk; ++kt) {
        const int sn = st == NBUF - 1 ? 0 : st + 1;  // buffer of stage kt + 1
#pragma unroll
        for (int kb = 0; kb < KB - 1; ++kb) {
            read_kblock(st, kb + 1, fa[(kb + 1) & 1], fb[(kb + 1) & 1]);
            mma_range(fa[kb & 1], fb[kb & 1], 0, NMF);
            interleave_reads<NRD, NMF>();
        }
        constexpr int L = (KB - 1) & 1;
        mma_range(fa[L], fb[L], 0, NMF - TAIL);
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - TAIL, 0);
        __builtin_amdgcn_sched_barrier(0);
        // vmcnt(NDMA): stage kt + 1 has landed (stage kt + 2 may not have);
        // lgkmcnt(0): this wave's reads of buffer st are done
        __builtin_amdgcn_s_waitcnt(0x0070 | ((NDMA & 15) | ((NDMA >> 4) << 14)));
        __syncthreads();
#pragma unroll
        for (int r = 0; r < TAIL; ++r) {
            issue_part(st, min(kt + 3, nk - 1), r * NDMA / TAIL, (r + 1) * NDMA / TAIL);
            read_kblock(sn, 0, fa[0], fb[0], r * NRD / TAIL, (r + 1) * NRD / TAIL);
        }
        mma_range(fa[L], fb[L], NMF - TAIL, NMF);
        tail_reads<TAIL, NRD>();
        st = sn;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    };

    // Main loop of the fused q4 kernel over three LDS stages.  Stage s lives
    // in buffer s % 3: its A tile comes by direct loads issued after the
    // barrier that ends stage s - 3 (as in mainloop3), its raw q4 blocks one
    // stage earlier, after the barrier that ends stage s - 4, into the raw
    // area of the same buffer (free by then: the blocks of stage s - 3 were
    // decoded during stage s - 4), and its B tile is decoded from them by all
    // threads during stage s - 1, between the MFMAs of its first k-block.  The
    // barrier ending stage s waits for all but the newest group of loads:
    // that lands A of stage s + 1 and the raw blocks of stage s + 2, which
    // the next stage decodes.  Stages past the last re-fetch the last one
    // (never read), so every stage issues the same loads.
    constexpr int NG = NDMA + NRW;  // loads per wave issued after each barrier
    auto mainloop3_q4 = [&](int nk) __attribute__((always_inline)) {
    if constexpr (Q4_3) {
    const int l1 = min(1, nk - 1), l2 = min(2, nk - 1), l3 = min(3, nk - 1);
    issue_raw(0, 0, 0, NRW);                                 // raw 0
    issue_part(0, 0, 0, NDMA);                               // A 0, raw 1
    issue_raw(1, l1, 0, NRW);
    issue_part(1, l1, 0, NDMA);                              // A 1, raw 2
    issue_raw(2, l2, 0, NRW);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (((2 * NG) & 15) | (((2 * NG) >> 4) << 14)));  // raw 0 in
    __syncthreads();
    q4_raw_read(0);
    q4_decode_write(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): raw area 0 read, B 0 written
    __syncthreads();
    issue_part(2, l2, 0, NDMA);                              // A 2, raw 3 (raw area 0 is free)
    issue_raw(0, l3, 0, NRW);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (((2 * NG) & 15) | (((2 * NG) >> 4) << 14)));  // A 0, raw 1 in
    __syncthreads();
    q4_raw_read(1);
    read_kblock(0, 0, fa[0], fb[0]);
    int st = 0;  // buffer of stage kt
    for (int kt = 0; kt < nk; ++kt) {
        const int sn = st == 2 ? 0 : st + 1;  // buffer of stage kt + 1
        static_assert(KB == 2, "two k-blocks per stage");
        // k-block 0: its MFMAs, the fragment reads of k-block 1 and the
        // decode of stage kt + 1's B tile
        read_kblock(st, 1, fa[1], fb[1]);
        q4_decode_write(sn);
        mma_range(fa[0], fb[0], 0, NMF);
        interleave_q4<NMF, NRD, 36, 2>();
        __builtin_amdgcn_sched_barrier(0);
        // stage kt + 1 complete: its A and (decoded) B; raw blocks of stage
        // kt + 2 landed (vmcnt(NG): only the newest group may be in flight)
        __builtin_amdgcn_s_waitcnt(0x0070 | ((NG & 15) | ((NG >> 4) << 14)));
        __syncthreads();
        // A of stage kt + 3 into buffer st, raw of stage kt + 4 into buffer
        // sn's raw area, one load per MFMA of k-block 1, with the reads of
        // stage kt + 1's k-block 0
        const int la = min(kt + 3, nk - 1), lr = min(kt + 4, nk - 1);
        // the raw blocks stage kt + 1 decodes (buffer kt + 2), landed by this
        // barrier, read ahead of the fragments
        q4_raw_read(sn == 2 ? 0 : sn + 1);
#pragma unroll
        for (int r = 0; r < TAIL; ++r) {
            const int lo = r * NG / TAIL, hi = (r + 1) * NG / TAIL;
            issue_part(st, la, lo, min(hi, NDMA));
            issue_raw(sn, lr, max(lo - NDMA, 0), max(hi - NDMA, 0));
            read_kblock(sn, 0, fa[0], fb[0], r * NRD / TAIL, (r + 1) * NRD / TAIL);
        }
        mma_range(fa[1], fb[1], 0, NMF);
        tail_reads<TAIL, NRD>();
        st = sn;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    }
    };

    // the fused epilogue of tile (em0, en0), staged through buffer 0
    auto epilogue = [&](int em0, int en0, int split) __attribute__((always_inline)) {
        epilogue_tile_t<DT, BM, BN, WM, WN, MS, TM, TN, A_BYTES + B_BYTES>(
            p, acc, (DGE_LDS char*)&lds[0][0], em0, en0, split);
    };

    if constexpr (!SK) {
        // one (tile, K slice) per workgroup
        unsigned long long clk0 = 0, rt0 = 0;
        if (p.clk) {
            clk0 = __builtin_amdgcn_s_memtime();
            rt0 = __builtin_amdgcn_s_memrealtime();
        }
        const int ntiles = p.tiles_m * p.tiles_n;
        const int lin = remap_xcd(blockIdx.x, ntiles * p.splits);
        const int split = lin / ntiles;
        int tm, tn;
        grouped_tile(lin % ntiles, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        const int k0 = split * p.k_per_split;
        start_tile(tm * BM, tn * BN, k0);
        zero_acc();
        if constexpr (Q4_3)
            mainloop3_q4((min(k0 + p.k_per_split, p.K) - k0) / BK);
        else if constexpr (NBUF == 3)
            mainloop3((min(k0 + p.k_per_split, p.K) - k0) / BK);
        else
            mainloop((min(k0 + p.k_per_split, p.K) - k0) / BK, 0, false);
        epilogue(m0, n0, split);
        if (p.clk) {
            const unsigned long long clk1 = __builtin_amdgcn_s_memtime();
            const unsigned long long rt1 = __builtin_amdgcn_s_memrealtime();
            if (tid == 0) {
                unsigned long long* c = p.clk + 4 * (int64_t)blockIdx.x;
                c[0] = clk0;
                c[1] = rt0;
                c[2] = clk1;
                c[3] = rt1;
            }
        }
    } else {
        // Persistent schedule over the grid's G workgroups: first R rounds of
        // whole tiles, round r giving tile r G + v to workgroup v (so the
        // tiles running at once are consecutive in the grouped order and sit
        // at the same K stage, as in a data-parallel launch); then stream-K
        // over the T - R G tail tiles: their I = (T - R G) x S (tile, stage)
        // iterations split into equal contiguous ranges, consecutive ranges
        // on one XCD.  A range covers at most a partial tile at each end and
        // whole tiles between.  A whole tile ends with the fused epilogue.  A partial segment stores
        // its fp32 accumulators in a slot of the workspace and counts itself
        // in the tile's counter; the segment that completes the count sums all
        // segments of the tile in k order (bitwise the same sum whichever
        // segment finishes) and runs the epilogue.  No workgroup ever waits
        // for another.  Between segments, the next tile's first stage is
        // loaded into buffer 1 while the epilogue stages through buffer 0.
        const int G = gridDim.x;
        const int v = remap_xcd(blockIdx.x, G);
        const int S = p.sk_stages;
        const int R = p.sk_rounds, TB = R * G;  // whole-tile rounds; first tail tile
        const int64_t I = (int64_t)(p.tiles_m * p.tiles_n - TB) * S;
        auto it_of = [&](int w) __attribute__((always_inline)) { return (int64_t)w * I / G; };
        constexpr int CH = TM * TN * NACC / 4;  // 16-byte accumulator chunks per lane
        // slot of workgroup w's partial of the tile starting at iteration x:
        // 0 if it is the first segment of w's range, 1 if the last
        auto slot = [&](int w, int64_t x) __attribute__((always_inline)) {
            return p.sk_ws + (int64_t)(2 * w + (it_of(w) >= x ? 0 : 1)) * (BM * BN);
        };
        // chunk c of the lane's accumulators: elements 4 (c % Q) .. + 3 of
        // block c / Q, Q = NACC / 4 (indices are compile-time after unrolling)
        constexpr int Q = NACC / 4;
        auto get_chunk = [&](const Acc (&a)[TM][TN], int c) {
            const Acc& b = a[(c / Q) / TN][(c / Q) % TN];
            const int e = 4 * (c % Q);
            return (f32x4){b[e], b[e + 1], b[e + 2], b[e + 3]};
        };
        auto set_chunk = [&](Acc (&a)[TM][TN], int c, const f32x4& y) {
            Acc& b = a[(c / Q) / TN][(c / Q) % TN];
            const int e = 4 * (c % Q);
#pragma unroll
            for (int r = 0; r < 4; ++r) b[e + r] = y[r];
        };
        auto finish = [&](int tile, int ks, int ke, int em0, int en0) __attribute__((always_inline)) {
            if (ks == 0 && ke == S) {
                epilogue(em0, en0, 0);
                return;
            }
            const int64_t x = (int64_t)(tile - TB) * S;     // the tile's first tail iteration
            const int w0 = (int)(((x + 1) * G - 1) / I);  // owner of the tile's first stage
            const int nseg = (int)(((x + S) * G - 1) / I) - w0 + 1;
            const int j = v - w0;
            bool write = true;
            if (j == 0) {
                // the first segment usually finishes last (it closes its
                // workgroup's range): if every other one has counted itself,
                // finish without storing
                if (tid == 0)
                    sk_flag = (int)__hip_atomic_load(&p.sk_cnt[tile], __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
                write = sk_flag != nseg - 1;
                __syncthreads();
            }
            if (write) {
                // device-scope stores write through this XCD's L2; waiting
                // for them puts the partial at device scope before the count
                // (an agent-scope fence would write back and invalidate the
                // whole L2 instead, for every partial)
                // slot layout: element e of chunk c of thread t at (4 c + e) x
                // threads + t, so each store covers 256 contiguous bytes
                float* dst = slot(v, x) + tid;
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const f32x4 y = get_chunk(acc, c);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        __hip_atomic_store(dst + (4 * c + e) * NW * 64, y[e], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                __syncthreads();
                if (tid == 0) sk_flag = (int)atomicAdd(&p.sk_cnt[tile], 1u);
                __syncthreads();
                const bool last = sk_flag == nseg - 1;
                __syncthreads();
                if (!last) return;
            }
            // sum in k order, in place (device-scope loads: each slot was
            // written once in this launch, by one workgroup, through to
            // device scope before it was counted): a finisher that stored its partial
            // reads it back (each lane reads what it wrote) and starts from
            // segment 0's; one that did not is segment 0 and starts from its
            // own accumulators
            constexpr int GRP = CH < 8 ? CH : 8;  // chunks loaded at once (bounds the registers)
            for (int jj = write ? 0 : 1; jj < nseg; ++jj) {
                const float* src = slot(w0 + jj, x) + tid;
#pragma unroll
                for (int c0 = 0; c0 < CH; c0 += GRP) {
                    f32x4 y[GRP];
#pragma unroll
                    for (int c = 0; c < GRP; ++c)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            y[c][e] = __hip_atomic_load(src + (4 * (c0 + c) + e) * NW * 64,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                    for (int c = 0; c < GRP; ++c)
                        set_chunk(acc, c0 + c, jj == 0 ? y[c] : get_chunk(acc, c0 + c) + y[c]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            epilogue(em0, en0, 0);
        };

        // segments of this workgroup in order: the round tiles, then its
        // stream-K range of the tail
        int r = 0;
        int64_t it = I > 0 ? it_of(v) : 0;
        const int64_t it1 = I > 0 ? it_of(v + 1) : 0;
        auto next_segment = [&](int& tile, int& ks, int& ke) __attribute__((always_inline)) {
            if (r < R) {
                tile = r++ * G + v;
                ks = 0;
                ke = S;
                return true;
            }
            if (it >= it1) return false;
            const int lt = (int)(it / S);
            ks = (int)(it - (int64_t)lt * S);
            ke = (int)min((int64_t)S, ks + (it1 - it));
            tile = TB + lt;
            it += ke - ks;
            return true;
        };
        auto begin = [&](int tile, int ks) __attribute__((always_inline)) {
            int tm, tn;
            grouped_tile(tile, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
            start_tile(tm * BM, tn * BN, ks * BK);
        };
        int tile = 0, ks = 0, ke = 0;
        bool have = next_segment(tile, ks, ke);
        if (have) begin(tile, ks);
        int par = 0;
        bool pre = false;
        while (have) {
            zero_acc();
            mainloop(ke - ks, par, pre);
            const int em0 = m0, en0 = n0, ctile = tile, cks = ks, cke = ke;
            have = next_segment(tile, ks, ke);
            pre = false;
            if (have) {
                begin(tile, ks);
                // the next segment's first stage, into buffer 1
                issue_part(1, 0, 0, NDMA);
                pre = true;
            }
            finish(ctile, cks, cke, em0, en0);
            // the epilogue stages through buffer 0 without a closing barrier;
            // the next segment loads into it once every wave is done
            __syncthreads();
            par = pre ? 1 : 0;
        }
    }
}

}  // namespace dge

// Decode-shaped GEMM: C = epi(alpha X W^T + beta C) for a few input rows
// (M <= 64) against an N x K weight ("Matrix Multiplication: The Operation
// Behind Modern AI", "The shape a language model actually runs": at M = 1
// the best possible intensity is ~1 FLOP per byte, so the time is the time
// to read W once).  Everything is arranged around streaming W from HBM:
//
//  * A workgroup owns 16 weight rows and all M input rows; its 8 waves split
//    K into 8 slices of whole 32-deep k-blocks.  Within a wave, the MFMA "A"
//    operand is 8 consecutive k of one weight row per lane, i.e. a 16-byte
//    load straight from W into registers (no LDS), and the "B" operand is 8
//    consecutive k of one row of X (L2-resident: X is at most 64 x K; for
//    M > 1 loaded with whole 64-byte row pieces per lane quad and moved
//    into the operand layout through a small per-wave LDS slot).  The
//    product is C^T = W X^T in 16 x 16 blocks, MT = ceil(M / 16) of them.
//  * Loads for 16 k-blocks (8 for M > 32) are issued before their MFMAs, so
//    each lane keeps up to 256 bytes of W (and of X) in flight; with 8 waves
//    per CU that is ~128 KB of W per CU, and a 4096-deep K costs each wave a
//    single round trip to memory.
//  * The 8 partial blocks are summed through LDS in a fixed order (slice 0
//    first), so results do not depend on timing, and the fused epilogue
//    writes 16 consecutive columns per output row.
#pragma once

#include "device_common.h"
#include "mfma_gemm.h"

namespace dge {

struct DecodeArgs {
    const void* X;  // M x K, row-major
    const void* W;  // N x K, row-major
    void* C;        // M x N
    int64_t ldx, ldw, ldc;
    int M, N, K;
    int c_type;
    Epilogue ep;
    // split schedule (gemm_decode_split_kernel): K slices and the fp32
    // partial sums, ksplit x M x N (ld N)
    int ksplit;
    float* ws;
};

constexpr int DECODE_WAVES = 8;
constexpr int DPAD = 17;  // floats per 16-wide row of a partial block in LDS
// k-blocks whose loads are issued together: 16 (a 4096-deep K in one round
// trip per wave) while the registers allow, 8 for M > 32
__host__ __device__ constexpr int decode_batch(int mt) { return mt <= 2 ? 16 : 8; }

// XT: X goes through the per-wave transpose slot (below); off for M = 1,
// whose clamped rows make every quad read one address anyway.
template <int DT, int MT, bool XT = true>
__global__ __launch_bounds__(DECODE_WAVES * 64) void gemm_decode_kernel(DecodeArgs p) {
    // partial C^T blocks of every wave: [wave][mt][16 n][16 m] fp32, each n
    // row padded to DPAD floats so that the summation's reads (16 rows of one
    // column) fall in different banks
    __shared__ __attribute__((aligned(16))) float part[DECODE_WAVES][MT][16 * DPAD];
    // each wave's X transpose slot: MT blocks of 16 rows x 4 16-byte chunks
    __shared__ __attribute__((aligned(16))) u32x4 xslot[XT ? DECODE_WAVES : 1][MT][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int nkb = (p.K + 31) / 32;
    const int kb0 = wave * nkb / DECODE_WAVES, kb1 = (wave + 1) * nkb / DECODE_WAVES;

    // this lane's weight row: n0 + (lane & 15) (clamped to the last row:
    // valid memory, never stored); input rows are clamped to M - 1 the same way
    const int nr = min(n0 + (lane & 15), p.N - 1);
    const char* wrow = (const char*)p.W + ((int64_t)nr * p.ldw + 8 * (lane >> 4)) * 2;
    // X is loaded with the four lanes of a quad on one row's 64 contiguous
    // bytes (lane L: row 16 mt + L / 4, chunk L % 4): in the MFMA operand
    // layout (row L % 16) every quad would touch four rows, and the address
    // unit spends a cycle per row (M = 64: 24.4 -> 19.1 us for the loads
    // alone).  Each k-block's X then goes through the wave's LDS slot into
    // the operand layout; chunk c of row r sits at r * 4 + (c ^ ((r >> 2) & 3)),
    // so the sixteen rows of one chunk fall in different bank groups.
    const int xrl = XT ? lane >> 2 : lane & 15, xcl = XT ? lane & 3 : lane >> 4;  // row, chunk
    const char* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int mr = min(16 * mt + xrl, p.M - 1);
        xrow[mt] = (const char*)p.X + ((int64_t)mr * p.ldx + 8 * xcl) * 2;
    }
    const int xw = 4 * (lane >> 2) + ((lane & 3) ^ ((lane >> 4) & 3));  // where this lane's load goes
    const int xr = 4 * (lane & 15) + ((lane >> 4) ^ ((lane >> 2) & 3));  // where its operand comes from
    const int kchunk = 8 * (lane >> 4);  // this lane's k offset within a k-block

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    constexpr int DECODE_BATCH = decode_batch(MT);
    for (int kb = kb0; kb < kb1; kb += DECODE_BATCH) {
        u32x4 wf[DECODE_BATCH], xf[DECODE_BATCH][MT];
#pragma unroll
        for (int i = 0; i < DECODE_BATCH; ++i) {
            // K % 8 == 0: a chunk is all in or all out (W and X lanes hold
            // different chunks, each masked by its own k)
            const int k = (kb + i) * 32 + kchunk, kx = (kb + i) * 32 + 8 * xcl;
            const bool in = kb + i < kb1 && k < p.K, inx = kb + i < kb1 && kx < p.K;
            wf[i] = in ? load16(wrow + (int64_t)(kb + i) * 64) : (u32x4){0, 0, 0, 0};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xf[i][mt] = inx ? load16(xrow[mt] + (int64_t)(kb + i) * 64) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < DECODE_BATCH; ++i) {
            // the wave's own LDS operations complete in order: the reads see
            // these writes, and the next k-block's writes land after them
            u32x4 xo[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (XT)
                    xslot[wave][mt][xw] = xf[i][mt];
                else
                    xo[mt] = xf[i][mt];
            }
            if constexpr (XT) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) xo[mt] = xslot[wave][mt][xr];
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mma_chunk<DT>(acc[mt], wf[i], xo[mt]);
        }
    }

    // lane holds C^T rows n = 4 (lane / 16) + e, column m = lane % 16 of each block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][mt][(4 * (lane >> 4) + e) * DPAD + (lane & 15)] = acc[mt][e];
    __syncthreads();

    // output (m, n0 + j) for t = 16 m + j: 16 consecutive columns per row
    for (int t = tid; t < 16 * p.M; t += DECODE_WAVES * 64) {
        const int m = t >> 4, j = t & 15, n = n0 + j;
        if (n >= p.N) continue;
        const int mt = m >> 4, ml = m & 15;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < DECODE_WAVES; ++w) s += part[w][mt][j * DPAD + ml];  // m < 16 MT
        const int64_t idx = (int64_t)m * p.ldc + n;
        if (p.c_type == OUT_F32) {
            float* c = (float*)p.C + idx;
            *c = apply_epilogue<DT>(p.ep, s, p.ep.beta != 0.0f ? *c : 0.0f, n);
        } else if (p.c_type == OUT_F16) {
            _Float16* c = (_Float16*)p.C + idx;
            *c = (_Float16)apply_epilogue<DT>(p.ep, s, p.ep.beta != 0.0f ? (float)*c : 0.0f, n);
        } else {
            __bf16* c = (__bf16*)p.C + idx;
            *c = (__bf16)apply_epilogue<DT>(p.ep, s, p.ep.beta != 0.0f ? (float)*c : 0.0f, n);
        }
    }
}

// Split schedule for 33 <= M <= 64 rows (the kernel above re-reads all of X
// for every 16 weight rows: at M = 64 that is four times the weight's own
// bytes).  A workgroup owns DSPLIT_ROWS = 64 weight rows and one of ksplit
// K slices (grid (N / 64) x ksplit, 256 workgroups for N = 4096 with ksplit
// = 4); its 8 waves split the slice's k-blocks.  Each wave loads, per
// k-block, the four 16-row weight fragments and the MT X fragments straight
// into MFMA operand registers (16 bytes per lane) and applies every X
// fragment to all four weight blocks, so X crosses from L2 once per
// workgroup and slice: as many bytes as the weight.  The 8 waves' partial
// C^T blocks are summed through LDS in wave order and the workgroup writes
// its fp32 partial of the slice to ws[slice][m][n]; the split-K fixup sums
// the slices in slice order and applies the epilogue, so the result does
// not depend on timing.
constexpr int DSPLIT_ROWS = 64;
constexpr int DSPLIT_BATCH = 4;  // k-blocks whose loads are issued together

template <int DT, int MT>
__global__ __launch_bounds__(DECODE_WAVES * 64) void gemm_decode_split_kernel(DecodeArgs p) {
    constexpr int NB = DSPLIT_ROWS / 16;  // weight blocks per workgroup
    // partial C^T blocks [wave][nb][mt][16 n x 16 m]
    __shared__ __attribute__((aligned(16))) float part[DECODE_WAVES][NB][MT][16 * DPAD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ntile = p.N / DSPLIT_ROWS;
    const int nb_i = blockIdx.x % ntile, ks = blockIdx.x / ntile;
    const int n0 = nb_i * DSPLIT_ROWS;
    const int nkb = p.K / 32;
    const int s0 = ks * nkb / p.ksplit, s1 = (ks + 1) * nkb / p.ksplit;  // the slice's k-blocks
    const int kb0 = s0 + wave * (s1 - s0) / DECODE_WAVES;
    const int kb1 = s0 + (wave + 1) * (s1 - s0) / DECODE_WAVES;
    const int kch = 8 * (lane >> 4);  // this lane's k offset within a k-block
    const char* wrow[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        wrow[b] = (const char*)p.W + ((int64_t)(n0 + 16 * b + (lane & 15)) * p.ldw + kch) * 2;
    const char* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        xrow[mt] = (const char*)p.X + ((int64_t)min(16 * mt + (lane & 15), p.M - 1) * p.ldx + kch) * 2;

    f32x4 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[b][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    for (int kb = kb0; kb < kb1; kb += DSPLIT_BATCH) {
        u32x4 wf[DSPLIT_BATCH][NB], xf[DSPLIT_BATCH][MT];
#pragma unroll
        for (int i = 0; i < DSPLIT_BATCH; ++i) {
            const bool in = kb + i < kb1;
#pragma unroll
            for (int b = 0; b < NB; ++b)
                wf[i][b] = in ? load16(wrow[b] + (int64_t)(kb + i) * 64) : (u32x4){0, 0, 0, 0};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xf[i][mt] = in ? load16(xrow[mt] + (int64_t)(kb + i) * 64) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < DSPLIT_BATCH; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) mma_chunk<DT>(acc[b][mt], wf[i][b], xf[i][mt]);
    }
    // lane holds C^T rows n = 4 (lane / 16) + e, column m = lane % 16 of each block
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                part[wave][b][mt][(4 * (lane >> 4) + e) * DPAD + (lane & 15)] = acc[b][mt][e];
    __syncthreads();
    // the slice's partial (m, n0 + j), t = 64 m + j: 64 consecutive columns per row
    float* ws = p.ws + (int64_t)ks * p.M * p.N;
    for (int t = tid; t < DSPLIT_ROWS * p.M; t += DECODE_WAVES * 64) {
        const int m = t / DSPLIT_ROWS, j = t % DSPLIT_ROWS;
        const int b = j >> 4, nl = j & 15, mt = m >> 4, ml = m & 15;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < DECODE_WAVES; ++w) sum += part[w][b][mt][nl * DPAD + ml];
        ws[(int64_t)m * p.N + n0 + j] = sum;
    }
}

}  // namespace dge
